"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moe.h declares, validates arguments before touching
memory, and sizes buffers by the documented formulas."""
import ctypes
import os
import re

import numpy as np
import pytest

from routing_grouped_expert_router_amd import binding as B
from workloads import configs
from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    inc = os.path.join(ROOT, "include")
    txt = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 14
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(B.EXPORTED) == names


def test_status_strings():
    for code in range(5):
        assert B.lib().moe_status_string(code)


def _d(**kw):
    return B.Desc.from_config(configs.tiny()).__class__(**{**B.Desc.from_config(configs.tiny()).__dict__, **kw})


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), B.MOE_ERR_ARG), (dict(K=9), B.MOE_ERR_ARG), (dict(E_phys=0), B.MOE_ERR_ARG),
    (dict(n_shared=2), B.MOE_ERR_ARG), (dict(act_dtype=7), B.MOE_ERR_ARG),
    (dict(layout=5), B.MOE_ERR_ARG), (dict(M_max=0), B.MOE_ERR_ARG),
    (dict(H=100), B.MOE_ERR_UNSUPPORTED), (dict(I=200), B.MOE_ERR_UNSUPPORTED),
    (dict(E=2000, E_phys=2000), B.MOE_ERR_UNSUPPORTED), (dict(K=17, E=32, E_phys=32), B.MOE_ERR_UNSUPPORTED),
])
def test_desc_validation(kw, code):
    assert B.check_desc(_d(**kw)) == code


@pytest.mark.parametrize("flags,code", [
    (0, B.MOE_OK), (8, B.MOE_OK), (9, B.MOE_ERR_ARG),
    (B.MOE_DEBUG_TILED_WIDE_HYB << B.MOE_DEBUG_TILED_SHIFT, B.MOE_OK),
    (B.MOE_DEBUG_A8_STREAM << B.MOE_DEBUG_TILED_SHIFT, B.MOE_OK),
    (15 << B.MOE_DEBUG_TILED_SHIFT, B.MOE_ERR_ARG), (B.MOE_DEBUG_FUSED_NO_WAIT, B.MOE_OK),
    (0x200, B.MOE_ERR_ARG), (-1, B.MOE_ERR_ARG),
])
def test_debug_flags_validation(flags, code):
    """The test switches in moe_desc_t.debug_flags are checked like every
    other field: unknown bits and out-of-range values are argument errors."""
    assert B.check_desc(_d(debug_flags=flags)) == code


def test_calls_reject_bad_arguments_before_enqueueing():
    """Every failure below is decided on the host; null device pointers are
    never dereferenced and no stream is touched."""
    L = B.lib()
    d = _d()
    dc = ctypes.byref(d.c())
    rt = B.moe_route_t()                       # all-null tables
    null = None
    # T above T_max
    assert L.moe_route(dc, null, d.T_max + 1, null, null, ctypes.byref(rt), null, 0, null) == B.MOE_ERR_ARG
    assert L.moe_permute(dc, null, -1, ctypes.byref(rt), null, null) == B.MOE_ERR_ARG
    assert L.moe_router_logits(dc, null, null, null, 4, null, null) == B.MOE_ERR_ARG
    # null route tables
    assert L.moe_combine(dc, ctypes.byref(rt), 4, null, null, null) == B.MOE_ERR_ARG
    # workspace too small (table pointers non-null but never used)
    fake = ctypes.c_void_p(16)
    rt2 = B.moe_route_t(*([fake] * len(B.moe_route_t._fields_)))
    assert L.moe_route(dc, fake, 4, null, null, ctypes.byref(rt2), fake, 1, null) == B.MOE_ERR_WORKSPACE
    # fewer slots than experts: only for an expert-parallel share
    d7 = ctypes.byref(_d(E_phys=7).c())
    assert L.moe_route(d7, fake, 4, null, null, ctypes.byref(rt2), fake, 1 << 20, null) == B.MOE_ERR_ARG
    # only one of the two replica arrays
    assert L.moe_route(dc, fake, 4, fake, null, ctypes.byref(rt2), fake, 1 << 20, null) == B.MOE_ERR_ARG
    # grouped router parameters are checked on the host (E = 8 here)
    for bad in ((0, 1, 1), (3, 1, 1), (4, 5, 1), (4, 2, 3), (1, 1, 9)):
        g = B.moe_grouped_router_t(None, bad[0], bad[1], bad[2], 1, 1.0)
        assert L.moe_route_grouped(dc, fake, 4, ctypes.byref(g), null, null, ctypes.byref(rt2), fake,
                                   1 << 20, null) == B.MOE_ERR_ARG, bad
    g = B.moe_grouped_router_t(None, 8, 1, 1, 1, 1.0)     # one group of 1 kept, K = 2
    assert L.moe_route_grouped(dc, fake, 4, ctypes.byref(g), null, null, ctypes.byref(rt2), fake,
                               1 << 20, null) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_route_grouped(dc, fake, 4, null, null, null, ctypes.byref(rt2), fake, 1 << 20,
                               null) == B.MOE_ERR_ARG
    # expert-parallel routing: a map is required; without a replica map the
    # global slots must cover the E experts (E = 8 here); received counts
    # need the masked layout
    assert L.moe_route_ep(dc, fake, 4, null, null, null, null, ctypes.byref(rt2), fake, 1 << 20,
                          null) == B.MOE_ERR_ARG
    for bad in (B.moe_ep_map_t(None, 8), B.moe_ep_map_t(fake, 7), B.moe_ep_map_t(fake, 0),
                B.moe_ep_map_t(fake, 4097)):
        assert L.moe_route_ep(dc, fake, 4, null, ctypes.byref(bad), null, null, ctypes.byref(rt2), fake,
                              1 << 20, null) == B.MOE_ERR_ARG
    dcon = ctypes.byref(_d(layout=B.MOE_CONTIG, BM=16).c())
    assert L.moe_route_received(dcon, fake, 4, ctypes.byref(rt2), null) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_route_received(dc, null, 4, ctypes.byref(rt2), null) == B.MOE_ERR_ARG
    # W8A8 needs fp8 weights; the quantizer needs C a multiple of 128 and ld >= C
    assert L.moe_expert_gate_up_a8(dc, ctypes.byref(B.moe_weights_t(*([fake] * 12))), ctypes.byref(rt2), 4,
                                   fake, fake, fake, null) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_quantize_1x128(fake, 200, 4, 200, fake, fake, null) == B.MOE_ERR_ARG
    assert L.moe_quantize_1x128(fake, 64, 4, 128, fake, fake, null) == B.MOE_ERR_ARG
    assert L.moe_quantize_1x128(fake, 128, 0, 128, null, null, null) == B.MOE_OK
    # the fused gather needs bf16 activations (the tiny descriptor's are fp32)
    w0 = B.moe_weights_t(fake, fake, fake, None, None, None, None, None, None, None, None, None)
    assert L.moe_expert_gate_up_x(dc, ctypes.byref(w0), ctypes.byref(rt2), 4, fake, fake,
                                  null) == B.MOE_ERR_UNSUPPORTED
    # fp8 weights without scales
    d8 = _d(w_dtype=B.MOE_FP8E4M3_B128)
    w = B.moe_weights_t(fake, fake, fake, None, None, None, None, None, None, None, None, None)
    assert L.moe_grouped_ffn(ctypes.byref(d8.c()), ctypes.byref(w), ctypes.byref(rt2), 4, fake, fake,
                             fake, null) == B.MOE_ERR_ARG


def test_decode_fused_rejects_before_launch():
    """moe_decode_fused decides every refusal on the host: activations and
    weight layout it does not take, T above 16, null buffers, a too-small
    fused workspace, E too large for the single-workgroup route."""
    L = B.lib()
    fake = ctypes.c_void_p(16)
    rt2 = B.moe_route_t(*([fake] * len(B.moe_route_t._fields_)))
    w = B.moe_weights_t(*([fake] * 12))

    def call(d, T=4, fws_bytes=1 << 20, x=fake, g=None):
        return L.moe_decode_fused(ctypes.byref(d.c()), x, fake, None, g, None, None, ctypes.byref(w), T, fake,
                                  ctypes.byref(rt2), fake, 1 << 24, fake, fake, fake, fake, fws_bytes, None)

    bf = _d(act_dtype=B.MOE_BF16, w_packed=1, T_max=32)
    assert call(_d(w_packed=1)) == B.MOE_ERR_UNSUPPORTED                    # fp32 activations
    assert call(_d(act_dtype=B.MOE_BF16)) == B.MOE_ERR_UNSUPPORTED          # row-major weights
    assert call(bf, T=17) == B.MOE_ERR_UNSUPPORTED
    assert call(bf, T=33) == B.MOE_ERR_ARG                                   # above T_max
    assert call(bf, x=None) == B.MOE_ERR_ARG
    need = L.moe_decode_fused_workspace_bytes(ctypes.byref(bf.c()))
    assert need >= 768 + 4 * (1 + bf.E_phys)
    assert call(bf, fws_bytes=need - 1) == B.MOE_ERR_WORKSPACE
    big = _d(act_dtype=B.MOE_BF16, w_packed=1, E=1024, E_phys=1024, M_max=4)
    assert call(big) == B.MOE_ERR_UNSUPPORTED                                # softmax route above E = 512
    g = B.moe_grouped_router_t(None, 64, 8, 2, 1, 1.0)                       # E = 512 grouped
    assert call(_d(act_dtype=B.MOE_BF16, w_packed=1, E=512, E_phys=512, M_max=4),
                g=ctypes.byref(g)) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_decode_fused_workspace_bytes(ctypes.byref(_d(K=0).c())) == 0


@pytest.mark.parametrize("cfg", configs.all_configs(), ids=lambda c: c.name)
def test_buffer_sizing_formulas(cfg):
    d = B.Desc.from_config(cfg)
    if cfg.layout == "masked":
        cap = cfg.E_phys * cfg.M_max + cfg.K * max(0, cfg.T - cfg.M_max)
    else:
        cap = cfg.T * cfg.K + cfg.E_phys * (cfg.BM - 1)
    assert B.shared_base(d) == cap
    assert B.buffer_rows(d) == cap + cfg.n_shared * cfg.T
    s = B.down_splits(d, cfg.T)
    assert s >= 1 and (cfg.I // 128) % s == 0
    plane = B.buffer_rows(d) * cfg.H
    assert B.y_bytes(d, cfg.T) == (plane * 2 if s == 1 else plane * 4 * s)
    assert B.route_workspace_bytes(d) >= 4 * cfg.T * cfg.K
    assert B.workspace_bytes(d) == B.route_workspace_bytes(d)
    # the split router's arrival counts and partial 16 x 16 tiles (16 slices
    # of 64 lanes x 16 bytes) for up to 64 tokens, when it applies
    tiles = -(-cfg.E // 16) * -(-min(cfg.T, 64) // 16)
    split = (cfg.E > 64 and cfg.act_dtype == "bf16" and cfg.H % 1024 == 0 and cfg.H >= 4096
             and tiles * 2 <= 256)
    extra = (-(-4 * tiles // 256) * 256 + tiles * 16 * 64 * 16) if split else 0
    assert B.router_route_workspace_bytes(d) == B.route_workspace_bytes(d) + extra
    # one y buffer for every T: moe_y_bytes_max bounds moe_y_bytes at each T
    ymax = B.y_bytes_max(d)
    ts = sorted({1, 2, 3, cfg.T} | set(range(1, cfg.T + 1, max(1, cfg.T // 64))))
    assert ymax == max(B.y_bytes(d, t) for t in range(1, cfg.T + 1)) if cfg.T <= 512 else \
        ymax >= max(B.y_bytes(d, t) for t in ts)


def test_replica_map_helper_matches_reference_and_page():
    l2p, cnt = B.moe_replica_map_from_p2l([0, 1, 2, 3, 0, 1], 4, 2)
    assert l2p.tolist() == [[0, 4], [1, 5], [2, -1], [3, -1]] and cnt.tolist() == [2, 2, 1, 1]
    from workloads import generate
    cfg = configs.replica_decode()
    p2l = generate.make_p2l(cfg)
    ref_l2p, ref_cnt = O.replica_tables(p2l, cfg.E)
    l2p, cnt = B.moe_replica_map_from_p2l(p2l, cfg.E, ref_l2p.shape[1])
    assert (l2p.numpy() == ref_l2p).all() and (cnt.numpy() == ref_cnt).all()
    with pytest.raises(B.MoEError):
        B.moe_replica_map_from_p2l([0, 1, 5], 3, 2)      # logical id out of range
    with pytest.raises(B.MoEError):
        B.moe_replica_map_from_p2l([0, 0, 1], 3, 2)      # logical expert 2 has no slot
    with pytest.raises(B.MoEError):
        B.moe_replica_map_from_p2l([0, 0, 0, 1, 2], 3, 2)  # more than max_replicas


def test_ep_local_map_helper_matches_reference():
    for layout, name in ((B.MOE_EP_LINEAR, "linear"), (B.MOE_EP_ROUND_ROBIN, "round_robin")):
        for n, ep in ((4, 2), (5, 2), (7, 3), (256, 8), (544, 32), (3, 5)):
            for r in range(ep):
                got, nl = B.moe_ep_local_map(n, ep, r, layout)
                ref = O.ep_local_map(n, ep, r, name)
                assert got.tolist() == ref.tolist() and nl == int((ref >= 0).sum())
    for args in ((0, 2, 0, 0), (4, 0, 0, 0), (4, 2, 2, 0), (4, 2, -1, 0), (4, 2, 0, 7)):
        with pytest.raises(B.MoEError):
            B.moe_ep_local_map(*args)


def test_eplb_plan_helper_matches_reference():
    assert B.moe_eplb_plan([30.0, 5.0, 30.0, 5.0], 2, 2).tolist() == [0, 2, 1, 0, 2, 3]
    rng = np.random.default_rng(5)
    for _ in range(60):
        ep = int(rng.integers(1, 9)); S = int(rng.integers(1, 9))
        E = int(rng.integers(max(1, ep * S - 6), ep * S + 1))
        load = rng.integers(0, 20, size=E).astype(np.float64)      # ties on purpose
        got = B.moe_eplb_plan(load, ep * S - E, ep)
        assert got.tolist() == O.eplb_plan(load, ep * S - E, ep).tolist()
    E = 256
    load = (np.random.default_rng(2).permutation(E) + 1.0) ** -1.1
    for ep in (8, 32):
        assert B.moe_eplb_plan(load, 32, ep).tolist() == O.eplb_plan(load, 32, ep).tolist()
    for load, nr, ep in (([1.0, 2.0, 3.0], 0, 2), ([1.0, float("nan")], 0, 1), ([1.0, -1.0], 0, 1),
                         ([], 0, 1), ([1.0], -1, 1)):
        with pytest.raises(B.MoEError):
            B.moe_eplb_plan(load, nr, ep)


def test_expert_kernel_names_follow_the_size_classes():
    """The kernel a call runs for its largest groups: the streaming kernel
    for decode-sized groups, a large-group kernel for the prefill batch
    (packed weights, fused gather), the narrow tile when forced."""
    dec = B.Desc.from_config(configs.mixtral_decode(64), w_packed=1)
    assert B.expert_kernel(dec, 64, 0) == "ffn_stream_kernel"
    pre = B.Desc.from_config(configs.dsv3_prefill(), w_packed=1)
    assert B.expert_kernel(pre, 8192, 0) != "ffn_stream_kernel"
    assert B.expert_kernel(pre, 8192, 1) != "ffn_stream_kernel"
    pre.debug_flags = B.MOE_DEBUG_TILED_NARROW << B.MOE_DEBUG_TILED_SHIFT
    assert B.expert_kernel(pre, 8192, 0) == "ffn_tiled_kernel"
    assert B.expert_kernel(pre, 0, 0) == "none" and B.expert_kernel(pre, 8192, 2) == "none"


def test_a8_kernel_names_follow_the_size_classes():
    """The W8A8 calls: the large-group kernel for the fp8 prefill batch
    (groups large on average, packed weights), the streaming kernel for
    decode batches, row-major weights, K ranges that are not whole
    1024-element blocks, walk overrides that do not divide the tile count,
    and when forced by MOE_DEBUG_A8_STREAM; "none" for bf16 weights.  The
    bf16 calls ignore the W8A8 switch."""
    pre = B.Desc.from_config(configs.dsv3_prefill_fp8(), w_packed=1)
    assert [B.expert_kernel_a8(pre, 8192, w) for w in (0, 1)] == ["ffn_a8_tall_kernel"] * 2
    assert B.expert_kernel_a8(pre, 64, 0) == "ffn_a8_kernel"           # T*K < 64 E_phys
    dec = B.Desc.from_config(configs.dsv3_decode(256), w_packed=1)
    assert B.expert_kernel_a8(dec, 256, 0) == "ffn_a8_kernel"
    rowmajor = B.Desc.from_config(configs.dsv3_prefill_fp8(), w_packed=0)
    assert B.expert_kernel_a8(rowmajor, 8192, 0) == "ffn_a8_kernel"
    odd_k = B.Desc.from_config(configs.dsv3_prefill_fp8().with_(H=7168 - 512), w_packed=1)
    assert B.expert_kernel_a8(odd_k, 8192, 0) == "ffn_a8_kernel"      # gate/up K = H not whole 1024s
    assert B.expert_kernel_a8(odd_k, 8192, 1) == "ffn_a8_tall_kernel"
    pre.debug_flags = 3                                                # walk 3 divides neither tile count
    assert B.expert_kernel_a8(pre, 8192, 0) == "ffn_a8_kernel"
    pre.debug_flags = 4
    assert B.expert_kernel_a8(pre, 8192, 0) == "ffn_a8_tall_kernel"
    pre.debug_flags = B.MOE_DEBUG_A8_STREAM << B.MOE_DEBUG_TILED_SHIFT
    assert B.expert_kernel_a8(pre, 8192, 0) == "ffn_a8_kernel"
    bf = B.Desc.from_config(configs.dsv3_prefill(), w_packed=1)
    assert B.expert_kernel_a8(bf, 8192, 0) == "none"
    tall = B.expert_kernel(bf, 8192, 0)
    bf.debug_flags = B.MOE_DEBUG_A8_STREAM << B.MOE_DEBUG_TILED_SHIFT
    assert B.expert_kernel(bf, 8192, 0) == tall


def test_probes_reject_bad_arguments():
    L = B.lib()
    fake = ctypes.c_void_p(256)
    assert L.moe_probe_read(fake, 100, fake, None) == B.MOE_ERR_ARG          # not a multiple of 16
    assert L.moe_probe_read(None, 1024, fake, None) == B.MOE_ERR_ARG
    assert L.moe_probe_read(fake, 0, fake, None) == B.MOE_ERR_ARG
    assert L.moe_probe_mfma_bf16(0, 8, fake, None) == B.MOE_ERR_ARG
    assert L.moe_probe_mfma_bf16(10, B.MOE_PROBE_SINK_WORDS + 1, fake, None) == B.MOE_ERR_ARG
    assert L.moe_probe_mfma_bf16(10, 8, None, None) == B.MOE_ERR_ARG


def test_route_noalloc_rejects_a_workspace_beyond_its_array():
    """moe_route_noalloc's static workspace holds MOE_NOALLOC_WORKSPACE_BYTES;
    a descriptor needing more is refused on the host, before any device
    call."""
    L = B.lib()
    fake = ctypes.c_void_p(16)
    rt2 = B.moe_route_t(*([fake] * len(B.moe_route_t._fields_)))
    big = _d(T_max=200000, E=256, E_phys=256, K=8, M_max=64)
    assert B.route_workspace_bytes(big) > B.MOE_NOALLOC_WORKSPACE_BYTES
    assert L.moe_route_noalloc(ctypes.byref(big.c()), fake, 4, None, None, ctypes.byref(rt2),
                               None) == B.MOE_ERR_WORKSPACE
    assert L.moe_route_noalloc(ctypes.byref(_d(K=0).c()), fake, 4, None, None, ctypes.byref(rt2),
                               None) == B.MOE_ERR_ARG


def test_router_route_rejects_bad_arguments():
    """moe_router_route checks the router's and the routing's arguments on the
    host, before any device call."""
    L = B.lib()
    fake = ctypes.c_void_p(16)
    rt2 = B.moe_route_t(*([fake] * len(B.moe_route_t._fields_)))
    d = _d(T_max=4)
    ws_ok = B.route_workspace_bytes(d)
    args = lambda T, x, ws_bytes: (ctypes.byref(d.c()), x, fake, None, T, fake, None, None, ctypes.byref(rt2),
                                   fake, ws_bytes, None)
    assert L.moe_router_route(*args(5, fake, ws_ok)) == B.MOE_ERR_ARG        # T > T_max
    assert L.moe_router_route(*args(-1, fake, ws_ok)) == B.MOE_ERR_ARG
    assert L.moe_router_route(*args(2, None, ws_ok)) == B.MOE_ERR_ARG        # no x
    assert L.moe_router_route(*args(2, fake, ws_ok - 1)) == B.MOE_ERR_WORKSPACE
