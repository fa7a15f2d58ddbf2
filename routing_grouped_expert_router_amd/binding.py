"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only:
every step of the layer runs in the library's HIP kernels; PyTorch supplies
device memory and the current stream.

The library must be built (``python -m routing_grouped_expert_router_amd.build``);
loading fails loudly when it is missing.  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8E4M3_B128 = 0, 1, 2
MOE_CONTIG, MOE_MASKED = 0, 1
MOE_STATUS_SPILL, MOE_STATUS_BAD_REPLICA, MOE_STATUS_NONFINITE, MOE_STATUS_INTERNAL = 1, 2, 4, 8
MOE_STATUS_BAD_EP_MAP, MOE_STATUS_RECV_OVERFLOW, MOE_STATUS_SYNC_TIMEOUT = 16, 32, 64
MOE_EP_LINEAR, MOE_EP_ROUND_ROBIN = 0, 1
MOE_DEBUG_NBLK_MASK, MOE_DEBUG_TILED_SHIFT, MOE_DEBUG_FUSED_NO_WAIT = 0xF, 4, 0x100
MOE_DEBUG_TILED_NARROW, MOE_DEBUG_TILED_WIDE_REGS, MOE_DEBUG_TILED_WIDE_LDS, MOE_DEBUG_TILED_WIDE_HYB = 1, 2, 3, 4
MOE_DEBUG_TILED_TALL = 5
MOE_DEBUG_A8_STREAM = 6

EXPORTED = [
    "moe_status_string", "moe_check_desc", "moe_route_workspace_bytes", "moe_buffer_rows",
    "moe_shared_base", "moe_down_splits", "moe_y_bytes", "moe_y_bytes_max", "moe_workspace_bytes",
    "moe_router_route_workspace_bytes",
    "moe_router_logits", "moe_route",
    "moe_route_grouped",
    "moe_permute", "moe_expert_gate_up", "moe_expert_gate_up_x", "moe_expert_down",
    "moe_grouped_ffn", "moe_grouped_ffn_x", "moe_combine", "moe_forward", "moe_pack_weights",
    "moe_replica_map_from_p2l", "moe_route_ep", "moe_route_received", "moe_ep_local_map",
    "moe_eplb_plan", "moe_quantize_1x128", "moe_expert_gate_up_a8", "moe_expert_down_a8",
    "moe_grouped_ffn_a8", "moe_decode_fused_workspace_bytes", "moe_decode_fused",
    "moe_expert_kernel", "moe_expert_kernel_a8", "moe_probe_read", "moe_probe_mfma_bf16", "moe_route_noalloc", "moe_router_route",
]
MOE_NOALLOC_WORKSPACE_BYTES = 4 << 20
MOE_PROBE_SINK_WORDS = 8192
MOE_CLAIM_WORDS = 256


class moe_desc_t(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T_max", "H", "I", "E", "E_phys", "K", "n_shared", "max_replicas",
        "act_dtype", "w_dtype", "layout", "M_max", "BM", "w_packed", "debug_flags")]


_P = ctypes.c_void_p


class moe_route_t(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "topk_ids", "topk_w", "topk_phys", "row_of", "slot_of", "src_of", "counts",
        "offsets", "masked_m", "spill_off", "pad_off", "tile_off", "status", "claim")]


class moe_ep_map_t(ctypes.Structure):
    _fields_ = [("local_of", _P), ("n_global", ctypes.c_int32)]


class moe_grouped_router_t(ctypes.Structure):
    _fields_ = [("score_bias", _P), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("group_k", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("scale", ctypes.c_float)]


class moe_weights_t(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "w1", "w3", "w2", "s1", "s3", "s2", "sw1", "sw3", "sw2", "ss1", "ss3", "ss2")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m routing_grouped_expert_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(moe_desc_t)
        R = ctypes.POINTER(moe_route_t)
        W = ctypes.POINTER(moe_weights_t)
        GR = ctypes.POINTER(moe_grouped_router_t)
        i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_check_desc": (ctypes.c_int, [D]),
            "moe_route_workspace_bytes": (sz, [D]),
            "moe_buffer_rows": (i64, [D]),
            "moe_shared_base": (i64, [D]),
            "moe_down_splits": (i32, [D, i32]),
            "moe_y_bytes": (sz, [D, i32]),
            "moe_y_bytes_max": (sz, [D]),
            "moe_workspace_bytes": (sz, [D]),
            "moe_router_route_workspace_bytes": (sz, [D]),
            "moe_router_logits": (ctypes.c_int, [D, _P, _P, _P, i32, _P, _P]),
            "moe_route": (ctypes.c_int, [D, _P, i32, _P, _P, R, _P, sz, _P]),
            "moe_route_grouped": (ctypes.c_int, [D, _P, i32, GR, _P, _P, R, _P, sz, _P]),
            "moe_route_noalloc": (ctypes.c_int, [D, _P, i32, _P, _P, R, _P]),
            "moe_router_route": (ctypes.c_int, [D, _P, _P, _P, i32, _P, _P, _P, R, _P, sz, _P]),
            "moe_permute": (ctypes.c_int, [D, _P, i32, R, _P, _P]),
            "moe_expert_gate_up": (ctypes.c_int, [D, W, R, i32, _P, _P, _P]),
            "moe_expert_gate_up_x": (ctypes.c_int, [D, W, R, i32, _P, _P, _P]),
            "moe_expert_down": (ctypes.c_int, [D, W, R, i32, _P, _P, _P]),
            "moe_grouped_ffn": (ctypes.c_int, [D, W, R, i32, _P, _P, _P, _P]),
            "moe_grouped_ffn_x": (ctypes.c_int, [D, W, R, i32, _P, _P, _P, _P]),
            "moe_combine": (ctypes.c_int, [D, R, i32, _P, _P, _P]),
            "moe_forward": (ctypes.c_int, [D, _P, _P, _P, _P, _P, W, i32, _P, R, _P, sz,
                                           _P, _P, _P, _P, _P]),
            "moe_pack_weights": (ctypes.c_int, [D, i32, i32, _P, _P, _P]),
            "moe_replica_map_from_p2l": (ctypes.c_int, [_P, i32, i32, i32, _P, _P]),
            "moe_route_ep": (ctypes.c_int, [D, _P, i32, _P, ctypes.POINTER(moe_ep_map_t), _P, _P, R,
                                            _P, sz, _P]),
            "moe_route_received": (ctypes.c_int, [D, _P, i32, R, _P]),
            "moe_ep_local_map": (ctypes.c_int, [i32, i32, i32, i32, _P, _P]),
            "moe_eplb_plan": (ctypes.c_int, [_P, i32, i32, i32, _P]),
            "moe_quantize_1x128": (ctypes.c_int, [_P, i64, i64, i32, _P, _P, _P]),
            "moe_expert_gate_up_a8": (ctypes.c_int, [D, W, R, i32, _P, _P, _P, _P]),
            "moe_expert_down_a8": (ctypes.c_int, [D, W, R, i32, _P, _P, _P, _P]),
            "moe_grouped_ffn_a8": (ctypes.c_int, [D, W, R, i32, _P, _P, _P, _P, _P, _P, _P, _P]),
            "moe_decode_fused_workspace_bytes": (sz, [D]),
            "moe_expert_kernel": (ctypes.c_char_p, [D, i32, i32]),
            "moe_expert_kernel_a8": (ctypes.c_char_p, [D, i32, i32]),
            "moe_probe_read": (ctypes.c_int, [_P, sz, _P, _P]),
            "moe_probe_mfma_bf16": (ctypes.c_int, [i32, i32, _P, _P]),
            "moe_decode_fused": (ctypes.c_int, [D, _P, _P, _P, GR, _P, _P, W, i32, _P, R, _P, sz, _P, _P,
                                                _P, _P, sz, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class MoEError(RuntimeError):
    pass


def _check(code: int, what: str):
    if code != MOE_OK:
        msg = lib().moe_status_string(code).decode()
        raise MoEError(f"{what}: {msg} (status {code})")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Desc:
    T_max: int
    H: int
    I: int
    E: int
    E_phys: int
    K: int
    n_shared: int = 0
    max_replicas: int = 1
    act_dtype: int = MOE_BF16
    w_dtype: int = MOE_BF16
    layout: int = MOE_CONTIG
    M_max: int = 1
    BM: int = 16
    w_packed: int = 0
    debug_flags: int = 0

    def c(self) -> moe_desc_t:
        return moe_desc_t(*[int(getattr(self, f)) for f, _ in moe_desc_t._fields_])

    @staticmethod
    def from_config(cfg, max_replicas: int = 1, w_packed: int = 0) -> "Desc":
        return Desc(T_max=cfg.T, H=cfg.H, I=cfg.I, E=cfg.E, E_phys=cfg.E_phys, K=cfg.K,
                    n_shared=cfg.n_shared, max_replicas=max_replicas,
                    act_dtype=MOE_F32 if cfg.act_dtype == "f32" else MOE_BF16,
                    w_dtype=MOE_BF16 if cfg.w_dtype == "bf16" else MOE_FP8E4M3_B128,
                    layout=MOE_MASKED if cfg.layout == "masked" else MOE_CONTIG,
                    M_max=max(1, cfg.M_max), BM=max(1, cfg.BM), w_packed=w_packed)


# ---- sizing -------------------------------------------------------------------

def check_desc(d: Desc) -> int:
    return lib().moe_check_desc(ctypes.byref(d.c()))


def route_workspace_bytes(d: Desc) -> int:
    return lib().moe_route_workspace_bytes(ctypes.byref(d.c()))


def buffer_rows(d: Desc) -> int:
    return lib().moe_buffer_rows(ctypes.byref(d.c()))


def shared_base(d: Desc) -> int:
    return lib().moe_shared_base(ctypes.byref(d.c()))


def down_splits(d: Desc, T: int) -> int:
    return lib().moe_down_splits(ctypes.byref(d.c()), T)


def y_bytes(d: Desc, T: int) -> int:
    return lib().moe_y_bytes(ctypes.byref(d.c()), T)


def y_bytes_max(d: Desc) -> int:
    return lib().moe_y_bytes_max(ctypes.byref(d.c()))


def workspace_bytes(d: Desc) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(d.c()))


def router_route_workspace_bytes(d: Desc) -> int:
    """moe_router_route_workspace_bytes: the route workspace plus the split
    router's zero-filled counts and partial tiles."""
    return lib().moe_router_route_workspace_bytes(ctypes.byref(d.c()))


def expert_kernel(d: Desc, T: int, which: int) -> str:
    """Name of the kernel the expert call runs for the largest groups
    (which = 0 gate/up, 1 down)."""
    return lib().moe_expert_kernel(ctypes.byref(d.c()), T, which).decode()


def expert_kernel_a8(d: Desc, T: int, which: int) -> str:
    """The same for the W8A8 expert calls."""
    return lib().moe_expert_kernel_a8(ctypes.byref(d.c()), T, which).decode()


# ---- measurement probes (include/moe_probe.h) ---------------------------------

def moe_probe_read(buf, sink, stream=None):
    """One non-temporal streaming read of the device tensor ``buf``."""
    _check(lib().moe_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "moe_probe_read")


def moe_probe_mfma_bf16(iters: int, workgroups: int, sink, stream=None):
    """``workgroups`` x 4 waves x ``iters`` x 8 bf16 16x16x32 matrix-core
    products (16384 FLOP each), no memory traffic."""
    _check(lib().moe_probe_mfma_bf16(iters, workgroups, _ptr(sink), _stream(stream)), "moe_probe_mfma_bf16")


# ---- buffers ------------------------------------------------------------------

class RouteTables:
    """Device tensors behind a moe_route_t (allocated with torch)."""

    def __init__(self, d: Desc, device="cuda"):
        TK = max(1, d.T_max * d.K)
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_ids = torch.zeros(TK, **i32)
        self.topk_w = torch.zeros(TK, dtype=torch.float32, device=device)
        self.topk_phys = torch.zeros(TK, **i32)
        self.row_of = torch.zeros(TK, **i32)
        self.slot_of = torch.zeros(TK, **i32)
        self.src_of = torch.zeros(TK, **i32)
        self.counts = torch.zeros(d.E_phys, **i32)
        self.offsets = torch.zeros(d.E_phys + 1, **i32)
        self.masked_m = torch.zeros(d.E_phys, **i32)
        self.spill_off = torch.zeros(d.E_phys + 1, **i32)
        self.pad_off = torch.zeros(d.E_phys + 1, **i32)
        self.tile_off = torch.zeros(d.E_phys + 2, **i32)
        self.status = torch.zeros(1, **i32)
        self.claim = torch.zeros(MOE_CLAIM_WORDS, **i32)
        self.c = moe_route_t(*[_ptr(getattr(self, f)) for f, _ in moe_route_t._fields_])


class Weights:
    """moe_weights_t over torch tensors (kept alive here)."""

    def __init__(self, w: dict, shared: dict | None = None):
        self._keep = (w, shared)
        s = shared or {}
        self.c = moe_weights_t(
            _ptr(w["w1"]), _ptr(w["w3"]), _ptr(w["w2"]),
            _ptr(w.get("s1")), _ptr(w.get("s3")), _ptr(w.get("s2")),
            _ptr(s.get("w1")), _ptr(s.get("w3")), _ptr(s.get("w2")),
            _ptr(s.get("s1")), _ptr(s.get("s3")), _ptr(s.get("s2")))


# ---- the five steps (same names as the C ABI) ------------------------------------

def moe_router_logits(d: Desc, x, w_router, bias, T, logits, stream=None):
    _check(lib().moe_router_logits(ctypes.byref(d.c()), _ptr(x), _ptr(w_router), _ptr(bias),
                                   T, _ptr(logits), _stream(stream)), "moe_router_logits")


def moe_route(d: Desc, logits, T, rt: RouteTables, ws, l2p=None, replica_count=None, stream=None):
    _check(lib().moe_route(ctypes.byref(d.c()), _ptr(logits), T, _ptr(l2p), _ptr(replica_count),
                           ctypes.byref(rt.c), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)), "moe_route")


def moe_router_route(d: Desc, x, w_router, bias, T, logits, rt: RouteTables, ws, l2p=None, replica_count=None,
                     stream=None):
    """moe_router_logits then moe_route in one call (one launch for tiny T * E)."""
    _check(lib().moe_router_route(ctypes.byref(d.c()), _ptr(x), _ptr(w_router), _ptr(bias), T, _ptr(logits),
                                  _ptr(l2p), _ptr(replica_count), ctypes.byref(rt.c), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "moe_router_route")


def moe_route_noalloc(d: Desc, logits, T, rt: RouteTables, l2p=None, replica_count=None, stream=None):
    """moe_route with the library's static per-GPU workspace (no workspace
    argument, nothing allocated)."""
    _check(lib().moe_route_noalloc(ctypes.byref(d.c()), _ptr(logits), T, _ptr(l2p), _ptr(replica_count),
                                   ctypes.byref(rt.c), _stream(stream)), "moe_route_noalloc")


class GroupedRouter:
    """Parameters of the grouped sigmoid router (moe_grouped_router_t);
    ``score_bias`` is a device fp32 tensor [E] or None."""

    def __init__(self, n_group, topk_group, group_k, renormalize=True, scale=1.0, score_bias=None):
        self.score_bias = score_bias
        self.c = moe_grouped_router_t(_ptr(score_bias), n_group, topk_group, group_k,
                                      int(bool(renormalize)), float(scale))


def moe_route_grouped(d: Desc, logits, T, rt: RouteTables, ws, router: GroupedRouter, l2p=None,
                      replica_count=None, stream=None):
    _check(lib().moe_route_grouped(ctypes.byref(d.c()), _ptr(logits), T, ctypes.byref(router.c),
                                   _ptr(l2p), _ptr(replica_count), ctypes.byref(rt.c), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "moe_route_grouped")


def moe_permute(d: Desc, x, T, rt: RouteTables, xg, stream=None):
    _check(lib().moe_permute(ctypes.byref(d.c()), _ptr(x), T, ctypes.byref(rt.c), _ptr(xg),
                             _stream(stream)), "moe_permute")


def moe_grouped_ffn(d: Desc, w: Weights, rt: RouteTables, T, xg, h, y, stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                 _ptr(xg), _ptr(h), _ptr(y), _stream(stream)), "moe_grouped_ffn")


def moe_grouped_ffn_x(d: Desc, w: Weights, rt: RouteTables, T, x, h, y, stream=None):
    _check(lib().moe_grouped_ffn_x(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                   _ptr(x), _ptr(h), _ptr(y), _stream(stream)), "moe_grouped_ffn_x")


def moe_expert_gate_up_x(d: Desc, w: Weights, rt: RouteTables, T, x, h, stream=None):
    _check(lib().moe_expert_gate_up_x(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                      _ptr(x), _ptr(h), _stream(stream)), "moe_expert_gate_up_x")


def moe_expert_gate_up(d: Desc, w: Weights, rt: RouteTables, T, xg, h, stream=None):
    _check(lib().moe_expert_gate_up(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                    _ptr(xg), _ptr(h), _stream(stream)), "moe_expert_gate_up")


def moe_expert_down(d: Desc, w: Weights, rt: RouteTables, T, h, y, stream=None):
    _check(lib().moe_expert_down(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                 _ptr(h), _ptr(y), _stream(stream)), "moe_expert_down")


def moe_combine(d: Desc, rt: RouteTables, T, y, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(d.c()), ctypes.byref(rt.c), T, _ptr(y), _ptr(out),
                             _stream(stream)), "moe_combine")


def moe_forward(d: Desc, x, w_router, bias, w: Weights, T, logits, rt: RouteTables, ws, xg, h, y, out,
                l2p=None, replica_count=None, stream=None):
    """The five steps in one C call (router logits, moe_route, permute or the
    fused gather, grouped FFN, combine)."""
    _check(lib().moe_forward(ctypes.byref(d.c()), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(l2p),
                             _ptr(replica_count), ctypes.byref(w.c), T, _ptr(logits), ctypes.byref(rt.c),
                             _ptr(ws), ws.numel() * ws.element_size(), _ptr(xg), _ptr(h), _ptr(y), _ptr(out),
                             _stream(stream)), "moe_forward")


def moe_pack_weights(d: Desc, which: int, src, dst, stream=None):
    """Packs G row-major expert matrices (src [G, N, Kdim]) into dst (same
    shape and dtype) in the layout the expert kernels stream."""
    G = src.shape[0] if src.dim() == 3 else 1
    _check(lib().moe_pack_weights(ctypes.byref(d.c()), which, G, _ptr(src), _ptr(dst),
                                  _stream(stream)), "moe_pack_weights")


def pack_expert_weights(d: Desc, weights: dict) -> dict:
    """A copy of a weight dict (w1, w3 [G, I, H], w2 [G, H, I], fp8 scales)
    with the matrices packed; scales are shared unchanged."""
    out = dict(weights)
    for name, which in (("w1", 0), ("w3", 0), ("w2", 1)):
        src = weights[name].contiguous()
        dst = torch.empty_like(src)
        moe_pack_weights(d, which, src, dst)
        out[name] = dst
    return out


class EPMap:
    """One rank's local map (moe_ep_map_t): ``local_of`` a device int32
    tensor over the n_global global physical slots."""

    def __init__(self, local_of, n_global=None):
        self.local_of = local_of
        self.c = moe_ep_map_t(_ptr(local_of), int(local_of.numel() if n_global is None else n_global))


def moe_route_ep(d: Desc, logits, T, rt: RouteTables, ws, ep: EPMap, router: "GroupedRouter | None" = None,
                 l2p=None, replica_count=None, stream=None):
    _check(lib().moe_route_ep(ctypes.byref(d.c()), _ptr(logits), T,
                              None if router is None else ctypes.byref(router.c), ctypes.byref(ep.c),
                              _ptr(l2p), _ptr(replica_count), ctypes.byref(rt.c), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "moe_route_ep")


def moe_route_received(d: Desc, counts, T, rt: RouteTables, stream=None):
    _check(lib().moe_route_received(ctypes.byref(d.c()), _ptr(counts), T, ctypes.byref(rt.c),
                                    _stream(stream)), "moe_route_received")


def moe_ep_local_map(n_global: int, ep_size: int, rank: int, layout: int = MOE_EP_LINEAR):
    """Host helper: (local_of [n_global] CPU int32 tensor, local slot count)."""
    out = torch.empty(n_global, dtype=torch.int32)
    n = ctypes.c_int32(0)
    _check(lib().moe_ep_local_map(n_global, ep_size, rank, layout, _ptr(out), ctypes.byref(n)),
           "moe_ep_local_map")
    return out, n.value


def moe_eplb_plan(load, n_redundant: int, ep_size: int):
    """Host helper: physical_to_logical map [E + n_redundant] (CPU int32) of
    the EPLB placement for per-expert ``load`` (float64)."""
    load = torch.as_tensor(load, dtype=torch.float64).contiguous()
    E = load.numel()
    out = torch.empty(E + n_redundant, dtype=torch.int32)
    _check(lib().moe_eplb_plan(_ptr(load), E, n_redundant, ep_size, _ptr(out)), "moe_eplb_plan")
    return out


def moe_quantize_1x128(src, rows: int, q, s, stream=None):
    """src bf16 [>=rows, >=C] (row stride src.stride(0)) -> q uint8 [rows, C],
    s fp32 [rows, C/128]; C = q.shape[1]."""
    C = q.shape[1]
    _check(lib().moe_quantize_1x128(_ptr(src), src.stride(0), rows, C, _ptr(q), _ptr(s),
                                    _stream(stream)), "moe_quantize_1x128")


def moe_expert_gate_up_a8(d: Desc, w: Weights, rt: RouteTables, T, xq, xs, h, stream=None):
    _check(lib().moe_expert_gate_up_a8(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                       _ptr(xq), _ptr(xs), _ptr(h), _stream(stream)), "moe_expert_gate_up_a8")


def moe_expert_down_a8(d: Desc, w: Weights, rt: RouteTables, T, hq, hs, y, stream=None):
    _check(lib().moe_expert_down_a8(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                    _ptr(hq), _ptr(hs), _ptr(y), _stream(stream)), "moe_expert_down_a8")


def moe_grouped_ffn_a8(d: Desc, w: Weights, rt: RouteTables, T, x, xq, xs, h, hq, hs, y, stream=None):
    _check(lib().moe_grouped_ffn_a8(ctypes.byref(d.c()), ctypes.byref(w.c), ctypes.byref(rt.c), T,
                                    _ptr(x), _ptr(xq), _ptr(xs), _ptr(h), _ptr(hq), _ptr(hs), _ptr(y),
                                    _stream(stream)), "moe_grouped_ffn_a8")


def moe_replica_map_from_p2l(p2l, E: int, max_replicas: int):
    """Host helper: physical_to_logical_map -> (logical_to_physical_map,
    logical_replica_count) as CPU int32 tensors."""
    p2l = torch.as_tensor(p2l, dtype=torch.int32).contiguous()
    l2p = torch.empty((E, max_replicas), dtype=torch.int32)
    cnt = torch.empty(E, dtype=torch.int32)
    _check(lib().moe_replica_map_from_p2l(_ptr(p2l), E, p2l.numel(), max_replicas,
                                          _ptr(l2p), _ptr(cnt)), "moe_replica_map_from_p2l")
    return l2p, cnt


def moe_decode_fused_workspace_bytes(d: Desc) -> int:
    return int(lib().moe_decode_fused_workspace_bytes(ctypes.byref(d.c())))


def moe_decode_fused(d: Desc, x, w_router, bias, T, logits, rt: RouteTables, ws, w: Weights, h, y, out, fws,
                     router: "GroupedRouter | None" = None, l2p=None, replica_count=None, stream=None):
    """The whole decode layer in one launch (T <= 16); ``fws`` is a device
    uint8 tensor of moe_decode_fused_workspace_bytes(d) bytes, zero-filled
    once before the first call."""
    _check(lib().moe_decode_fused(ctypes.byref(d.c()), _ptr(x), _ptr(w_router), _ptr(bias),
                                  ctypes.byref(router.c) if router is not None else None, _ptr(l2p),
                                  _ptr(replica_count), ctypes.byref(w.c), T, _ptr(logits), ctypes.byref(rt.c),
                                  _ptr(ws), ws.numel() * ws.element_size(), _ptr(h), _ptr(y), _ptr(out),
                                  _ptr(fws), fws.numel() * fws.element_size(), _stream(stream)),
           "moe_decode_fused")


class MoELayer:
    """One layer's device buffers and the C calls in order.  Weights are a
    dict of device tensors as produced for the C ABI layout
    (w1/w3 [E_phys(+1 shared), I, H], w2 [.., H, I], fp8 scales s1/s3/s2);
    the shared expert, if any, is the last slot."""

    def __init__(self, d: Desc, weights: dict, w_router, bias=None, l2p=None,
                 replica_count=None, device="cuda", router: GroupedRouter | None = None,
                 ep: "EPMap | None" = None, a8: bool = False):
        self.d = d
        self.a8 = a8                   # fp8 activations (moe_grouped_ffn_a8), fp8 weights only
        self.router = router           # None: softmax top-K (moe_route)
        self.ep = ep                   # one rank's expert-parallel share (moe_route_ep)
        self.device = device
        self.rt = RouteTables(d, device)
        self.ws = torch.zeros(router_route_workspace_bytes(d), dtype=torch.uint8, device=device)
        rows = buffer_rows(d)
        self.xg = torch.zeros((rows, d.H), dtype=torch.bfloat16, device=device)
        self.h = torch.zeros((rows, d.I), dtype=torch.bfloat16, device=device)
        # the down projection splits K more for fewer tokens: size y for every T
        self.y = torch.zeros(y_bytes_max(d), dtype=torch.uint8, device=device)
        self.logits = torch.zeros((max(1, d.T_max), d.E), dtype=torch.float32, device=device)
        self.w_router = w_router
        self.bias = bias
        self.l2p = l2p
        self.rcount = replica_count
        G = d.E_phys
        routed = {k: (v[:G] if v is not None else None) for k, v in weights.items()}
        shared = None
        if d.n_shared:
            shared = {k: v[G] for k, v in weights.items() if v is not None}
        self.weights = Weights(routed, shared)
        odt = torch.float32 if d.act_dtype == MOE_F32 else torch.bfloat16
        self.out = torch.zeros((max(1, d.T_max), d.H), dtype=odt, device=device)
        # fused decode workspace: zero-filled once, then kept by every call
        self.fws = torch.zeros(moe_decode_fused_workspace_bytes(d), dtype=torch.uint8, device=device)
        if a8:
            T1 = max(1, d.T_max)
            self.xq = torch.zeros((T1, d.H), dtype=torch.uint8, device=device)
            self.xs = torch.zeros((T1, d.H // 128), dtype=torch.float32, device=device)
            self.hq = torch.zeros((rows, d.I), dtype=torch.uint8, device=device)
            self.hs = torch.zeros((rows, d.I // 128), dtype=torch.float32, device=device)

    def y_for(self, T: int) -> torch.Tensor:
        return self.y[: y_bytes(self.d, T)]

    def forward(self, x, T=None, logits=None, stream=None, fused_gather=True):
        """Runs the five steps; ``logits`` (fp32 [T, E]) replaces the router
        step when given.  With bf16 activations the permute is fused into the
        expert kernel (moe_grouped_ffn_x) unless ``fused_gather`` is False.
        Returns the output view [T, H]."""
        d = self.d
        T = x.shape[0] if T is None else T
        if logits is None and self.ep is None and self.router is None:
            # router logits and routing in one call (one launch for tiny T * E)
            moe_router_route(d, x, self.w_router, self.bias, T, self.logits, self.rt, self.ws, self.l2p,
                             self.rcount, stream)
        else:
            if logits is None:
                moe_router_logits(d, x, self.w_router, self.bias, T, self.logits, stream)
                logits = self.logits
            if self.ep is not None:
                moe_route_ep(d, logits, T, self.rt, self.ws, self.ep, self.router, self.l2p, self.rcount,
                             stream)
            elif self.router is None:
                moe_route(d, logits, T, self.rt, self.ws, self.l2p, self.rcount, stream)
            else:
                moe_route_grouped(d, logits, T, self.rt, self.ws, self.router, self.l2p, self.rcount, stream)
        if self.a8:
            moe_grouped_ffn_a8(d, self.weights, self.rt, T, x, self.xq, self.xs, self.h, self.hq, self.hs,
                               self.y, stream)
        elif fused_gather and d.act_dtype == MOE_BF16:
            moe_grouped_ffn_x(d, self.weights, self.rt, T, x, self.h, self.y, stream)
        else:
            moe_permute(d, x, T, self.rt, self.xg, stream)
            moe_grouped_ffn(d, self.weights, self.rt, T, self.xg, self.h, self.y, stream)
        moe_combine(d, self.rt, T, self.y, self.out, stream)
        return self.out[:T]

    def forward_fused(self, x, T=None, stream=None):
        """The same layer in one persistent launch (moe_decode_fused): bf16
        activations, packed weights, T <= 16.  Returns the output view [T, H]."""
        T = x.shape[0] if T is None else T
        moe_decode_fused(self.d, x, self.w_router, self.bias, T, self.logits, self.rt, self.ws, self.weights,
                         self.h, self.y, self.out, self.fws, self.router, self.l2p, self.rcount, stream)
        return self.out[:T]
