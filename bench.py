"""Benchmark of the single-GPU MoE layer forward on MI355X.

One step = one pass of the whole layer over one batch: router logits ->
route (top-K, counts, offsets, grouped order) -> permute -> expert gate/up
(+SwiGLU) -> expert down -> combine, all HIP kernels through the C ABI, on
one stream, with inputs and weights already resident in HBM.  With bf16
activations the permute is done by the gate/up kernel itself (it gathers
each group's rows from x through the route tables).

Default run: every workload at its full size -- the Mixtral-8x7B-shaped
decode layer at B = 1, 8, 32, 64; the DeepSeek-V3-shaped fp8 decode layer at
B = 32, 128, 256; the DeepSeek-V3-shaped bf16 prefill layer at T = 8192; the
544-slot replica decode layer at B = 256 -- each under "batches" with its own
roofline and diagnostics.  The headline value is the Mixtral-shaped B = 64
decode layer.  ``--workload NAME`` times one workload only.

Metric: decode MoE-layer latency (us), lower is better, with the expert-weight
HBM bandwidth it implies (touched weight bytes -- slots with >= 1 token, plus
the shared expert and the router -- over the latency); prefill TFLOP/s.  Each
workload's roofline object is for its dominant kernel, expert gate/up:
algorithmic bytes per launch (W1 + W3 of every touched slot) over its mean
duration for decode, against 8 TB/s; algorithmic FLOPs per launch over its
mean duration for prefill, against 2.5 PFLOP/s bf16.  Durations come from HIP
events on the launch stream over the timed region.  The achievable peaks of
the same device (a streaming read and a matrix-core loop, include/moe_probe.h)
are measured in the same run and reported beside the spec peaks.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, vendor figure
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="time this workload only (default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU reference timing")
    ap.add_argument("--row-major", action="store_true",
                    help="stream the row-major weights instead of the packed layout")
    ap.add_argument("--router", choices=("softmax", "grouped"), default="softmax",
                    help="softmax top-K (default) or the grouped sigmoid router with "
                         "8 groups, 4 kept, group score = sum of the 2 best, weights x2.5")
    ap.add_argument("--a8", action="store_true",
                    help="fp8 weights only: quantize the activations per 1x128 block and run the "
                         "W8A8 expert kernels (fp8 MFMA)")
    ap.add_argument("--ep-ranks", type=int, default=1,
                    help="time rank 0's expert-parallel share of the layer: the linear map over "
                         "the physical slots, E_phys / N local slots (routing of every token, "
                         "experts and combine of the local choices)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 512 MiB device copy three times (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--no-sweep", action="store_true",
                    help="no effect (a named --workload is the only one timed); accepted so that the commands "
                         "recorded in older profiles still run")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no timing: turn the counter_collection.csv files of a FETCH_SIZE and a "
                         "WRITE_SIZE rocprofv3 pass over `bench.py --workload W --copy-calibration` "
                         "into profiles/gate_up_traffic_W.md (needs --workload)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "LOG"),
                    help="no timing: turn a rocprofv3 --kernel-trace --stats run_kernel_stats.csv of "
                         "`bench.py --workload W` (and that run's stderr log, for its bench line) into "
                         "profiles/W_kernel_stats.md (needs --workload)")
    ap.add_argument("--debug-flags", type=int, default=0,
                    help="moe_desc_t.debug_flags for an ablation (MOE_DEBUG_* in include/moe.h: e.g. "
                         "a forced large-group kernel); outputs stay bit-identical")
    return ap.parse_args()


def weight_bytes_per_slot(cfg):
    """Bytes of one SwiGLU expert: 3 matrices of H x I, plus one fp32 scale
    per 128x128 block for fp8."""
    if cfg.w_dtype == "bf16":
        return 3 * cfg.H * cfg.I * 2
    return 3 * cfg.H * cfg.I + 3 * (cfg.H // 128) * (cfg.I // 128) * 4


GROUPED_ROUTER = dict(n_group=8, topk_group=4, group_k=2, renormalize=True, scale=2.5)


class Setup:
    def __init__(self, cfg, packed=True, router="softmax", ep_ranks=1, a8=False, debug_flags=0):
        import numpy as np
        import torch
        from routing_grouped_expert_router_amd import binding as B
        from workloads import generate
        self.cfg = cfg
        self.inp = generate.make_inputs(cfg, wdevice="cuda")
        # expert-parallel share: rank 0 of ep_ranks under the linear map over
        # the physical slots holds only its local slots' weights
        self.local_of = None
        ep = None
        if ep_ranks > 1:
            lo, n_local = B.moe_ep_local_map(cfg.E_phys, ep_ranks, 0, B.MOE_EP_LINEAR)
            self.local_of = lo.numpy()
            slots = [p for p in range(cfg.E_phys) if self.local_of[p] >= 0]
            w = generate.upload_weights(self.inp, "cuda", slots=slots + ([cfg.E_phys] if cfg.n_shared else []))
            idx = torch.tensor(slots + ([cfg.E_phys] if cfg.n_shared else []), device="cuda")
            self.w = {k: v[idx].contiguous() for k, v in w.items()}
            del w
            torch.cuda.empty_cache()
            ep = B.EPMap(lo.cuda())
            cfg = cfg.with_(E_phys=n_local)
            self.cfg = cfg
        else:
            self.w = generate.upload_weights(self.inp, "cuda")
        l2p = rc = None
        max_rep = 1
        if self.inp.p2l is not None:
            import numpy as np
            counts = np.bincount(self.inp.p2l, minlength=cfg.E)
            max_rep = int(counts.max())
            l2p_t, rc_t = B.moe_replica_map_from_p2l(self.inp.p2l, cfg.E, max_rep)
            l2p, rc = l2p_t.cuda(), rc_t.cuda()
        self.d = B.Desc.from_config(cfg, max_replicas=max_rep, w_packed=int(packed))
        self.d.debug_flags = debug_flags
        if packed:   # one-time repack into the streamed layout; free the row-major copy
            w = B.pack_expert_weights(self.d, self.w)
            del self.w
            torch.cuda.empty_cache()
            self.w = w
        self.x = self.inp.x.cuda()
        self.wr = self.inp.w_router.cuda()
        self.bias = None if self.inp.bias is None else self.inp.bias.cuda()
        self.grouped = None
        gr = None
        if router == "grouped":
            sb = generate.make_score_bias(cfg)
            self.grouped = dict(GROUPED_ROUTER, score_bias=sb.numpy())
            gr = B.GroupedRouter(score_bias=sb.cuda(), **GROUPED_ROUTER)
        if a8 and cfg.w_dtype != "fp8":
            raise SystemExit("--a8 needs an fp8-weight workload")
        self.a8 = a8
        self.layer = B.MoELayer(self.d, self.w, self.wr, self.bias, l2p, rc, "cuda", router=gr, ep=ep, a8=a8)
        self.B = B
        torch.cuda.synchronize()

    def step(self, ev=None):
        B, L, d, T = self.B, self.layer, self.d, self.cfg.T
        if L.ep is None and L.router is None:
            B.moe_router_route(d, self.x, self.wr, self.bias, T, L.logits, L.rt, L.ws, L.l2p, L.rcount)
        else:
            B.moe_router_logits(d, self.x, self.wr, self.bias, T, L.logits)
            if L.ep is not None:
                B.moe_route_ep(d, L.logits, T, L.rt, L.ws, L.ep, L.router, L.l2p, L.rcount)
            else:
                B.moe_route_grouped(d, L.logits, T, L.rt, L.ws, L.router, L.l2p, L.rcount)
        if self.a8:
            B.moe_quantize_1x128(self.x, T, L.xq, L.xs)
            if ev is not None:
                ev[0].record()
            B.moe_expert_gate_up_a8(d, L.weights, L.rt, T, L.xq, L.xs, L.h)
            if ev is not None:
                ev[1].record()
            B.moe_quantize_1x128(L.h, B.buffer_rows(d), L.hq, L.hs)
            B.moe_expert_down_a8(d, L.weights, L.rt, T, L.hq, L.hs, L.y)
            if ev is not None:
                ev[2].record()
            B.moe_combine(d, L.rt, T, L.y, L.out)
            return
        gather = d.act_dtype == B.MOE_BF16     # the gate/up kernel gathers rows from x itself
        if not gather:
            B.moe_permute(d, self.x, T, L.rt, L.xg)
        if ev is not None:
            ev[0].record()
        if gather:
            B.moe_expert_gate_up_x(d, L.weights, L.rt, T, self.x, L.h)
        else:
            B.moe_expert_gate_up(d, L.weights, L.rt, T, L.xg, L.h)
        if ev is not None:
            ev[1].record()
        B.moe_expert_down(d, L.weights, L.rt, T, L.h, L.y)
        if ev is not None:
            ev[2].record()
        B.moe_combine(d, L.rt, T, L.y, L.out)

    def fused_ok(self):
        """The single-launch decode layer takes this step: bf16 activations,
        packed weights, T <= 16, bf16 expert activations (not W8A8), no
        expert-parallel map."""
        B, d = self.B, self.d
        return (d.act_dtype == B.MOE_BF16 and d.w_packed == 1 and self.cfg.T <= 16 and not self.a8
                and self.layer.ep is None)

    def step_fused(self):
        self.layer.forward_fused(self.x, self.cfg.T)

    def gate_up_flops(self):
        """Algorithmic FLOPs of the gate/up kernel: 2 * rows * 2I * H over the
        token rows (T*K routed + n_shared*T shared); pad rows not counted."""
        cfg = self.cfg
        rows = cfg.T * cfg.K + cfg.n_shared * cfg.T
        return 2.0 * rows * 2 * cfg.I * cfg.H

    def layer_flops(self):
        cfg = self.cfg
        rows = cfg.T * cfg.K + cfg.n_shared * cfg.T
        return 2.0 * rows * 3 * cfg.I * cfg.H + 2.0 * cfg.T * cfg.E * cfg.H

    def touched(self):
        """(touched slots, touched routed-weight bytes, gate/up bytes, all bytes)"""
        import numpy as np
        cfg = self.cfg
        counts = self.layer.rt.counts.cpu().numpy()
        slots = int((counts > 0).sum())
        per = weight_bytes_per_slot(cfg)
        bpp = 2 if cfg.w_dtype == "bf16" else 1
        scale_gu = 0 if cfg.w_dtype == "bf16" else 2 * (cfg.I // 128) * (cfg.H // 128) * 4
        gu = (slots + cfg.n_shared) * (2 * cfg.I * cfg.H * bpp + scale_gu)
        routed = slots * per
        total = routed + cfg.n_shared * per + cfg.E * cfg.H * 2
        return slots, routed, gu, total


def time_workload(cfg, steps, warmup, packed=True, router="softmax", ep_ranks=1, a8=False, debug_flags=0):
    """Eager steps (HIP events around the gate/up and down kernels on the
    launch stream), then the same step captured once in a HIP graph and
    replayed ``steps`` times (the layer latency reported)."""
    import torch
    s = Setup(cfg, packed, router, ep_ranks, a8, debug_flags)
    cfg = s.cfg
    for _ in range(warmup):
        s.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        s.step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / steps
    gu_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    down_ms = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    ref = s.layer.out.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(s.layer.out, ref), "graph replay differs from the eager step"
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    slots, routed, gu_bytes, total = s.touched()
    status = int(s.layer.rt.status.item())
    res = dict(cfg=cfg, ms=ms, eager_ms=eager_ms, gu_ms=gu_ms, down_ms=down_ms, wall=wall, slots=slots,
               routed_bytes=routed, gu_bytes=gu_bytes, total_bytes=total, status=status, setup=s,
               gu_flops=s.gate_up_flops(), layer_flops=s.layer_flops(),
               counts=s.layer.rt.counts.cpu().numpy(),
               gu_kernel=kernel_name(s, 0), down_kernel=kernel_name(s, 1), a8=s.a8)
    del graph
    if s.fused_ok():
        # the single-launch step is reported beside the multi-launch one; a
        # failure there (e.g. a barrier timeout) is reported, not fatal
        try:
            res.update(time_fused(s, steps, warmup, ref))
        except (AssertionError, RuntimeError) as e:
            print(f"# {cfg.name}: single-launch step not timed: {e}", file=sys.stderr, flush=True)
            s.layer.fws.zero_()
            torch.cuda.synchronize()
    return res


def kernel_name(s, which):
    """The expert kernel the step runs for its largest groups (which = 0
    gate/up, 1 down)."""
    return (s.B.expert_kernel_a8 if s.a8 else s.B.expert_kernel)(s.d, s.cfg.T, which)


def time_fused(s, steps, warmup, ref):
    """The same layer step as one persistent launch (moe_decode_fused):
    checked bit for bit against the multi-launch step, then timed launched
    directly and as a replayed HIP graph."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        s.step_fused()
    torch.cuda.synchronize()
    assert torch.equal(s.layer.out, ref), "the single-launch step differs from the multi-launch step"
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        s.step_fused()
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        s.step_fused()
    for _ in range(warmup):
        graph.replay()
    start.record(stream)
    for _ in range(steps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(s.layer.out, ref), "graph replay of the single-launch step differs"
    status = int(s.layer.rt.status.item())
    assert not status & s.B.MOE_STATUS_SYNC_TIMEOUT, "grid barrier timed out"
    del graph
    return dict(fused_ms=start.elapsed_time(end) / steps, fused_eager_ms=eager_ms)


def achievable_peaks(reps=5):
    """Streaming-read GB/s over a 4 GiB buffer (16x the last-level cache) and
    bf16 matrix-core TFLOP/s of a loop with no memory traffic, measured on
    this device with HIP events (include/moe_probe.h)."""
    import torch
    from routing_grouped_expert_router_amd import binding as B
    stream = torch.cuda.current_stream()
    sink = torch.zeros(B.MOE_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        B.moe_probe_read(buf, sink)
    start.record(stream)
    for _ in range(reps):
        B.moe_probe_read(buf, sink)
    end.record(stream)
    torch.cuda.synchronize()
    read_gbs = buf.numel() * reps / (start.elapsed_time(end) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = min(8 * cus, B.MOE_PROBE_SINK_WORDS), 10000
    B.moe_probe_mfma_bf16(iters, wgs, sink)
    start.record(stream)
    for _ in range(reps):
        B.moe_probe_mfma_bf16(iters, wgs, sink)
    end.record(stream)
    torch.cuda.synchronize()
    flops = wgs * 4.0 * iters * 8 * 16384 * reps
    mfma_tf = flops / (start.elapsed_time(end) * 1e-3) / 1e12
    return {"hbm_read_gbs": round(read_gbs, 1), "mfma_bf16_tflops": round(mfma_tf, 1),
            "how": "moe_probe_read: one non-temporal 16-byte-load pass over 4 GiB; moe_probe_mfma_bf16: "
                   f"{wgs} workgroups x 4 waves x {iters} x 8 independent v_mfma_f32_16x16x32_bf16; "
                   f"mean of {reps} launches timed with HIP events"}


PREFILL_MIN_T = 1024   # token counts from here on are timed against the MFMA peak

DEFAULT_WORKLOADS = ["mixtral_decode_b1", "mixtral_decode_b8", "mixtral_decode_b32", "mixtral_decode_b64",
                     "dsv3_decode_b32", "dsv3_decode_b128", "dsv3_decode_b256", "dsv3_prefill_t8192",
                     "dsv3_prefill_t8192_fp8", "replica_decode_b256"]
# workloads timed on the W8A8 path (fp8 activations on fp8 MFMA) whatever --a8 says
A8_WORKLOADS = {"dsv3_prefill_t8192_fp8"}
HEADLINE = "mixtral_decode_b64"


def kernel_sources_hash(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "routing_grouped_expert_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary (profiles/gate_up_traffic_<workload>.md: FETCH_SIZE and
    WRITE_SIZE passes scaled by a plain copy of known size), or None when
    there is none, it was taken of another kernel, or the kernel's sources
    (listed in the summary) changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"gate_up_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "*", "#", "|")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    files = vals.get("kernel_sources", "").split()
    if vals.get("kernel") != kernel or not files or \
            vals.get("kernel_sources_sha256_16") != kernel_sources_hash(files):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


KERNEL_FILE = {"ffn_stream_kernel": "ffn_stream.hip", "ffn_tall_kernel": "ffn_tiled.hip",
               "ffn_a8_tall_kernel": "ffn_a8_tall.hip", "ffn_a8_kernel": "ffn_a8.hip",
               "ffn_whyb_kernel": "ffn_tiled.hip", "ffn_wdma_kernel": "ffn_tiled.hip",
               "ffn_wide_kernel": "ffn_tiled.hip", "ffn_tiled_kernel": "ffn_tiled.hip"}


def kernel_sources(kernel: str) -> list:
    """The csrc files a kernel is compiled from: its translation unit and the
    local headers it includes, recursively."""
    import re
    csrc = os.path.join(ROOT, "routing_grouped_expert_router_amd", "csrc")
    seen, todo = [], [KERNEL_FILE[kernel]]
    while todo:
        f = todo.pop(0)
        if f in seen or not os.path.exists(os.path.join(csrc, f)):
            continue
        seen.append(f)
        with open(os.path.join(csrc, f)) as fh:
            todo += re.findall(r'^#include "([^"]+)"', fh.read(), re.M)
    return sorted(seen)


def summarize_traffic(workload: str, fetch_csv: str, write_csv: str, cmd_prefix: str):
    """profiles/gate_up_traffic_<workload>.md from two counter passes: the
    first three device copies (the 512 MiB calibration of --copy-calibration)
    give the factor from counter units to bytes, the gate/up kernel's
    dispatches the bytes per launch."""
    import csv
    import re
    from workloads import configs
    from routing_grouped_expert_router_amd import binding as B
    cfg = configs.by_name(workload)
    d = B.Desc.from_config(cfg, w_packed=1)
    kernel = (B.expert_kernel_a8 if workload in A8_WORKLOADS else B.expert_kernel)(d, cfg.T, 0)
    mode0 = (re.compile(r"ffn_stream_kernel<(true|false), 0,") if kernel == "ffn_stream_kernel"
             else re.compile(re.escape(kernel) + r"<0[,>]"))
    cal_bytes = 512 << 20
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        with open(path) as fh:
            rows = [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        cal = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"] == "__amd_rocclr_copyBuffer"][:3]
        ker = [float(r["Counter_Value"]) for r in rows if mode0.search(r["Kernel_Name"])]
        names = sorted({r["Kernel_Name"] for r in rows if mode0.search(r["Kernel_Name"])})
        if len(cal) < 3 or max(cal) > 1.05 * min(cal) or not ker:
            raise SystemExit(f"{path}: calibration copies {cal} / {len(ker)} gate/up dispatches unusable")
        factor = cal_bytes / 1024 / (sum(cal) / 3)
        out[counter] = dict(cal=sum(cal) / 3, factor=factor, n=len(ker), kib=sum(ker) / len(ker),
                            bytes=int(round(sum(ker) / len(ker) * 1024 * factor)), names=names)
    rd, wr = out["FETCH_SIZE"], out["WRITE_SIZE"]
    files = kernel_sources(kernel)
    lines = [
        f"# HBM traffic of the expert gate/up kernel, workload {workload}",
        "",
        "Two counter passes, one counter each, over the bench with a 512 MiB plain device copy run "
        "three times first as the calibration kernel of known traffic (repository root on the GPU "
        "box, `R=$PWD`):",
        "",
        f"    {cmd_prefix} --kernel-include-regex '{kernel}|copyBuffer' --pmc FETCH_SIZE --output-format csv "
        f"-d $OUT/{workload}_FETCH_SIZE -o run -- "
        f"python3 $R/bench.py --workload {workload} --no-cpu --no-peaks --steps 3 --warmup 1 --copy-calibration",
        f"    {cmd_prefix} --kernel-include-regex '{kernel}|copyBuffer' --pmc WRITE_SIZE --output-format csv "
        f"-d $OUT/{workload}_WRITE_SIZE -o run -- "
        f"python3 $R/bench.py --workload {workload} --no-cpu --no-peaks --steps 3 --warmup 1 --copy-calibration",
        f"    python3 bench.py --workload {workload} --summarize-traffic "
        f"$OUT/{workload}_FETCH_SIZE/run_counter_collection.csv "
        f"$OUT/{workload}_WRITE_SIZE/run_counter_collection.csv",
        "",
        f"* calibration copy (512 MiB each way): FETCH_SIZE {rd['cal']:.0f} KiB -> factor {rd['factor']:.4f}; "
        f"WRITE_SIZE {wr['cal']:.0f} KiB -> factor {wr['factor']:.4f}",
        f"* kernel `{', '.join(rd['names'])}` ({rd['n']} dispatches): FETCH_SIZE {rd['kib']:.0f} KiB, "
        f"WRITE_SIZE {wr['kib']:.0f} KiB per dispatch",
        f"* scaled HBM bytes per launch: read {rd['bytes']} + write {wr['bytes']} = {rd['bytes'] + wr['bytes']}",
        "",
        f"traffic_bytes_per_launch: {rd['bytes'] + wr['bytes']}",
        f"kernel: {kernel}",
        f"kernel_sources: {' '.join(files)}",
        f"kernel_sources_sha256_16: {kernel_sources_hash(files)}",
        "",
    ]
    path = os.path.join(ROOT, "profiles", f"gate_up_traffic_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {path}: {rd['bytes'] + wr['bytes']} bytes per launch")


def summarize_stats(workload: str, stats_csv: str, log: str, steps: int, warmup: int):
    """profiles/<workload>_kernel_stats.md from the per-kernel statistics of a
    kernel-trace run of the bench on that workload (the library's kernels)."""
    import csv
    from workloads import configs
    cfg = configs.by_name(workload)
    with open(stats_csv) as fh:
        rows = [r for r in csv.DictReader(fh) if "moe::" in r["Name"] and "pack_kernel" not in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    bench_lines = []
    with open(log) as fh:
        bench_lines = [ln.rstrip() for ln in fh if ln.startswith(f"# {workload}:")]
    name = lambda n: n.replace("void ", "").replace("moe::", "").split("(")[0]
    lines = [
        f"# rocprofv3 kernel statistics: workload {workload}",
        "",
        f"T={cfg.T}, H={cfg.H}, I={cfg.I}, E={cfg.E}, E_phys={cfg.E_phys}, K={cfg.K}, n_shared={cfg.n_shared}, "
        f"weights {cfg.w_dtype}, layout {cfg.layout}.  Command (`R` the repository root, `OUT` an output folder):",
        "",
        f"    cd /tmp && TMPDIR=/tmp timeout -k 10 300 rocprofv3 --kernel-include-regex 'moe' --kernel-trace --stats "
        f"--output-format csv "
        f"-d $OUT/{workload} -o run -- python3 $R/bench.py --workload {workload} --no-cpu --no-peaks "
        f"--steps {steps} --warmup {warmup} 2> $OUT/{workload}.log",
        f"    python3 bench.py --workload {workload} --summarize-stats "
        f"$OUT/{workload}/run_kernel_stats.csv $OUT/{workload}.log",
        "",
        "The library's kernels (the one-time weight packing left out); durations in microseconds, over the "
        "eager and graph-replayed steps of the run.",
        "",
        "| kernel | calls | avg us | min us | max us | share of these kernels |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(f"| `{name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")
    lines += ["", "Bench line printed by the same run:", ""] + [f"    {ln}" for ln in bench_lines] + [""]
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_stats.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {path}")


def roofline(cfg, r, peaks):
    """The dominant kernel (expert gate/up + SwiGLU) against its bound: HBM
    bytes for decode, bf16 MFMA FLOPs for prefill."""
    kernel = f"{r['gu_kernel']} gate/up (W1+W3, SwiGLU)"
    if cfg.T >= PREFILL_MIN_T:
        tf = r["gu_flops"] / (r["gu_ms"] * 1e-3) / 1e12
        peak = FP8_PEAK_TFLOPS if r.get("a8") else BF16_PEAK_TFLOPS   # the MFMA type the kernel runs
        out = {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 1),
               "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
               "mfma_dtype": "fp8" if r.get("a8") else "bf16",
               "traffic": measured_traffic(cfg.name, r["gu_kernel"]), "kernel_us": round(r["gu_ms"] * 1e3, 2),
               "algorithmic_flops": r["gu_flops"]}
        if peaks and not r.get("a8"):
            out["achievable_peak"] = peaks["mfma_bf16_tflops"]
            out["frac_of_achievable"] = round(tf / peaks["mfma_bf16_tflops"], 4)
        return out
    gbs = r["gu_bytes"] / (r["gu_ms"] * 1e-3) / 1e9
    out = {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "traffic": measured_traffic(cfg.name, r["gu_kernel"]),
           "kernel_us": round(r["gu_ms"] * 1e3, 2), "algorithmic_bytes": r["gu_bytes"]}
    if peaks:
        out["achievable_peak"] = peaks["hbm_read_gbs"]
        out["frac_of_achievable"] = round(gbs / peaks["hbm_read_gbs"], 4)
    return out


def diagnostics(cfg, r, splits):
    """The pages' cost terms for this batch ("推理 INFRA 方法论(5)", DeepGEMM
    and C(B) sections): pad-row FLOP waste ceil(M_e/BM)*BM/M_e summed over
    the groups at the row granularity the expert kernel skips empty rows at
    (16-row MFMA tiles when streaming, 32-row sub-tiles in the large-group
    kernels), rows sent to the spill region of a masked buffer, the
    activation bytes the step moves (reported apart from the weight bytes),
    and the expected distinct experts E*C(B) of a uniform router,
    C(B) = 1 - (1 - K/E)^B, beside the slots the batch touched."""
    import numpy as np
    counts = np.asarray(r["counts"], dtype=np.int64)
    T, K, H, I = cfg.T, cfg.K, cfg.H, cfg.I
    gran = 16 if r["gu_kernel"] == "ffn_stream_kernel" else 32
    rows = np.concatenate([counts[counts > 0], [T] * cfg.n_shared])
    waste = float((-(-rows // gran) * gran).sum() / max(1, rows.sum()))
    spill = int(np.maximum(counts - cfg.M_max, 0).sum()) if cfg.layout == "masked" else 0
    grouped = T * K + cfg.n_shared * T
    ybytes = 2 if splits == 1 else 4 * splits
    act = (T * H * 2                    # x read by the router
           + T * cfg.E * 4 * 2          # logits written and read
           + grouped * H * 2            # rows gathered by gate/up
           + grouped * I * 2 * 2        # h written and read
           + grouped * H * ybytes * 2   # y written and read
           + T * H * 2)                 # out
    cb = 1.0 - (1.0 - K / cfg.E) ** T
    return {"pad_flop_waste": round(waste, 4), "pad_rows_granularity": gran, "spill_rows": spill,
            "activation_bytes": int(act), "weight_bytes": int(r["total_bytes"]),
            "expected_experts_uniform": round(cfg.E * cb, 2), "touched_slots": r["slots"]}


def cpu_baseline(s, budget_s=30.0):
    """The CPU reference, as it stands, on a bounded sample of the workload:
    all routing for the whole batch plus the expert FFN and combine for a
    sample of tokens.  Returns (us per full layer call, sample description,
    threads)."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import moe_oracle as O
    from oracle_adapt import oracle_forward
    cfg = s.cfg
    inp = s.inp
    # copy every expert the batch touches to host memory first (not timed)
    counts = s.layer.rt.counts.cpu().numpy()
    print(f"# cpu reference: copying {int((counts > 0).sum())} experts to host memory",
          file=sys.stderr, flush=True)
    inp.prefetch(sorted({inp.slot_logical(p) for p in np.nonzero(counts)[0]}))
    T = cfg.T
    # double the token sample from 1 while the last run stayed under a quarter
    # of the budget (the cost per token is not known beforehand: it is set by
    # the distinct experts the sample touches)
    n = 1
    while True:
        toks = np.arange(0, T, max(1, T // n))[:n]
        t0 = time.perf_counter()
        if s.a8:
            from oracle_adapt import oracle_forward_w8a8
            oracle_forward_w8a8(inp, tokens=toks, local_of=s.local_of,
                                E_local=None if s.local_of is None else cfg.E_phys)
        else:
            oracle_forward(inp, tokens=toks, grouped=s.grouped, local_of=s.local_of,
                           E_local=None if s.local_of is None else cfg.E_phys)
        dt = time.perf_counter() - t0
        print(f"# cpu reference: {len(toks)} of {T} tokens in {dt:.1f} s", file=sys.stderr, flush=True)
        if n >= T or dt * 4 > budget_s:
            break
        n = min(T, 2 * n)
    # scale: routing is over the full batch; the FFN part is per token
    frac = len(toks) / T
    est = dt / frac if frac > 0 else dt
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    return est * 1e6, f"{len(toks)} of {T} tokens (routing over all {T}); fp64 numpy; " \
                      f"measured {dt:.1f} s, scaled by tokens", cores


def batch_entry(r, peaks):
    cfg = r["cfg"]
    B = r["setup"].B
    splits = B.down_splits(r["setup"].d, cfg.T)
    e = {"latency_us": round(r["ms"] * 1e3, 2),
         "eager_latency_us": round(r["eager_ms"] * 1e3, 2),
         "gbs": round(r["total_bytes"] / (r["ms"] * 1e-3) / 1e9, 1),
         "layer_tflops": round(r["layer_flops"] / (r["ms"] * 1e-3) / 1e12, 2),
         "gate_up_us": round(r["gu_ms"] * 1e3, 2),
         "down_us": round(r["down_ms"] * 1e3, 2),
         "down_kernel": r["down_kernel"],
         "touched_slots": r["slots"],
         "touched_bytes": r["total_bytes"],
         "w_dtype": cfg.w_dtype,
         "activations": "fp8-e4m3 1x128 (W8A8)" if r.get("a8") else "bf16",
         "status": r["status"],
         "roofline": roofline(cfg, r, peaks),
         "diagnostics": diagnostics(cfg, r, splits),
         "single_launch_latency_us": round(r["fused_ms"] * 1e3, 2) if "fused_ms" in r else None}
    if cfg.T >= PREFILL_MIN_T:
        down_flops = r["layer_flops"] - r["gu_flops"] - 2.0 * cfg.T * cfg.E * cfg.H
        e["down_tflops"] = round(down_flops / (r["down_ms"] * 1e-3) / 1e12, 1)
    return e


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the MoE layer here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.summarize_stats:
        if not args.workload:
            raise SystemExit("--summarize-stats needs --workload")
        summarize_stats(args.workload, *args.summarize_stats, args.steps, args.warmup)
        return
    if args.summarize_traffic:
        if not args.workload:
            raise SystemExit("--summarize-traffic needs --workload")
        summarize_traffic(args.workload, *args.summarize_traffic,
                          "cd /tmp && TMPDIR=/tmp timeout -s KILL 150 rocprofv3")
        return
    import torch
    from workloads import configs
    if args.copy_calibration:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = [configs.by_name(args.workload).name] if args.workload else list(DEFAULT_WORKLOADS)
    head_name = HEADLINE if HEADLINE in names else names[0]
    peaks = None
    if not args.no_peaks:
        peaks = achievable_peaks()
        print(f"# achievable: streaming read {peaks['hbm_read_gbs']:.0f} GB/s, "
              f"bf16 MFMA {peaks['mfma_bf16_tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    results = {}
    for n in names:
        c = configs.by_name(n)
        r = time_workload(c, args.steps, args.warmup, packed=not args.row_major,
                          router=args.router, ep_ranks=args.ep_ranks, a8=args.a8 or n in A8_WORKLOADS,
                          debug_flags=args.debug_flags)
        results[n] = r
        r["entry"] = batch_entry(r, peaks)
        print(f"# {n}: {r['ms']*1e3:.1f} us/layer (graph), {r['eager_ms']*1e3:.1f} eager, "
              f"gate/up {r['gu_ms']*1e3:.1f} us ({r['gu_flops']/(r['gu_ms']*1e-3)/1e12:.0f} TFLOP/s, "
              f"{r['gu_kernel']}), down {r['down_ms']*1e3:.1f} us, "
              f"layer {r['layer_flops']/(r['ms']*1e-3)/1e12:.0f} TFLOP/s, "
              f"slots {r['slots']}, touched {r['total_bytes']/1e9:.3f} GB -> "
              f"{r['total_bytes']/(r['ms']*1e-3)/1e9:.0f} GB/s, status {r['status']}"
              + (f"; single launch {r['fused_ms']*1e3:.1f} us (graph), {r['fused_eager_ms']*1e3:.1f} eager"
                 if "fused_ms" in r else ""),
              file=sys.stderr, flush=True)
        if n != head_name:
            del r["setup"]
            torch.cuda.empty_cache()
    head = results[head_name]
    cfg = head["cfg"]
    lat_us = head["ms"] * 1e3
    gb_s = head["total_bytes"] / (head["ms"] * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu:
        us, sample, cores = cpu_baseline(head["setup"])
        cpu = {"value": round(us, 1), "unit": "us", "cores": cores, "kind": "oracle",
               "sample": sample}
    prefill = next((results[n] for n in names if configs.by_name(n).T >= PREFILL_MIN_T), None)
    out = {
        "metric": "decode MoE-layer latency (us) + expert-weight HBM GB/s; prefill TFLOP/s",
        "value": round(lat_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.w_dtype == "bf16" else (
            "fp8-e4m3-b128 weights, fp8-e4m3 1x128 activations (W8A8)" if args.a8 or head_name in A8_WORKLOADS
            else "fp8-e4m3-b128 weights, bf16 activations"),
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "E_phys": cfg.E_phys, "K": cfg.K, "n_shared": cfg.n_shared,
                   "layout": cfg.layout, "M_max": cfg.M_max, "w_dtype": cfg.w_dtype,
                   "weights": "row-major" if args.row_major else "packed",
                   "debug_flags": args.debug_flags,
                   "router": args.router if args.router == "softmax" else
                   "grouped sigmoid (8 groups, 4 kept, top-2 group score, x2.5)",
                   "ep": None if args.ep_ranks == 1 else
                   {"ranks": args.ep_ranks, "rank": 0, "map": "linear",
                    "local_slots": head["cfg"].E_phys}},
        "expert_weight_hbm_gbs": round(gb_s, 1),
        "layer_tflops": round(head["layer_flops"] / (head["ms"] * 1e-3) / 1e12, 2),
        "prefill_tflops": None if prefill is None else
        round(prefill["layer_flops"] / (prefill["ms"] * 1e-3) / 1e12, 1),
        "touched_slots": head["slots"],
        "touched_bytes": head["total_bytes"],
        "roofline": head["entry"]["roofline"],
        "cpu_baseline": cpu,
        "achievable_peaks": peaks,
        "eager_latency_us": round(head["eager_ms"] * 1e3, 2),
        "timing": "HIP graph of one layer step replayed `steps` times between HIP events "
                  "on the launch stream; eager_latency_us is the same step launched directly; "
                  "kernel times from HIP events around each expert kernel in the eager steps",
        "batches": {n: r["entry"] for n, r in results.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
