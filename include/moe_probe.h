/*
 * moe_probe.h -- measurement helpers of the MoE-layer library: kernels of
 * known work that measure, on the device at hand and in the same process as
 * the layer, the peaks the layer's kernels are compared with.  Not part of
 * the layer's hot path.
 *
 * The MoE layer's decode steps are bound by reading the touched expert
 * weights from HBM and its prefill by the matrix cores ("推理 INFRA
 * 方法论(5)", C(B) and DeepGEMM sections: decode reads C(B) of the routed
 * weights; the tile knee where a tile stops being bandwidth-bound).  Vendor
 * figures give the spec peaks; these kernels give the achievable ones:
 *   - a streaming read of a device buffer, non-temporal 16-byte loads, four
 *     in flight per lane (the access the decode kernels make), and
 *   - a loop of independent bf16 16x16x32 matrix-core products (the product
 *     the expert kernels issue), no memory traffic.
 * Conventions as in moe.h: caller-owned device memory, enqueue only on
 * `stream`, argument errors returned before anything is enqueued.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the sink buffer every probe needs (device uint32). */
#define MOE_PROBE_SINK_WORDS 8192

/* Reads `bytes` (a positive multiple of 16) of device memory at `buf`
 * (16-byte aligned) once, in a grid-stride walk of 16-byte non-temporal
 * loads, and stores a digest of the data to `sink` only when a digest is
 * 0x9e3779b9 (which keeps the loads live and writes, in practice, nothing).
 * Bytes moved: `bytes` read.  MOE_ERR_ARG for a NULL pointer or a bad size. */
moe_status_t moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Runs `iters` (>= 1) iterations of eight independent
 * v_mfma_f32_16x16x32_bf16 per wave in `workgroups` (1..4096) workgroups of
 * four waves, and stores a digest to `sink` as moe_probe_read does.
 * FLOPs: workgroups * 4 * iters * 8 * 16384.  MOE_ERR_ARG for bad counts. */
moe_status_t moe_probe_mfma_bf16(int32_t iters, int32_t workgroups, uint32_t* sink,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H */
