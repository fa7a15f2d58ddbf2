// Measurement kernels of known work (include/moe_probe.h): a streaming read
// of device memory and a loop of independent bf16 matrix-core products.
#include <algorithm>

#include "common.hpp"
#include "../../include/moe_probe.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr uint32_t kNeverDigest = 0x9e3779b9u;

// grid-stride read, four 16-byte non-temporal loads in flight per lane
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                                   uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) + (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == kNeverDigest) sink[blockIdx.x] = acc;
}

// eight independent accumulators per wave (tied, as in the expert kernels),
// operands derived from the lane so nothing folds; one store of a digest
// that is, in practice, never taken
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(float)((lane + j) & 7);
    b[j] = (__bf16)(float)((lane * 3 + j) & 5);
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) mfma_acc(acc[j], a, b);
  }
  // the wait states, tied to every accumulator so that no read comes first
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]),
                 "+a"(acc[6]), "+a"(acc[7]));
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j].x + acc[j].y + acc[j].z + acc[j].w;
  if (__float_as_uint(s) == kNeverDigest) sink[blockIdx.x] = __float_as_uint(s);
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status_t moe_probe_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return MOE_ERR_ARG;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  // eight workgroups of four waves per compute unit, within the sink
  const int grid = std::min(std::max(cus, 1) * 8, (int)MOE_PROBE_SINK_WORDS);
  hipLaunchKernelGGL(moe::probe_read_kernel, dim3(grid), dim3(moe::kProbeThreads), 0, stream,
                     static_cast<const moe::u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_probe_mfma_bf16(int32_t iters, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
  if (!sink || iters < 1 || workgroups < 1 || workgroups > (int32_t)MOE_PROBE_SINK_WORDS) return MOE_ERR_ARG;
  hipLaunchKernelGGL(moe::probe_mfma_kernel, dim3(workgroups), dim3(moe::kProbeThreads), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
