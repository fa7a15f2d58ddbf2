// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// a compile-time int as a type, for generic lambdas that unroll over it
template <int V>
struct IntC { static constexpr int value = V; };

constexpr int kWave = 64;
constexpr int kMaxK = 16;      // experts per token supported by the router
constexpr int kMaxE = 4096;    // logical / physical experts supported
constexpr int kBlockTokens = 64;  // tokens per routing block (one u64 mask)

// ---- bf16 ---------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
// (a select, not a branch: in unrolled epilogues a branch per element splits
// the code into blocks that the register allocator handles badly)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = (u >> 16) | 0x40u;
  return uint16_t((u & 0x7fffffffu) > 0x7f800000u ? qnan : rne);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---- OCP E4M3FN -> bf16 (exact: every E4M3 value is a bf16 value) ---------
// Four fp8 bytes of `w` -> four bf16 in two dwords, byte order preserved.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// 16 fp8 bytes -> two bf16x8 MFMA operands (bytes 0..7, bytes 8..15).
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4 q, bf16x8& a0, bf16x8& a1) {
  u32x2 p0 = fp8x4_to_bf16x4(q.x), p1 = fp8x4_to_bf16x4(q.y);
  u32x2 p2 = fp8x4_to_bf16x4(q.z), p3 = fp8x4_to_bf16x4(q.w);
  u32x4 v0 = {p0.x, p0.y, p1.x, p1.y};
  u32x4 v1 = {p2.x, p2.y, p3.x, p3.y};
  a0 = __builtin_bit_cast(bf16x8, v0);
  a1 = __builtin_bit_cast(bf16x8, v1);
}

// Raw buffer resource over [p, p + bytes): loads take a 32-bit per-lane
// offset and a wave-uniform 32-bit offset, so the K step moves a scalar only
// (no per-load 64-bit address arithmetic or address registers), and a load
// past `bytes` returns zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// ---- MFMA ---------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16].
// Lane l supplies A row (l % 16), B column (l % 16), each with 8 K values
// (the K set of lane group l / 16); lane l receives D rows 4*(l/16)+0..3 of
// column l % 16.  Any K assignment works as long as A and B agree on it.
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 a, const bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D += A * B of v_mfma_f32_16x16x32_bf16 on an accumulator that stays in its
// accumulation registers: the operand is tied, so the register allocator
// cannot rotate the 256 accumulators of a wave through copies between loop
// stages (it does with the builtin's separate source and result at this
// register count, and the overlapping copies serialise the matrix core).
// Every use accumulates into exactly the registers it reads, which the
// matrix core chains back to back; the operands come from loads and LDS
// reads the compiler waits for.  The compiler does not know the statement is
// a multi-pass product, so it inserts no wait states before instructions
// that read its result: acc_fence() must separate the last product from any
// read of the accumulators, including moves the compiler adds at the exit of
// the loop holding the products.
__device__ __forceinline__ void mfma_acc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// wait states between the last product and the first read of its result
// (more than the longest product's passes); the scheduling barriers keep the
// compiler from moving reads of the accumulators above it
__device__ __forceinline__ void acc_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}


// ---- ordering key for top-K ------------------------------------------------
// Monotone map fp32 -> u32 with -0 == +0 and NaN below -inf (key 0).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key on finite values (key 0, the NaN class, maps back to
// NaN; -0 comes back as +0, which no arithmetic here tells apart).
__device__ __forceinline__ float order_key_value(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// (value, id) packed so that a larger key is a larger value, ties to the
// lower id.  A removed entry is 0, below every real key.
__device__ __forceinline__ uint64_t topk_key(float v, int id) {
  return (uint64_t(order_key(v)) << 32) | uint64_t(0xffffffffu - uint32_t(id));
}

// One step of a max-scan across lanes by a DPP move (row shift or row
// broadcast; lanes the move does not reach read 0, which every key exceeds)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROW_MASK, 0xf, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROW_MASK, 0xf, true);
  const uint64_t o = (uint64_t(hi) << 32) | lo;
  return o > v ? o : v;
}

// The largest 64-bit value over the 64 lanes, returned to every lane: row
// shifts by 1, 2, 4 and 8 leave each 16-lane row's maximum in its lane 15,
// the row broadcasts of lanes 15 and 31 carry them on to lane 63, which is
// read back.  No lane exchange goes through LDS (as __shfl_xor does), so a
// step costs a few ALU cycles instead of an LDS round trip.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111, 0xf>(v);   // row_shr:1
  v = dpp_max_step<0x112, 0xf>(v);   // row_shr:2
  v = dpp_max_step<0x114, 0xf>(v);   // row_shr:4
  v = dpp_max_step<0x118, 0xf>(v);   // row_shr:8
  v = dpp_max_step<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return (uint64_t(hi) << 32) | lo;
}

// The largest 32-bit value over the 64 lanes, to every lane (the same row
// shifts and broadcasts as wave_max_u64 on one word).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_step32(uint32_t v) {
  const uint32_t o = __builtin_amdgcn_update_dpp(0u, v, CTRL, ROW_MASK, 0xf, true);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step32<0x111, 0xf>(v);
  v = dpp_max_step32<0x112, 0xf>(v);
  v = dpp_max_step32<0x114, 0xf>(v);
  v = dpp_max_step32<0x118, 0xf>(v);
  v = dpp_max_step32<0x142, 0xa>(v);
  v = dpp_max_step32<0x143, 0xc>(v);
  return __builtin_amdgcn_readlane(v, 63);
}

// wave_max_u64 by 32-bit steps: the maximum of the high words; then, if one
// lane holds it, that lane's low word, else the maximum low word among the
// lanes that hold it.  Same result, about a third of the instructions when
// high words rarely tie (the top-K keys: a tie is two equal logits).
// Every lane of the wave must be active.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
  const uint32_t mh = wave_max_u32(hi);
  const uint64_t tie = __ballot(hi == mh);
  uint32_t ml;
  if (__popcll(tie) == 1) ml = __builtin_amdgcn_readlane(lo, __builtin_ctzll(tie));
  else ml = wave_max_u32(hi == mh ? lo : 0u);
  return (uint64_t(mh) << 32) | ml;
}

// A workgroup barrier that orders LDS accesses only: it waits for the
// wave's LDS operations, not for its outstanding global stores, which
// __syncthreads() also waits for (an L2 round trip).  For phases that hand
// each other data in LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive scans of N arrays of n (<= 4 * blockDim.x) ints each in LDS
// (arr[0..N-1]), in place, by the whole workgroup, sharing one set of
// barriers; total[q] = the sum of arr[q].  `tmp` needs N * (blockDim.x/64 + 1)
// ints.  Integer sums: the results do not depend on the grouping.
template <int N>
__device__ inline void block_exclusive_scan_n(int* const (&arr)[N], int n, int* tmp, int (&total)[N]) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int nw = nt / 64;
  const int per = (n + nt - 1) / nt;
  const int lo = tid * per, hi = min(lo + per, n);
  const int lane = tid & 63, wv = tid >> 6;
  int s[N], x[N];
#pragma unroll
  for (int q = 0; q < N; ++q) {
    s[q] = 0;
    for (int i = lo; i < hi; ++i) s[q] += arr[q][i];
    // inclusive scan of s across the wave
    x[q] = s[q];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x[q], off, kWave);
      if (lane >= off) x[q] += y;
    }
    if (lane == 63) tmp[q * (nw + 1) + wv] = x[q];
  }
  lds_barrier();
  // the waves' totals (at most 16 per array) scanned by the first wave's lanes
  if (wv == 0) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      int* t = tmp + q * (nw + 1);
      const int c = lane < nw ? t[lane] : 0;
      int r = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(r, off, kWave);
        if (lane >= off) r += y;
      }
      if (lane < nw) t[lane] = r - c;
      if (lane == nw - 1) t[nw] = r;
    }
  }
  lds_barrier();
#pragma unroll
  for (int q = 0; q < N; ++q) {
    const int* t = tmp + q * (nw + 1);
    int base = t[wv] + x[q] - s[q];
    for (int i = lo; i < hi; ++i) { const int c = arr[q][i]; arr[q][i] = base; base += c; }
    total[q] = t[nw];
  }
  lds_barrier();
}

// Exclusive scan of n (<= 4 * blockDim.x) ints in LDS `a`, in place, by the
// whole workgroup; returns the total.  `tmp` needs blockDim.x/64 + 1 ints.
__device__ inline int block_exclusive_scan(int* a, int n, int* tmp) {
  int* const arr[1] = {a};
  int total[1];
  block_exclusive_scan_n<1>(arr, n, tmp, total);
  return total[0];
}

}  // namespace moe
