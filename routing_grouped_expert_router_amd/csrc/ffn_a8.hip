// W8A8 expert projections on gfx950: fp8 (E4M3FN) weights and activations,
// fp8 MFMA, per-128 block scales, two-level accumulation.
//
// ("推理 INFRA 方法论(5)", DeepGEMM section: FP8 operands with per-128 scales;
// the matrix unit sums one 128-wide K block, the block sum is promoted to fp32,
// multiplied by its scales and accumulated.)
//
//  * quant_1x128_kernel: each row's 128-wide K block gets s = amax / 448
//    (1 for an all-zero block) and E4M3FN codes of x / s (IEEE fp32 division,
//    round to nearest even, clamped to +-448), stored in natural K order.
//  * ffn_a8_kernel: a streaming kernel for decode-sized groups.  A workgroup
//    owns 64 weight rows of one group (wave w: the 16-row panel n0 + 16w, and
//    for gate/up the same rows of W3); the group's token rows run in passes
//    of MT tiles of 16.  Per 128-wide K step each lane holds 32 weight bytes
//    -- the packed layout's two 16-byte pieces, K offsets 16g..16g+15 and
//    64+16g..64+16g+15 for lane group g -- and the same 32 K of its token row,
//    so one v_mfma_scale_f32_16x16x128_f8f6f4 (unit E8M0 scales) gives the
//    block sum; it is scaled by the weight block's scale times the token's
//    and added to the fp32 accumulator.  Weights and activations run NB - 1
//    steps ahead in registers.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float a8_silu(float g) { return g / (1.0f + __expf(-g)); }

// E4M3FN codes of four fp32 values, bytes in order
__device__ __forceinline__ uint32_t a8_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__global__ __launch_bounds__(256) void quant_1x128_kernel(QuantArgs a) {
  const int nb = a.C / 128;
  const int64_t blk = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;   // (row, block)
  const int sub = threadIdx.x & 15;                                    // 8 values each
  const bool live = blk < a.rows * nb;
  const int64_t row = live ? blk / nb : 0;
  const int b = live ? int(blk % nb) : 0;
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.src + row * a.ld + b * 128 + sub * 8);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
  const float s = m > 0.f ? m / 448.0f : 1.0f;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = fminf(fmaxf(f[i] / s, -448.0f), 448.0f);
  const uint32_t lo = a8_pack4(q[0], q[1], q[2], q[3]);
  const uint32_t hi = a8_pack4(q[4], q[5], q[6], q[7]);
  if (live) {
    *reinterpret_cast<u32x2*>(a.q + row * a.C + b * 128 + sub * 8) = u32x2{lo, hi};
    if (sub == 0) a.s[row * nb + b] = s;
  }
}

hipError_t launch_quant_1x128(const QuantArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int64_t threads = a.rows * (a.C / 128) * 16;
  hipLaunchKernelGGL(quant_1x128_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// XL (down projection, single-tile passes, K range of at most kA8XlSteps
// steps): the tile's activation codes and scales for the whole K range are
// staged once into LDS, in the lane order the MFMA reads them, and shared by
// the four waves and every output block the workgroup walks; the loads then
// carry weights only.
constexpr int kA8XlSteps = 16;

template <int MODE, int MT, bool PACKED, bool XL>
__device__ __forceinline__ void ffn_a8_body(const A8Args& a, int g, bool big_class) {
  constexpr bool GU = MODE == MODE_GATEUP;
  static_assert(!XL || (MT == 1 && !GU), "LDS-staged activations: single-tile down projection");
  __shared__ __attribute__((aligned(16))) u32x4 xl_s[XL ? kA8XlSteps * 64 * 2 : 1];   // [step][lane][2]
  __shared__ float sxl_s[XL ? kA8XlSteps * 16 : 1];                                   // [step][row]
  // register stages (NB - 1 steps in flight), as many as the registers allow
  constexpr int NB = MT == 1 ? (GU ? 4 : 8) : 3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: weight scales load as scalars
  const bool shared = g == a.E_phys;
  int64_t s0 = 0, s1 = 0;
  int c0 = 0, c1 = 0;
  if (shared) { s0 = a.shared_base; c0 = a.T; }
  else if (a.layout == MOE_MASKED) {
    const int mm = a.masked_m[g];
    s0 = (int64_t)g * a.M_max; c0 = mm;
    s1 = (int64_t)a.E_phys * a.M_max + a.spill_off[g]; c1 = a.counts[g] - mm;
  } else {
    s0 = a.pad_off[g]; c0 = a.counts[g];
  }
  const int R = c0 + c1;
  if (R <= 0 || (big_class ? R <= 16 : R > 16)) return;   // the other class's group
  const int N = a.N, Kdim = a.Kdim;
  const int nkb = Kdim / 128;
  const int kper = nkb / a.ksplit;
  const int kb0 = blockIdx.z * kper;
  // the workgroup owns a.nblk consecutive 64-row blocks; this wave's 16
  // weight rows in block j start at n0(j)
  const int nblk = a.nblk;
  auto n0_of = [&](int j) { return (blockIdx.x * nblk + j) * 64 + 16 * wave; };
  const int lr = lane & 15, lg = lane >> 4;
  const uint8_t* Wa = shared ? a.SW : a.W + (int64_t)g * N * Kdim;
  const uint8_t* Wb = GU ? (shared ? a.SW3 : a.W3 + (int64_t)g * N * Kdim) : nullptr;
  const float* Sa0 = shared ? a.SS : a.S + (int64_t)g * (N / 128) * nkb;
  const float* Sb0 = GU ? (shared ? a.SS3 : a.S3 + (int64_t)g * (N / 128) * nkb) : nullptr;
  // byte offset of this lane's 16-byte weight piece `instr` of K step kb, block j
  auto woff = [&](int j, int kb, int instr) -> int64_t {
    const int n0 = n0_of(j);
    if (PACKED) return ((int64_t)kb * (N / 16) + n0 / 16) * 2048 + instr * 1024 + lane * 16;
    return (int64_t)(n0 + lr) * Kdim + kb * 128 + 64 * instr + 16 * lg;
  };
  auto srow_w = [&](int j) { return (int64_t)(n0_of(j) / 128) * nkb; };
  const int ntiles = (R + 15) / 16;
  for (int t0 = 0; t0 < ntiles; t0 += MT) {
    const uint8_t* xrow[MT];
    const float* srow[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int gr = (t0 + i) * 16 + lr;
      const int rank = gr < R ? gr : 0;              // rows past the group read a valid row
      int64_t row;
      if (a.gather_src) row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
      else row = rank < c0 ? s0 + rank : s1 + (rank - c0);
      xrow[i] = a.X + row * a.ldx + 16 * lg;
      srow[i] = a.XS + row * nkb;
    }
    u32x4 wr[NB][2], w3r[NB][2], xr[NB][MT][2];
    float sx[NB][MT], swa[NB], swb[NB];
    int kbk[NB];   // XL: the bank's K step
    auto load = [&](int bank, int jw, int kb) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        wr[bank][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wa + woff(jw, kb, j)));
        if constexpr (GU)
          w3r[bank][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wb + woff(jw, kb, j)));
      }
      if constexpr (XL) {
        kbk[bank] = kb - kb0;
      } else {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          xr[bank][i][0] = *reinterpret_cast<const u32x4*>(xrow[i] + kb * 128);
          xr[bank][i][1] = *reinterpret_cast<const u32x4*>(xrow[i] + kb * 128 + 64);
          sx[bank][i] = srow[i][kb];
        }
      }
      swa[bank] = Sa0[srow_w(jw) + kb];
      if constexpr (GU) swb[bank] = Sb0[srow_w(jw) + kb];
    };
    f32x4 acc[MT], acc3[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) { acc[i] = f32x4{0, 0, 0, 0}; acc3[i] = f32x4{0, 0, 0, 0}; }
    auto compute = [&](int bank, bool valid) {
      const v8i w = __builtin_bit_cast(v8i, u32x8{wr[bank][0].x, wr[bank][0].y, wr[bank][0].z, wr[bank][0].w,
                                                  wr[bank][1].x, wr[bank][1].y, wr[bank][1].z, wr[bank][1].w});
      v8i w3 = w;
      if constexpr (GU)
        w3 = __builtin_bit_cast(v8i, u32x8{w3r[bank][0].x, w3r[bank][0].y, w3r[bank][0].z, w3r[bank][0].w,
                                           w3r[bank][1].x, w3r[bank][1].y, w3r[bank][1].z, w3r[bank][1].w});
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        u32x4 x0, x1;
        float sxi;
        if constexpr (XL) {
          x0 = xl_s[(kbk[bank] * 64 + lane) * 2];
          x1 = xl_s[(kbk[bank] * 64 + lane) * 2 + 1];
          sxi = sxl_s[kbk[bank] * 16 + lr];
        } else {
          x0 = xr[bank][i][0];
          x1 = xr[bank][i][1];
          sxi = sx[bank][i];
        }
        const v8i x = __builtin_bit_cast(v8i, u32x8{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w});
        const f32x4 zero = {0, 0, 0, 0};
        const f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, zero, 0, 0, 0, 127, 0, 127);
        // padding steps (past the K range) add d * 0
        const float sc = valid ? swa[bank] * sxi : 0.0f;
        acc[i] += d * sc;
        if constexpr (GU) {
          const f32x4 d3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w3, x, zero, 0, 0, 0, 127, 0, 127);
          acc3[i] += d3 * (valid ? swb[bank] * sxi : 0.0f);
        }
      }
    };
    // acc[i] holds D[w-row 4*lg + j][token lr of tile i] of block jo
    auto epilogue = [&](int jo) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int gr = (t0 + i) * 16 + lr;
        if (gr < R) {
          const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
          const int col = n0_of(jo) + 4 * lg;
          if constexpr (GU) {
            const f32x4 gt = acc[i], up = acc3[i];
            const u32x2 o = {pack_bf16x2(a8_silu(gt.x) * up.x, a8_silu(gt.y) * up.y),
                             pack_bf16x2(a8_silu(gt.z) * up.z, a8_silu(gt.w) * up.w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + col) = o;
          } else if (a.out_f32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + blockIdx.z * a.split_stride + row * a.ldo + col) =
                acc[i];
          } else {
            const u32x2 o = {pack_bf16x2(acc[i].x, acc[i].y), pack_bf16x2(acc[i].z, acc[i].w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + col) = o;
          }
        }
        acc[i] = f32x4{0, 0, 0, 0};
        acc3[i] = f32x4{0, 0, 0, 0};
      }
    };
    // Single-tile passes walk the workgroup's blocks as one stream of
    // nblk * kper steps (loads run NB - 1 steps ahead across block
    // boundaries); multi-tile passes run one stream per block.  The step
    // count of a stream is padded to whole passes of NB so that the loop
    // body has no branches around loads (a guarded step makes the compiler
    // wait for every outstanding load); loads past the end re-read the last
    // step, and padding steps add d * 0.
    const int span = MT == 1 ? nblk : 1;
    const int vsteps = span * kper;
    const int npad = (vsteps + NB - 1) / NB * NB;
    // XL: piece p = (s * 64 + l) * 2 + j of the LDS tile is the 16 bytes j of
    // K step s lane l reads (row l % 16, K bytes 16 (l / 16) + 64 j); thread
    // t moves pieces t + 256 i.  Issued before the first weights, so the
    // wait for them leaves the weight loads in flight.
    u32x4 xst[XL ? 8 : 1];
    float sxst = 0.f;
    if constexpr (XL) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pc = tid + 256 * i, st = pc >> 7, l = (pc >> 1) & 63, j = pc & 1;
        const int gr = t0 * 16 + (l & 15);
        const int rank = gr < R ? gr : 0;
        const int64_t row = rank < c0 ? s0 + rank : s1 + (rank - c0);
        const int k = kb0 + (st < kper ? st : 0);
        xst[i] = *reinterpret_cast<const u32x4*>(a.X + row * a.ldx + k * 128 + 16 * (l >> 4) + 64 * j);
      }
      {
        const int st = tid >> 4, r = tid & 15;
        const int gr = t0 * 16 + r;
        const int rank = gr < R ? gr : 0;
        const int64_t row = rank < c0 ? s0 + rank : s1 + (rank - c0);
        sxst = a.XS[row * nkb + kb0 + (st < kper ? st : 0)];
      }
    }
    for (int jb = 0; jb < nblk; jb += span) {
      auto load_v = [&](int bank, int v) {
        const int vc = min(v, vsteps - 1);
        load(bank, jb + vc / kper, kb0 + vc % kper);
      };
#pragma unroll
      for (int p = 0; p < NB - 1; ++p) load_v(p, p);
      if constexpr (XL) {
        if (jb == 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (((tid + 256 * i) >> 7) < kper) xl_s[tid + 256 * i] = xst[i];
          if ((tid >> 4) < kper) sxl_s[tid] = sxst;
          __syncthreads();
        }
      }
      int cj = jb, ck = 0;   // block and step being multiplied
      for (int sb = 0; sb < npad; sb += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int st = sb + u;
          load_v((u + NB - 1) % NB, st + NB - 1);
          // (fences keep each step's loads in their step: hoisted together the
          // loads of a pass serialise the pipeline)
          __builtin_amdgcn_sched_barrier(0);
          compute(u, st < vsteps);
          __builtin_amdgcn_sched_barrier(0);
          if (st < vsteps && ++ck == kper) {
            epilogue(cj);
            ck = 0;
            ++cj;
          }
        }
      }
    }
    if constexpr (XL) __syncthreads();   // the LDS tile is restaged by the next pass
  }
}

// One launch: groups of up to 16 rows take one tile per pass (the deeper
// load pipeline), larger ones four; the large-group workgroups come first in
// the grid (grid.y row 0 .. n_big-1 re-reads group ids from the top) so that
// their longer streams start early.  BIG = false: every group takes the
// one-tile path (T <= 16, no group can be larger).
// XL: the single-tile class of the down projection stages its activations
// in LDS (K range of at most kA8XlSteps steps).
template <int MODE, bool PACKED, bool BIG, bool XL>
__global__ __launch_bounds__(256) void ffn_a8_kernel(A8Args a) {
  if constexpr (BIG) {
    const int groups = a.E_phys + a.n_shared;
    if ((int)blockIdx.y < groups) { ffn_a8_body<MODE, 4, PACKED, false>(a, blockIdx.y, true); return; }
    ffn_a8_body<MODE, 1, PACKED, XL>(a, blockIdx.y - groups, false);
  } else {
    ffn_a8_body<MODE, 1, PACKED, XL>(a, blockIdx.y, false);
  }
}

template <int MODE, bool BIG>
static void launch_a8_big(const A8Args& a, int packed, dim3 grid, hipStream_t s) {
  constexpr bool kXl = MODE == MODE_DOWN;
  const bool xl = kXl && a.Kdim / 128 / a.ksplit <= kA8XlSteps;
  if (xl) {
    if (packed) hipLaunchKernelGGL((ffn_a8_kernel<MODE, true, BIG, kXl>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ffn_a8_kernel<MODE, false, BIG, kXl>), grid, dim3(256), 0, s, a);
  } else {
    if (packed) hipLaunchKernelGGL((ffn_a8_kernel<MODE, true, BIG, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ffn_a8_kernel<MODE, false, BIG, false>), grid, dim3(256), 0, s, a);
  }
}

hipError_t launch_ffn_a8(const A8Args& a, int packed, int mode, hipStream_t s) {
  if (a.N % 64 || a.Kdim % 128 || (a.Kdim / 128) % a.ksplit) return hipErrorInvalidValue;
  const int groups = a.E_phys + a.n_shared;
  const bool big = a.T > 16;
  if (a.nblk < 1 || a.nblk > 8 || (a.N / 64) % a.nblk) return hipErrorInvalidValue;
  const dim3 grid(a.N / (64 * a.nblk), big ? 2 * groups : groups, a.ksplit);
  if (mode == MODE_GATEUP) {
    if (big) launch_a8_big<MODE_GATEUP, true>(a, packed, grid, s);
    else launch_a8_big<MODE_GATEUP, false>(a, packed, grid, s);
  } else {
    if (big) launch_a8_big<MODE_DOWN, true>(a, packed, grid, s);
    else launch_a8_big<MODE_DOWN, false>(a, packed, grid, s);
  }
  return hipGetLastError();
}

}  // namespace moe
