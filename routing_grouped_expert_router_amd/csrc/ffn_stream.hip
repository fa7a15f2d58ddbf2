// Streaming grouped GEMM for decode-sized groups on gfx950 (CDNA4).
//
// One workgroup (4 waves) owns 64 output features (weight rows) of one group
// (a physical expert slot, the shared expert, or the router) and all of that
// group's token rows.  Decode moves far more weight bytes than activation
// bytes ("推理 INFRA 方法论(5)": the weight traffic is
// [C(B) W_routed + W_shared] * bpp), so the design streams every weight byte
// from HBM exactly once, straight into registers in the MFMA operand layout,
// and keeps the small activation tile in LDS where the four waves share it.
//
//  * Weights W [N, Kdim] (row = output feature, K contiguous).  Lane l of a
//    wave loads row n0 + l%16; the four lane groups l/16 take consecutive
//    16-byte pieces, so each load instruction reads 64 contiguous bytes of
//    16 rows.  The next 128-wide K step is loaded while the current one is
//    multiplied.
//  * Activations X [rows, Kdim] bf16: the group's row tiles (16 rows each,
//    up to MT tiles per pass) are staged per K step in a double-buffered LDS
//    tile and read as the MFMA B operand.
//  * v_mfma_f32_16x16x32_bf16 computes D[n, m] = sum_k W[n, k] X[m, k].
//  * Masked layout ("推理 INFRA 方法论(5)", DeepGEMM section): the valid rows of
//    slot p are masked_m[p] rows at p*M_max, plus any spill rows; row tiles
//    that hold no valid row are never formed, so a slot without tokens
//    issues no weight load and no MFMA.
//  * fp8 weights (OCP E4M3FN + one fp32 scale per 128x128 block): 16 bytes
//    become two bf16x8 operands by an exact conversion; the four MFMAs of a
//    128-wide K block start from zero and their sum is scaled and added to an
//    fp32 accumulator (the same page's two-level accumulation: promote every
//    128 K with the block scale).
//  * MODE_GATEUP: both W1 (gate) and W3 (up); epilogue h = SiLU(g) * u in
//    bf16.  MODE_DOWN: W2; bf16 output, or fp32 partials when K is split
//    over grid.z.  MODE_ROUTER: router weight [E, H], fp32 logits + bias.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kThreads = 256;      // 4 waves
constexpr int kBN = 64;            // weight rows per workgroup
constexpr int kKS = 128;           // K per pipeline step
constexpr int kLdsStride = kKS + 8;  // bf16 elements per LDS row (pad vs bank conflicts)

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <bool FP8>
struct WFrag {
  // bf16: 4 x 16 B per 128 K (K offsets 32j + 8*lg); fp8: 2 x 16 B (64i + 16*lg)
  static constexpr int N = FP8 ? 2 : 4;
  u32x4 v[N];
};

template <bool FP8>
__device__ __forceinline__ void load_w(WFrag<FP8>& f, const void* wrow, int k0, int lg, bool ok) {
  if (FP8) {
    const uint8_t* p = static_cast<const uint8_t*>(wrow) + k0 + 16 * lg;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      f.v[i] = ok ? *reinterpret_cast<const u32x4*>(p + 64 * i) : u32x4{0, 0, 0, 0};
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(wrow) + k0 + 8 * lg;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.v[j] = ok ? *reinterpret_cast<const u32x4*>(p + 32 * j) : u32x4{0, 0, 0, 0};
  }
}

template <int MT>
struct Pass {
  int64_t start[MT];
  int valid[MT];
  int n;   // tiles in this pass
};

// one 16-row tile index -> (first row, valid rows) over the two segments
__device__ __forceinline__ void tile_rows(int tile, int64_t s0, int c0, int nt0, int64_t s1, int c1,
                                          int64_t& start, int& valid) {
  if (tile < nt0) { start = s0 + 16 * tile; valid = min(16, c0 - 16 * tile); }
  else { const int u = tile - nt0; start = s1 + 16 * u; valid = min(16, c1 - 16 * u); }
}

template <bool FP8, int MODE, int MT>
__global__ __launch_bounds__(kThreads) void ffn_stream_kernel(StreamArgs a) {
  constexpr bool TWO = MODE == MODE_GATEUP;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT * 16][kLdsStride];

  const int g = blockIdx.y;
  const int ks = blockIdx.z % a.ksplit;
  const int mc = blockIdx.z / a.ksplit;
  // ---- the group's row segments
  int64_t s0 = 0, s1 = 0;
  int c0 = 0, c1 = 0;
  const bool shared = (MODE != MODE_ROUTER) && g == a.E_phys;
  if (MODE == MODE_ROUTER) { c0 = a.T; }
  else if (shared) { s0 = a.shared_base; c0 = a.T; }
  else if (a.layout == MOE_MASKED) {
    const int mm = a.masked_m[g];
    s0 = (int64_t)g * a.M_max; c0 = mm;
    s1 = (int64_t)a.E_phys * a.M_max + a.spill_off[g]; c1 = a.counts[g] - mm;
  } else {
    s0 = a.pad_off[g]; c0 = a.counts[g];
  }
  const int nt0 = (c0 + 15) >> 4, nt1 = (c1 + 15) >> 4, ntiles = nt0 + nt1;
  if (ntiles == 0) return;   // no token: no weight load, no MFMA

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n_w0 = blockIdx.x * kBN + wave * 16;   // first weight row of this wave
  const int nrow = n_w0 + lr;
  const bool nok = nrow < a.N;
  const int Kdim = a.Kdim;
  const int kb_per_row = Kdim / kKS;

  // ---- weights of this group
  const size_t wbytes = FP8 ? 1 : 2;
  const void* Wg;
  const void* W3g = nullptr;
  const float* Sg = nullptr;
  const float* S3g = nullptr;
  if (shared) {
    Wg = a.SW; W3g = a.SW3; Sg = a.SS; S3g = a.SS3;
  } else {
    const int64_t gi = (MODE == MODE_ROUTER) ? 0 : g;
    Wg = static_cast<const char*>(a.W) + gi * (int64_t)a.N * Kdim * wbytes;
    if (TWO) W3g = static_cast<const char*>(a.W3) + gi * (int64_t)a.N * Kdim * wbytes;
    if (FP8) {
      Sg = a.S + gi * (int64_t)(a.N / 128) * kb_per_row;
      if (TWO) S3g = a.S3 + gi * (int64_t)(a.N / 128) * kb_per_row;
    }
  }
  const void* wrow = static_cast<const char*>(Wg) + (int64_t)(nok ? nrow : 0) * Kdim * wbytes;
  const void* w3row = TWO ? static_cast<const char*>(W3g) + (int64_t)nrow * Kdim * wbytes : nullptr;
  const int sb_row = (n_w0 / 128) * kb_per_row;    // scale row of this wave's 16 rows

  // ---- K range of this split
  const int steps_all = kb_per_row;
  const int steps = steps_all / a.ksplit;
  const int kstep0 = ks * steps;

  // staging assignment: thread -> (row r of a 16-row tile, 16-byte chunk c)
  const int sr = tid >> 4, sc = tid & 15;

  for (int tile0 = mc * MT; tile0 < ntiles; tile0 += a.mchunks * MT) {
    Pass<MT> ps;
    ps.n = min(MT, ntiles - tile0);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      ps.start[m] = 0; ps.valid[m] = 0;
      if (m < ps.n) tile_rows(tile0 + m, s0, c0, nt0, s1, c1, ps.start[m], ps.valid[m]);
    }

    auto load_x = [&](int kstep, u32x4* xr) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        xr[m] = u32x4{0, 0, 0, 0};
        if (m < ps.n && sr < ps.valid[m]) {
          const uint16_t* src = a.X + (ps.start[m] + sr) * a.ldx + (int64_t)kstep * kKS + 8 * sc;
          xr[m] = *reinterpret_cast<const u32x4*>(src);
        }
      }
    };
    auto store_x = [&](int buf, const u32x4* xr) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        *reinterpret_cast<u32x4*>(&xs[buf][m * 16 + sr][8 * sc]) = xr[m];
    };

    f32x4 acc[MT], acc3[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) { acc[m] = f32x4{0, 0, 0, 0}; acc3[m] = f32x4{0, 0, 0, 0}; }

    WFrag<FP8> wa, wb;
    load_w<FP8>(wa, wrow, kstep0 * kKS, lg, nok);
    if (TWO) load_w<FP8>(wb, w3row, kstep0 * kKS, lg, true);
    {
      u32x4 xr[MT];
      load_x(kstep0, xr);
      store_x(0, xr);
    }
    __syncthreads();

    for (int s = 0; s < steps; ++s) {
      const int buf = s & 1;
      const bool more = s + 1 < steps;
      WFrag<FP8> na, nb;
      u32x4 xr[MT];
      if (more) {
        load_w<FP8>(na, wrow, (kstep0 + s + 1) * kKS, lg, nok);
        if (TWO) load_w<FP8>(nb, w3row, (kstep0 + s + 1) * kKS, lg, true);
        load_x(kstep0 + s + 1, xr);
      }
      if (FP8) {
        float sc1 = Sg[sb_row + kstep0 + s];
        float sc3 = TWO ? S3g[sb_row + kstep0 + s] : 0.f;
        bf16x8 a1[4], a3[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          fp8x16_to_bf16(wa.v[i], a1[2 * i], a1[2 * i + 1]);
          if (TWO) fp8x16_to_bf16(wb.v[i], a3[2 * i], a3[2 * i + 1]);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < ps.n) {
            f32x4 p1 = {0, 0, 0, 0}, p3 = {0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              // operand q covers K offsets 64*(q/2) + 16*lg + 8*(q%2) .. +8
              const bf16x8 b = *reinterpret_cast<const bf16x8*>(
                  &xs[buf][m * 16 + lr][64 * (q >> 1) + 16 * lg + 8 * (q & 1)]);
              p1 = mfma16x16x32(a1[q], b, p1);
              if (TWO) p3 = mfma16x16x32(a3[q], b, p3);
            }
            acc[m] += p1 * sc1;
            if (TWO) acc3[m] += p3 * sc3;
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < ps.n) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x8 b = *reinterpret_cast<const bf16x8*>(&xs[buf][m * 16 + lr][32 * j + 8 * lg]);
              acc[m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wa.v[j]), b, acc[m]);
              if (TWO) acc3[m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wb.v[j]), b, acc3[m]);
            }
          }
        }
      }
      if (more) store_x(buf ^ 1, xr);
      __syncthreads();
      if (more) { wa = na; if (TWO) wb = nb; }
    }

    // ---- epilogue: lane holds D[n = n_w0 + 4*lg + j][m = lr], j = 0..3
    const int ncol = n_w0 + 4 * lg;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < ps.n && lr < ps.valid[m]) {
        const int64_t row = ps.start[m] + lr;
        if (MODE == MODE_GATEUP) {
          const f32x4 gt = acc[m], up = acc3[m];
          u32x2 o = {pack_bf16x2(silu(gt.x) * up.x, silu(gt.y) * up.y),
                     pack_bf16x2(silu(gt.z) * up.z, silu(gt.w) * up.w)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
        } else if (MODE == MODE_DOWN) {
          if (a.out_f32) {
            float* o = static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol;
            *reinterpret_cast<f32x4*>(o) = acc[m];
          } else {
            u32x2 o = {pack_bf16x2(acc[m].x, acc[m].y), pack_bf16x2(acc[m].z, acc[m].w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
          }
        } else {
          float* o = static_cast<float*>(a.out) + row * a.ldo;
          const float v[4] = {acc[m].x, acc[m].y, acc[m].z, acc[m].w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (ncol + j < a.N) o[ncol + j] = v[j] + (a.bias ? a.bias[ncol + j] : 0.f);
        }
      }
    }
  }
}

template <bool FP8, int MODE>
static hipError_t launch_mt(const StreamArgs& a, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 1>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 2>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 4>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ffn_stream(const StreamArgs& a, int fp8, int mode, int mt, dim3 grid, hipStream_t s) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (mode == MODE_GATEUP) return fp8 ? launch_mt<true, MODE_GATEUP>(a, mt, grid, s)
                                      : launch_mt<false, MODE_GATEUP>(a, mt, grid, s);
  if (mode == MODE_DOWN) return fp8 ? launch_mt<true, MODE_DOWN>(a, mt, grid, s)
                                    : launch_mt<false, MODE_DOWN>(a, mt, grid, s);
  if (mode == MODE_ROUTER && !fp8) return launch_mt<false, MODE_ROUTER>(a, mt, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
