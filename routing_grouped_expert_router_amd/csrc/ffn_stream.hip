// Streaming grouped GEMM for decode-sized expert groups on gfx950 (CDNA4).
//
// One workgroup (4 waves) owns 64 output features (weight rows) of one group
// (a physical expert slot or the shared expert) and all of that group's
// token rows.  Decode moves far more weight bytes than activation bytes
// ("推理 INFRA 方法论(5)", C(B) section: the weight traffic is
// [C(B) W_routed + W_shared] * bpp), so every weight byte is streamed from
// HBM exactly once, straight into registers in the MFMA operand layout, while
// the small activation tile sits in LDS where the four waves share it.
//
//  * Weights, per 16-row panel and 128-wide K step, are read by one wave as
//    NI 16-byte loads per lane (bf16: NI = 4, fp8: NI = 2).  In the packed
//    layout (moe_pack_weights) each load instruction reads 1 KiB of
//    contiguous memory and a panel is one contiguous stream; in the row-major
//    [out, in] layout each instruction reads 64 bytes of 16 rows.  Two K steps
//    are in flight while the current one is multiplied (three register
//    buffers in rotation).
//  * Activations X [rows, Kdim] bf16: with one 16-row tile per pass (MT = 1,
//    the common decode case) each lane loads its row's fragments straight
//    into registers two K steps ahead and the waves never synchronise; with
//    MT > 1 the group's row tiles are staged per K step in a double-buffered
//    LDS tile shared by the four waves.
//  * v_mfma_f32_16x16x32_bf16 computes D[n, m] = sum_k W[n, k] X[m, k]; lane l
//    supplies weight row l % 16 and activation row l % 16 with the K values
//    of lane group l / 16, and receives D rows 4*(l/16)+0..3 of column l % 16.
//  * Masked layout ("推理 INFRA 方法论(5)", DeepGEMM section): the valid rows
//    of slot p are masked_m[p] rows at p*M_max, plus any spill rows; a row
//    tile with no valid row is never formed, so a slot without tokens issues
//    no weight load and no MFMA.
//  * fp8 weights (OCP E4M3FN + one fp32 scale per 128x128 block): 16 bytes
//    become two bf16x8 operands by an exact conversion; the four MFMAs of a
//    128-wide K block start from zero and their sum is scaled into an fp32
//    accumulator (the same section's two-level accumulation: promote every
//    128 K with the block scale).
//  * MODE_GATEUP: W1 (gate) and W3 (up); epilogue h = SiLU(g) * u in bf16.
//    MODE_DOWN: W2; bf16 output, or fp32 partial planes when K is split over
//    grid.z (summed in split order by the combine).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kThreads = 256;        // 4 waves
constexpr int kBN = 64;              // weight rows per workgroup
constexpr int kKS = 128;             // K per pipeline step
constexpr int kLdsStride = kKS + 8;  // bf16 elements per LDS row (pad vs bank conflicts)

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <bool FP8>
struct WFrag {
  static constexpr int NI = FP8 ? 2 : 4;
  u32x4 v[NI];
};

// Byte addressing of one wave's weight stream:
//   address(kstep, i) = base + kstep * step_bytes + i * instr_bytes + lane_bytes
struct WStream {
  const char* base;
  int step_bytes, instr_bytes, lane_bytes;
};

// Weights are read once per call and never again by this kernel, so the
// loads are non-temporal: streamed past the caches instead of evicting the
// activations and routing tables other workgroups still read.
template <bool FP8>
__device__ __forceinline__ void load_w(WFrag<FP8>& f, const WStream& w, int kstep) {
  const char* p = w.base + (int64_t)kstep * w.step_bytes + w.lane_bytes;
#pragma unroll
  for (int i = 0; i < WFrag<FP8>::NI; ++i)
    f.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i * w.instr_bytes));
}

template <bool FP8, bool PACKED>
__device__ __forceinline__ WStream make_stream(const void* Wg, int n_w0, int lane, int N, int Kdim) {
  constexpr int wbytes = FP8 ? 1 : 2;
  WStream s;
  if (PACKED) {
    // K step s of panel n_w0/16 is the 16x128 block (s, panel) of the
    // step-major packed matrix
    s.base = static_cast<const char*>(Wg) + (int64_t)(n_w0 / 16) * 16 * kKS * wbytes;
    s.step_bytes = (N / 16) * 16 * kKS * wbytes;
    s.instr_bytes = 1024;
    s.lane_bytes = 16 * lane;
  } else {
    s.base = static_cast<const char*>(Wg) + (int64_t)(n_w0 + (lane & 15)) * Kdim * wbytes;
    s.step_bytes = kKS * wbytes;
    s.instr_bytes = 64;
    s.lane_bytes = 16 * (lane >> 4);
  }
  return s;
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

template <bool FP8, int MODE, int MT, bool PACKED, bool XDIRECT>
__global__ __launch_bounds__(kThreads) void ffn_stream_kernel(StreamArgs a) {
  constexpr bool TWO = MODE == MODE_GATEUP;
  static_assert(!XDIRECT || MT == 1, "register-staged activations hold one row tile");
  __shared__ __attribute__((aligned(16))) uint16_t xs[XDIRECT ? 1 : 2][XDIRECT ? 1 : MT * 16][kLdsStride];

  const int g = blockIdx.y;
  const int ks = blockIdx.z % a.ksplit;
  const int mc = blockIdx.z / a.ksplit;
  // ---- the group's row segments
  int64_t s0 = 0, s1 = 0;
  int c0 = 0, c1 = 0;
  const bool shared = g == a.E_phys;
  if (shared) { s0 = a.shared_base; c0 = a.T; }
  else if (a.layout == MOE_MASKED) {
    const int mm = a.masked_m[g];
    s0 = (int64_t)g * a.M_max; c0 = mm;
    s1 = (int64_t)a.E_phys * a.M_max + a.spill_off[g]; c1 = a.counts[g] - mm;
  } else {
    s0 = a.pad_off[g]; c0 = a.counts[g];
  }
  const int nt0 = (c0 + 15) >> 4, nt1 = (c1 + 15) >> 4, ntiles = nt0 + nt1;
  if (ntiles == 0) return;   // no token: no weight load, no MFMA
  // size classes: another launch owns groups outside (min_rows, max_rows]
  if (c0 + c1 <= a.min_rows || (a.max_rows > 0 && c0 + c1 > a.max_rows)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n_w0 = blockIdx.x * kBN + wave * 16;   // first weight row of this wave
  const int Kdim = a.Kdim;
  const int kb_per_row = Kdim / kKS;

  // ---- weights of this group
  constexpr int wbytes = FP8 ? 1 : 2;
  const void* Wg;
  const void* W3g = nullptr;
  const float* Sg = nullptr;
  const float* S3g = nullptr;
  if (shared) {
    Wg = a.SW; W3g = a.SW3; Sg = a.SS; S3g = a.SS3;
  } else {
    Wg = static_cast<const char*>(a.W) + (int64_t)g * a.N * Kdim * wbytes;
    if (TWO) W3g = static_cast<const char*>(a.W3) + (int64_t)g * a.N * Kdim * wbytes;
    if (FP8) {
      Sg = a.S + (int64_t)g * (a.N / 128) * kb_per_row;
      if (TWO) S3g = a.S3 + (int64_t)g * (a.N / 128) * kb_per_row;
    }
  }
  const WStream w1s = make_stream<FP8, PACKED>(Wg, n_w0, lane, a.N, Kdim);
  const WStream w3s = TWO ? make_stream<FP8, PACKED>(W3g, n_w0, lane, a.N, Kdim) : w1s;
  const int sb_row = (n_w0 / 128) * kb_per_row;    // scale row of this wave's 16 rows

  // ---- K range of this split
  const int steps = kb_per_row / a.ksplit;
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

    if constexpr (XDIRECT) {
      // One 16-row tile; each lane streams its own activation row (clamped
      // into the valid rows) straight into registers, two K steps ahead like
      // the weights.  Waves never synchronise.
      const uint16_t* xrow = a.X + (ps.start[0] + min(lr, ps.valid[0] - 1)) * a.ldx;
      auto xoff = [&](int q) { return FP8 ? 64 * (q >> 1) + 16 * lg + 8 * (q & 1) : 32 * q + 8 * lg; };
      auto load_xd = [&](u32x4* v, int kstep) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = *reinterpret_cast<const u32x4*>(xrow + (int64_t)kstep * kKS + xoff(q));
      };
      f32x4 acc1 = {0, 0, 0, 0}, acc3d = {0, 0, 0, 0};
      const int klast = kstep0 + steps - 1;
      WFrag<FP8> w1b[3], w3b[3];
      u32x4 xb[3][4];
      load_xd(xb[0], kstep0);
      load_w<FP8>(w1b[0], w1s, kstep0);
      if (TWO) load_w<FP8>(w3b[0], w3s, kstep0);
      load_xd(xb[1], min(kstep0 + 1, klast));
      load_w<FP8>(w1b[1], w1s, min(kstep0 + 1, klast));
      if (TWO) load_w<FP8>(w3b[1], w3s, min(kstep0 + 1, klast));
      for (int s0 = 0; s0 < steps; s0 += 3) {
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const int s = s0 + u;
          if (s < steps) {
            load_xd(xb[(u + 2) % 3], min(kstep0 + s + 2, klast));
            load_w<FP8>(w1b[(u + 2) % 3], w1s, min(kstep0 + s + 2, klast));
            if (TWO) load_w<FP8>(w3b[(u + 2) % 3], w3s, min(kstep0 + s + 2, klast));
            if (FP8) {
              const float sc1 = Sg[sb_row + kstep0 + s];
              const float sc3 = TWO ? S3g[sb_row + kstep0 + s] : 0.f;
              bf16x8 a1[4], a3[4];
#pragma unroll
              for (int i = 0; i < 2; ++i) {
                fp8x16_to_bf16(w1b[u].v[i], a1[2 * i], a1[2 * i + 1]);
                if (TWO) fp8x16_to_bf16(w3b[u].v[i], a3[2 * i], a3[2 * i + 1]);
              }
              f32x4 p1 = {0, 0, 0, 0}, p3 = {0, 0, 0, 0};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, xb[u][q]);
                p1 = mfma16x16x32(a1[q], b, p1);
                if (TWO) p3 = mfma16x16x32(a3[q], b, p3);
              }
              acc1 += p1 * sc1;
              if (TWO) acc3d += p3 * sc3;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, xb[u][q]);
                acc1 = mfma16x16x32(__builtin_bit_cast(bf16x8, w1b[u].v[q]), b, acc1);
                if (TWO) acc3d = mfma16x16x32(__builtin_bit_cast(bf16x8, w3b[u].v[q]), b, acc3d);
              }
            }
          }
        }
      }
      const int ncol = n_w0 + 4 * lg;
      if (lr < ps.valid[0]) {
        const int64_t row = ps.start[0] + lr;
        if (MODE == MODE_GATEUP) {
          u32x2 o = {pack_bf16x2(silu(acc1.x) * acc3d.x, silu(acc1.y) * acc3d.y),
                     pack_bf16x2(silu(acc1.z) * acc3d.z, silu(acc1.w) * acc3d.w)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
        } else if (a.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol) = acc1;
        } else {
          u32x2 o = {pack_bf16x2(acc1.x, acc1.y), pack_bf16x2(acc1.z, acc1.w)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
        }
      }
      continue;
    }

    // Activation rows, clamped into the tile's valid rows (rows past the valid
    // count only feed MFMA columns that are never stored).  The loads sit
    // outside any divergent branch so the compiler never waits on them early.
    const uint16_t* xsrc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int64_t row = (m < ps.n && ps.valid[m] > 0) ? ps.start[m] + min(sr, ps.valid[m] - 1) : s0;
      xsrc[m] = a.X + row * a.ldx + 8 * sc;
    }
    auto load_x = [&](int kstep, u32x4* xr) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        xr[m] = *reinterpret_cast<const u32x4*>(xsrc[m] + (int64_t)kstep * kKS);
    };
    auto store_x = [&](int buf, const u32x4* xr) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        *reinterpret_cast<u32x4*>(&xs[buf][m * 16 + sr][8 * sc]) = xr[m];
    };

    f32x4 acc[MT], acc3[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) { acc[m] = f32x4{0, 0, 0, 0}; acc3[m] = f32x4{0, 0, 0, 0}; }

    // one K step: multiply the weights in (wa, wb) with the staged tile
    auto compute = [&](const WFrag<FP8>& wa, const WFrag<FP8>& wb, int buf, int kstep) {
      if (FP8) {
        const float sc1 = Sg[sb_row + kstep];
        const float sc3 = TWO ? S3g[sb_row + kstep] : 0.f;
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
    };

    // Pipeline: at step s the weights of steps s+1, s+2 and the activations of
    // step s+2 are in flight while step s is multiplied and the (already
    // arrived) activations of step s+1 are staged.  Loads are issued
    // activations-first: vector-memory counters drain in order, so waiting for
    // an activation tile never waits for weights issued after it.  Steps past
    // the end re-load the last K block (clamped) instead of branching around
    // the loads; that data is never multiplied.
    const int klast = kstep0 + steps - 1;
    WFrag<FP8> w1b[3], w3b[3];
    u32x4 xb[3][MT];
    load_x(kstep0, xb[0]);
    load_w<FP8>(w1b[0], w1s, kstep0);
    if (TWO) load_w<FP8>(w3b[0], w3s, kstep0);
    load_x(min(kstep0 + 1, klast), xb[1]);
    load_w<FP8>(w1b[1], w1s, min(kstep0 + 1, klast));
    if (TWO) load_w<FP8>(w3b[1], w3s, min(kstep0 + 1, klast));
    store_x(0, xb[0]);
    __syncthreads();

    for (int s0 = 0; s0 < steps; s0 += 3) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int s = s0 + u;
        if (s < steps) {
          load_x(min(kstep0 + s + 2, klast), xb[(u + 2) % 3]);
          load_w<FP8>(w1b[(u + 2) % 3], w1s, min(kstep0 + s + 2, klast));
          if (TWO) load_w<FP8>(w3b[(u + 2) % 3], w3s, min(kstep0 + s + 2, klast));
          compute(w1b[u], w3b[u], s & 1, kstep0 + s);
          store_x((s + 1) & 1, xb[(u + 1) % 3]);
          __syncthreads();
        }
      }
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
        } else if (a.out_f32) {
          float* o = static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol;
          *reinterpret_cast<f32x4*>(o) = acc[m];
        } else {
          u32x2 o = {pack_bf16x2(acc[m].x, acc[m].y), pack_bf16x2(acc[m].z, acc[m].w)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
        }
      }
    }
  }
}

template <bool FP8, int MODE, bool PACKED>
static hipError_t launch_mt(const StreamArgs& a, int mt, dim3 grid, hipStream_t s) {
  // one row tile: activations staged in registers, no barriers; more tiles
  // share an LDS activation tile between the four waves
  switch (mt) {
    case 1: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 1, PACKED, true>), grid, dim3(kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 2, PACKED, false>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 4, PACKED, false>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(const StreamArgs& a, int fp8, int packed, int mt, dim3 grid, hipStream_t s) {
  if (fp8) return packed ? launch_mt<true, MODE, true>(a, mt, grid, s) : launch_mt<true, MODE, false>(a, mt, grid, s);
  return packed ? launch_mt<false, MODE, true>(a, mt, grid, s) : launch_mt<false, MODE, false>(a, mt, grid, s);
}

hipError_t launch_ffn_stream(const StreamArgs& a, int fp8, int packed, int mode, int mt, dim3 grid,
                             hipStream_t s) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (mode == MODE_GATEUP) return launch_mode<MODE_GATEUP>(a, fp8, packed, mt, grid, s);
  if (mode == MODE_DOWN) return launch_mode<MODE_DOWN>(a, fp8, packed, mt, grid, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Weight packing: row-major [G, N, Kdim] -> per 128-wide K step and 16-row
// panel (step-major: the blocks of one K step of all panels are adjacent), the
// NI 1-KiB blocks the expert kernels load, in lane order.  Element (n, k) of
// one matrix goes to
//   step k/128, panel n/16, then (bf16) block kk/32 lane 16*((kk%32)/8) + n%16
//   element kk%8, or (fp8) block kk/64 lane 16*((kk%64)/16) + n%16 byte kk%16,
// with kk = k % 128.  Workgroups that stream different panels advance through
// K at about the same pace, so at any moment the reads of the whole grid fall
// in a compact window of memory.  One thread moves one 16-byte piece.
template <bool FP8>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int64_t pieces, int N, int Kdim) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  constexpr int wbytes = FP8 ? 1 : 2;
  constexpr int NI = FP8 ? 2 : 4;
  // destination order: [g][step][panel][instr][lane] pieces of 16 bytes
  const int lane = int(i % 64);
  int64_t r = i / 64;
  const int instr = int(r % NI); r /= NI;
  const int64_t panel = r % (N / 16); r /= (N / 16);
  const int steps = Kdim / kKS;
  const int step = int(r % steps);
  const int64_t g = r / steps;
  const int64_t n = panel * 16 + (lane & 15);
  const int kk = FP8 ? 64 * instr + 16 * (lane >> 4) : 32 * instr + 8 * (lane >> 4);
  const int64_t k = (int64_t)step * kKS + kk;
  const int64_t soff = ((g * N + n) * Kdim + k) * wbytes;
  *reinterpret_cast<u32x4*>(dst + i * 16) = *reinterpret_cast<const u32x4*>(src + soff);
}

hipError_t launch_pack(const void* src, void* dst, int G, int N, int Kdim, int fp8, hipStream_t s) {
  const int64_t bytes = (int64_t)G * N * Kdim * (fp8 ? 1 : 2);
  const int64_t pieces = bytes / 16;
  if (pieces == 0) return hipSuccess;
  const dim3 grid((unsigned)((pieces + 255) / 256));
  if (fp8) hipLaunchKernelGGL((pack_kernel<true>), grid, dim3(256), 0, s,
                              static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), pieces, N, Kdim);
  else hipLaunchKernelGGL((pack_kernel<false>), grid, dim3(256), 0, s,
                          static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), pieces, N, Kdim);
  return hipGetLastError();
}

}  // namespace moe
