// Device functions of the streaming grouped GEMM (one group's 64-row output
// blocks), shared by the streaming kernel and the persistent decode kernel.
// The method is described in ffn_stream.hip.
#pragma once
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kThreads = 256;        // 4 waves
constexpr int kBN = 64;              // weight rows per workgroup
constexpr int kKS = 128;             // K per pipeline step
constexpr int kLdsStride = kKS + 8;  // bf16 elements per LDS row (pad vs bank conflicts)
constexpr int kXlSteps = 16;         // K steps of LDS-resident activations (16 x 4 KiB)

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <bool FP8>
struct WFrag {
  static constexpr int NI = FP8 ? 2 : 4;
  u32x4 v[NI];
};

// Byte addressing of one wave's weight stream, for the wave's 16 rows in the
// j-th 64-row block of its workgroup:
//   address(j, kstep, i) = base + j * blk_bytes + kstep * step_bytes + i * instr_bytes + lane_bytes
struct WStream {
  const char* base;
  int64_t blk_bytes;
  int step_bytes, instr_bytes, lane_bytes;
};

// NT: the weights are read once per call and never again, so the loads are
// non-temporal, streamed past the caches instead of evicting the activations
// and tables other workgroups still read.  Groups whose row-tile passes run
// on several workgroups (region B) re-read their weights and load normally.
template <bool FP8, bool NT>
__device__ __forceinline__ void load_w(WFrag<FP8>& f, const WStream& w, int j, int kstep) {
  const char* p = w.base + j * w.blk_bytes + (int64_t)kstep * w.step_bytes + w.lane_bytes;
#pragma unroll
  for (int i = 0; i < WFrag<FP8>::NI; ++i) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p + i * w.instr_bytes);
    f.v[i] = NT ? __builtin_nontemporal_load(q) : *q;
  }
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
    s.blk_bytes = (int64_t)kBN * kKS * wbytes;      // four panels further
    s.instr_bytes = 1024;
    s.lane_bytes = 16 * lane;
  } else {
    s.base = static_cast<const char*>(Wg) + (int64_t)(n_w0 + (lane & 15)) * Kdim * wbytes;
    s.step_bytes = kKS * wbytes;
    s.blk_bytes = (int64_t)kBN * Kdim * wbytes;     // 64 rows further
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

// LDS activation tile of the MT > 1 passes: two buffers of MT*16 rows
template <int MT>
constexpr int lds_elems() { return MT > 1 ? 2 * MT * 16 * kLdsStride : 1; }

// Pipeline depth of the main size class: NB register banks, NB - 1 K steps
// in flight.  An fp8 down step moves a quarter of the bytes of a bf16 gate/up
// step and its registers leave room, so it keeps three steps in flight.  The
// large-group class (region B) shares the kernel and its register count, so
// it never sets that count: with fp8 it takes two row tiles per pass and one
// step in flight; with bf16 four tiles, and two steps in flight for gate/up
// (whose main class needs more registers anyway) or one for down.
template <bool FP8, int MODE>
constexpr int banks_a() { return (FP8 && MODE == MODE_DOWN) ? 4 : 3; }
template <bool FP8, int MODE>
constexpr int banks_b() { return (FP8 || MODE == MODE_DOWN) ? 2 : 3; }
template <bool FP8>
constexpr int tiles_b() { return FP8 ? 2 : 4; }
// LDS-resident activations (fp8 down projection, one row tile, K range of at
// most kXlSteps steps = 64 KiB): with no activation registers the weight
// stream keeps NB - 1 = 11 steps (2 KiB a step and wave) in flight
template <bool FP8>
constexpr int banks_xl() { return FP8 ? 12 : 6; }

// The rows of group g if its row count is in (lo, hi] (hi = 0: no limit):
// row-tile passes mc, mc + mch, ... of it, K split ks, output blocks
// bx * nblk .. bx * nblk + nblk - 1.
// XL (single-tile passes only): the tile's activations for the split's whole
// K range (at most kXlSteps steps) are staged once into LDS, in MFMA fragment
// order, before the weight stream starts; the stream then carries weights
// only and never synchronises.
// Output stores.  WT: agent-scope stores (written through the XCD's L2), for
// outputs that workgroups on other XCDs read later in the same launch.
template <bool WT>
__device__ __forceinline__ void store_u32x2(void* p, u32x2 v) {
  if constexpr (WT)
    __hip_atomic_store(static_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *static_cast<u32x2*>(p) = v;
}
template <bool WT>
__device__ __forceinline__ void store_f32x4(float* p, f32x4 v) {
  if constexpr (WT) {
    store_u32x2<true>(p, u32x2{__float_as_uint(v.x), __float_as_uint(v.y)});
    store_u32x2<true>(p + 2, u32x2{__float_as_uint(v.z), __float_as_uint(v.w)});
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

template <bool FP8, int MODE, int MT, bool PACKED, int NB, bool NT, bool XL = false, bool WT = false>
__device__ __forceinline__ void stream_group(const StreamArgs& a, int g, int ks, int mc, int mch, int lo,
                                             int hi, uint16_t* __restrict__ xs_raw, int bx) {
  constexpr bool TWO = MODE == MODE_GATEUP;
  constexpr bool XDIRECT = MT == 1;
  static_assert(!XL || MT == 1, "LDS-resident activations hold one row tile");
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
  // size class: another part of the grid (or another launch) owns the rest
  if (c0 + c1 <= lo || (hi > 0 && c0 + c1 > hi)) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // the workgroup owns a.nblk consecutive 64-row blocks; first row of this
  // wave in the first of them
  const int nblk = a.nblk;
  const int n_w0 = bx * (kBN * nblk) + wave * 16;
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
  // scale row of this wave's 16 rows in block j
  auto sb_row = [&](int j) { return ((n_w0 + kBN * j) / 128) * kb_per_row; };

  // ---- K range of this split
  const int steps = kb_per_row / a.ksplit;
  const int kstep0 = ks * steps;

  using XS = uint16_t[MT * 16][kLdsStride];
  XS* xs = reinterpret_cast<XS*>(xs_raw);
  // staging assignment (MT > 1): thread -> (row r of a 16-row tile, 16-byte chunk c)
  const int sr = tid >> 4, sc = tid & 15;

  for (int tile0 = mc * MT; tile0 < ntiles; tile0 += mch * MT) {
    Pass<MT> ps;
    ps.n = min(MT, ntiles - tile0);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      ps.start[m] = 0; ps.valid[m] = 0;
      if (m < ps.n) tile_rows(tile0 + m, s0, c0, nt0, s1, c1, ps.start[m], ps.valid[m]);
    }

    // Activation sources, clamped into the tile's valid rows (rows past the
    // valid count only feed MFMA columns that are never stored).  All loads
    // sit outside any branch so the compiler never waits on them early.
    // MT == 1: each lane streams its own row's MFMA fragments straight into
    // registers and the waves never synchronise.  MT > 1: the workgroup
    // stages the tiles into LDS, one 16-byte chunk per thread and tile.
    // With a gather the source row is the token of the row's rank in the
    // group: ranks of segment 0 are 0 .. c0-1, of segment 1 c0 .. c0+c1-1.
    const uint16_t* xsrc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = XDIRECT ? lr : sr;
      const bool live = m < ps.n && ps.valid[m] > 0;
      int64_t row = live ? ps.start[m] + min(r, ps.valid[m] - 1) : s0;
      if (a.gather_src) {
        const int tile = tile0 + (live ? m : 0);
        const int rank = (tile < nt0 ? 16 * tile : c0 + 16 * (tile - nt0)) + (live ? min(r, ps.valid[m] - 1) : 0);
        row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
      }
      xsrc[m] = a.X + row * a.ldx + (XDIRECT ? 0 : 8 * sc);
    }
    // K offset of MFMA operand q inside a 128-wide step for this lane:
    // bf16 operand q covers 32q + 8*lg .. +8; an fp8 step's 16-byte weight
    // piece i expands to operands 2i, 2i+1 covering 64i + 16*lg + 8*(q%2).
    auto xoff_g = [&](int q, int grp) { return FP8 ? 64 * (q >> 1) + 16 * grp + 8 * (q & 1) : 32 * q + 8 * grp; };
    auto xoff = [&](int q) { return xoff_g(q, lg); };
    constexpr int XV = XL ? 1 : (XDIRECT ? 4 : MT);   // 16-byte activation loads per thread and step
    auto load_x = [&](int kstep, u32x4* xr) {
      if constexpr (XL) {
        (void)kstep; (void)xr;
      } else if constexpr (XDIRECT) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xr[q] = *reinterpret_cast<const u32x4*>(xsrc[0] + (int64_t)kstep * kKS + xoff(q));
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          xr[m] = *reinterpret_cast<const u32x4*>(xsrc[m] + (int64_t)kstep * kKS);
      }
    };
    auto store_x = [&](int buf, const u32x4* xr) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        *reinterpret_cast<u32x4*>(&xs[buf][m * 16 + sr][8 * sc]) = xr[m];
    };
    // B operand q of tile m at K step kstep: LDS-resident piece (XL), bank xr
    // (MT == 1) or LDS buffer buf (MT > 1)
    const u32x4* xl = reinterpret_cast<const u32x4*>(xs_raw);
    auto bop = [&](const u32x4* xr, int buf, int m, int q, int kstep) -> bf16x8 {
      if constexpr (XL) return __builtin_bit_cast(bf16x8, xl[((kstep - kstep0) * 4 + q) * 64 + lane]);
      else if constexpr (XDIRECT) return __builtin_bit_cast(bf16x8, xr[q]);
      else return *reinterpret_cast<const bf16x8*>(&xs[buf][m * 16 + lr][xoff(q)]);
    };

    f32x4 acc[MT], acc3[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) { acc[m] = f32x4{0, 0, 0, 0}; acc3[m] = f32x4{0, 0, 0, 0}; }

    // one K step: multiply the weights in (wa, wb) with the step's activations.
    // fp8 block scales are never loaded at compute time: the wait for such a
    // load (vector-memory counters drain in order) would also wait for every
    // weight load in flight.  The down projection's scales travel with their
    // step's weights (SCALE_AHEAD); gate/up (SCALE_PRE) reads all of a
    // stream's scales (at most 128 steps) into two registers before its
    // weights, lane l of register i holding step 64 i + l, and takes each
    // with a lane read (longer streams do load at compute time).  Measured on
    // the DeepSeek-V3-shaped B=256 layer: down 815 -> 677 us; gate/up
    // 1247 -> 1204 us at two waves per SIMD, while at three it lost time.
    constexpr bool SCALE_AHEAD = FP8 && MODE == MODE_DOWN;
    constexpr bool SCALE_PRE = FP8 && MODE == MODE_GATEUP;
    auto compute = [&](const WFrag<FP8>& wa, const WFrag<FP8>& wb, const u32x4* xr, int buf, bool have,
                       float s1a, float s3a, int j, int kstep) {
      if (FP8) {
        float sc1 = s1a, sc3 = s3a;
        if (!have) {
          sc1 = Sg[sb_row(j) + kstep];
          sc3 = TWO ? S3g[sb_row(j) + kstep] : 0.f;
        }
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
              const bf16x8 b = bop(xr, buf, m, q, kstep);
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
            for (int q = 0; q < 4; ++q) {
              const bf16x8 b = bop(xr, buf, m, q, kstep);
              acc[m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wa.v[q]), b, acc[m]);
              if (TWO) acc3[m] = mfma16x16x32(__builtin_bit_cast(bf16x8, wb.v[q]), b, acc3[m]);
            }
          }
        }
      }
    };

    // ---- epilogue of block j: lane holds D[n = n_w0 + 64j + 4*lg + i][m = lr], i = 0..3
    auto epilogue = [&](int j) {
      const int ncol = n_w0 + kBN * j + 4 * lg;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < ps.n && lr < ps.valid[m]) {
          const int64_t row = ps.start[m] + lr;
          if (MODE == MODE_GATEUP) {
            const f32x4 gt = acc[m], up = acc3[m];
            u32x2 o = {pack_bf16x2(silu(gt.x) * up.x, silu(gt.y) * up.y),
                       pack_bf16x2(silu(gt.z) * up.z, silu(gt.w) * up.w)};
            store_u32x2<WT>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol, o);
          } else if (a.out_f32) {
            store_f32x4<WT>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol, acc[m]);
          } else {
            u32x2 o = {pack_bf16x2(acc[m].x, acc[m].y), pack_bf16x2(acc[m].z, acc[m].w)};
            store_u32x2<WT>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol, o);
          }
        }
        acc[m] = f32x4{0, 0, 0, 0};
        acc3[m] = f32x4{0, 0, 0, 0};
      }
    };

    // Pipeline.  The single-tile path (MT == 1) runs the workgroup's nblk
    // blocks x steps K steps as one stream: at step v the weights and
    // activations of steps v+1 .. v+NB-1 are in flight while step v is
    // multiplied, across block boundaries too, so a short K range does not
    // pay the load latency once per block.  MT > 1 runs one such stream per
    // block (its registers are spent on row tiles), stages step v+1's
    // (already arrived) activations into the other LDS buffer and
    // synchronises once per step.  Loads are issued activations-first:
    // vector-memory counters drain in order, so waiting for an activation
    // block never waits for weights issued after it.  Steps past the end of
    // a stream re-load its last step (clamped) instead of branching around
    // the loads; that data is never multiplied.
    constexpr bool FLAT = XDIRECT;
    const int span = FLAT ? nblk : 1;       // blocks per stream
    const int vsteps = span * steps;
    WFrag<FP8> w1b[NB], w3b[NB];
    float s1b[NB], s3b[NB];   // SCALE_AHEAD: the banks' block scales
    const bool pre = SCALE_PRE && vsteps <= 128;
    u32x4 xb[NB][XV];
    for (int jb = 0; jb < nblk; jb += span) {
      float sp1[2] = {0.f, 0.f}, sp3[2] = {0.f, 0.f};   // SCALE_PRE: the stream's scales
      if constexpr (SCALE_PRE) {
        if (pre) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int v = min(64 * i + lane, vsteps - 1);
            const int j = jb + v / steps, k = kstep0 + v % steps;
            sp1[i] = Sg[sb_row(j) + k];
            if (TWO) sp3[i] = S3g[sb_row(j) + k];
          }
        }
      }
      auto lane_scale = [&](const float* r, int v) {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v < 64 ? r[0] : r[1]), v & 63));
      };
      int lj = jb, lk = 0;   // block and K step of the next loads
      auto issue = [&](int bank) {
        const bool in = lj < jb + span;
        const int j = in ? lj : jb + span - 1;
        const int k = kstep0 + (in ? lk : steps - 1);
        load_x(k, xb[bank]);
        if constexpr (SCALE_AHEAD) {
          s1b[bank] = Sg[sb_row(j) + k];
          s3b[bank] = TWO ? S3g[sb_row(j) + k] : 0.f;
        }
        load_w<FP8, NT>(w1b[bank], w1s, j, k);
        if (TWO) load_w<FP8, NT>(w3b[bank], w3s, j, k);
        if (++lk == steps) { lk = 0; ++lj; }
      };
      // XL: piece p = (s*4 + q)*64 + l of the LDS tile is operand q of K
      // step s for lane l (row l%16, K group l/16); thread t moves pieces
      // t + 256i.  The activation loads are issued before the weights so the
      // wait for them leaves the weight loads in flight.
      u32x4 xst[XL ? kXlSteps : 1];
      if constexpr (XL) {
        const int vrow = ps.valid[0] - 1;
#pragma unroll
        for (int i = 0; i < kXlSteps; ++i) {
          const int pc = tid + 256 * i, l = pc & 63, q = (pc >> 6) & 3, st = pc >> 8;
          const int64_t row = ps.start[0] + min(l & 15, vrow);
          const int k = kstep0 + (st < steps ? st : 0);
          xst[i] = *reinterpret_cast<const u32x4*>(a.X + row * a.ldx + (int64_t)k * kKS + xoff_g(q, l >> 4));
        }
      }
#pragma unroll
      for (int p = 0; p < NB - 1; ++p) issue(p);
      if constexpr (XL) {
        u32x4* xw = reinterpret_cast<u32x4*>(xs_raw);
#pragma unroll
        for (int i = 0; i < kXlSteps; ++i)
          if (((tid + 256 * i) >> 8) < steps) xw[tid + 256 * i] = xst[i];
        __syncthreads();
      }
      if constexpr (!XDIRECT) {
        store_x(0, xb[0]);
        __syncthreads();
      }
      int cj = jb, ck = 0;   // block and K step being multiplied
      for (int v0 = 0; v0 < vsteps; v0 += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int v = v0 + u;
          if (v < vsteps) {
            issue((u + NB - 1) % NB);
            float s1v = 0.f, s3v = 0.f;
            if constexpr (SCALE_AHEAD) {
              s1v = s1b[u];
              s3v = s3b[u];
            } else if constexpr (SCALE_PRE) {
              if (pre) {
                s1v = lane_scale(sp1, v);
                s3v = TWO ? lane_scale(sp3, v) : 0.f;
              }
            }
            compute(w1b[u], w3b[u], xb[u], v & 1, SCALE_AHEAD || pre, s1v, s3v, cj, kstep0 + ck);
            if constexpr (!XDIRECT) {
              store_x((v + 1) & 1, xb[(u + 1) % NB]);
              __syncthreads();
            }
            if constexpr (FLAT) {
              if (++ck == steps) { epilogue(cj); ck = 0; ++cj; }
            } else {
              ++ck;
            }
          }
        }
      }
      if constexpr (!FLAT) epilogue(jb);
    }

    if constexpr (!XDIRECT || XL) __syncthreads();   // LDS buffer reuse by the next pass
  }
}

}  // namespace moe
