// LDS-tiled grouped GEMM for large expert groups on gfx950 (CDNA4).
//
// Prefill rows per expert (hundreds), the shared expert of a large batch and
// hot replica slots have enough rows that each weight tile can be reused from
// LDS for a whole 128-row tile of tokens: the contiguous layout with large
// tiles that amortises weight reads ("推理 INFRA 方法论(5)", DeepGEMM
// section: prefill uses the contiguous layout and large tiles).
//
//  * Workgroup tile: 128 token rows x 256 weight rows (MODE_GATEUP: 128 gate
//    rows of W1 + the same 128 rows of W3, so SiLU(g) * u pairs sit in one
//    wave; MODE_DOWN: 256 rows of W2).  Four waves split the weight rows; each
//    wave owns all 128 token rows x 64 weight rows = 8 x 4 MFMA
//    tiles of 16 x 16.
//  * K advances in 64-wide stages, double-buffered in LDS.  Both operands are
//    stored in MFMA fragment order (per 16-row tile and 32-wide K step, the
//    16-byte piece of each lane, slots rotated by swz() against bank
//    conflicts), so every operand read is one conflict-free ds_read_b128.
//    Global loads run kTBanks - 1 stages ahead through kTBanks register
//    banks, so a stage's MFMAs overlap the following stages' memory latency.
//  * Work list: slot p owns ceil(T_p / 128) row tiles, the shared expert
//    ceil(T / 128), in the prefix tile_off; each row tile pairs with every
//    weight-row tile.  The list is ordered (group, weight tile, row tile) and
//    dealt to the XCDs in contiguous chunks, so the row tiles that share a
//    weight tile run back to back on one XCD and the later ones find it in
//    that XCD's L2.  Groups with at most `min_rows` rows are left to the
//    streaming kernel (none are when groups are large on average).
//  * A group's last row tile is usually partly empty (groups are 28..961
//    rows at the prefill workload): the tile is run with only its non-empty
//    32-row sub-tiles (a compile-time count, one instance per count), so no
//    MFMA, LDS read or activation load is spent on whole pad sub-tiles.
//  * Each output element accumulates its K range in 32-wide MFMA steps in
//    ascending order, exactly as the streaming kernel does, so the split of
//    groups between the two kernels does not change any bit of the result.
//
// Four kernels share the work list and that MFMA order (bit-identical
// outputs): ffn_tiled_kernel, the tile above; ffn_wide_kernel, 128 token rows
// x 512 weight rows with one wave per SIMD owning 128 x 128 outputs, operands
// staged through registers; ffn_wdma_kernel, the wide tile with both operands
// staged by direct-to-LDS loads; ffn_whyb_kernel, the wide tile with weights
// straight to registers and only activations through LDS (the default for
// packed weights whose K range is whole blocks of four 32-wide steps).
#include <cstdlib>

#include "common.hpp"
#include "kernels.hpp"
#include "tile_sched.hpp"

namespace moe {

constexpr int kTM = 128;     // token rows per tile
constexpr int kTN = 256;     // weight rows per tile
constexpr int kTK = 64;      // K per stage
constexpr int kTThreads = 256;
// register banks of the global-load pipeline: kTBanks - 1 stages in flight
// (a stage is 64 MFMAs per wave, about 0.43 us at full rate).  The kernel
// runs one wave per SIMD; three banks leave the registers for two sets of
// operand fragments (the LDS reads run one K step ahead of the MFMAs).
constexpr int kTBanks = 3;

// LDS bytes per stage: the 128 x 64 bf16 activation tile
constexpr int kXStage = kTM * kTK * 2;   // 16 KiB

__device__ __forceinline__ float silu_t(float g) { return g / (1.0f + __expf(-g)); }

// Physical 16-byte slot of fragment piece (lane, c) inside its 1 KiB block,
// c = 4*j + lane/16 being the piece's 16-byte column within the 128-byte row
// of the 64-wide K stage.  The low four slot bits are rotated by 2c: the
// lane-linear MFMA operand reads of one quarter wave still hit 16 distinct
// 16-byte bank groups, and so do the stores of 16 consecutive threads, which
// cover 2 rows x 8 columns of the row-major source.
__device__ __forceinline__ int swz(int lane, int j) {
  const int c = 4 * j + (lane >> 4);
  return (lane & 48) | (((lane & 15) + 2 * c) & 15);
}

// The hardware deals workgroups round-robin over the 8 XCDs (linear id L goes
// to XCD L % 8).  The live work list -- tile_off's ceil(rows/128) tiles per
// group times the weight-row tiles -- is cut into 8 contiguous chunks, one per
// XCD, ordered (group, weight tile, row tile), so the workgroups an XCD runs
// together share one group's weight and activation tiles in that XCD's L2.
// Returns false when this workgroup has no work.
__device__ __forceinline__ bool decode_work(const TiledArgs& ta, TileWork& w) {
  const StreamArgs& a = ta.s;
  const int ngroups = a.E_phys + 1;
  const int ntiles_n = gridDim.x;
  const int64_t work = (int64_t)ta.tile_off[ngroups] * ntiles_n;
  const int64_t L = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t chunk = (work + 7) / 8;
  const int64_t k_in = L / 8;
  if (k_in >= chunk) return false;
  const int64_t wi = (L % 8) * chunk + k_in;
  if (wi >= work) return false;
  int lo = 0, hi = ngroups;                  // largest g with tile_off[g] * ntiles_n <= wi
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)ta.tile_off[mid] * ntiles_n <= wi) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mtiles = ta.tile_off[g + 1] - ta.tile_off[g];
  const int64_t o = wi - (int64_t)ta.tile_off[g] * ntiles_n;
  group_rows(a, g, w);
  w.nt = int(o / mtiles);                    // weight-row tile
  w.mt = int(o % mtiles);                    // row tile within the group
  return w.R > ta.min_rows;                  // else the streaming kernel owns this group
}

template <int MODE, bool PACKED>
__global__ __launch_bounds__(kTThreads) void ffn_tiled_kernel(TiledArgs ta) {
  const StreamArgs& a = ta.s;
  __shared__ __attribute__((aligned(16))) char xsm[2 * kXStage];   // activation tile, 2 stages

  TileWork tw;
  if (!decode_work(ta, tw)) return;
  const int g = tw.g, nt = tw.nt, mt = tw.mt, c0 = tw.c0, R = tw.R;
  const int64_t s0 = tw.s0, s1 = tw.s1;
  const bool shared = tw.shared;
  // a work item is a kTileRows-row tile: its 128-row halves in turn
  for (int half = 0; half < kTileRows / kTM; ++half) {
    const int m0 = mt * kTileRows + half * kTM;   // first row of this half within the group
    if (m0 >= R) break;
    if (half) __syncthreads();             // the previous half is done with the LDS

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int Kdim = a.Kdim;
    const int ks = blockIdx.z;
    const int kper = Kdim / a.ksplit;
    const int kbeg = ks * kper;
    const int nstages = kper / kTK;

    // ---- weight rows of this tile: wave w owns four 16-row weight tiles
    //   GATEUP: W1 rows n0 + 32w .. +32 (tiles 0, 1) and the same W3 rows (tiles 2, 3)
    //   DOWN:   W2 rows n0 + 64w .. +64
    const int n0 = MODE == MODE_GATEUP ? nt * 128 : nt * kTN;
    const char* Wa;
    const char* Wb = nullptr;
    if (shared) { Wa = static_cast<const char*>(a.SW); Wb = static_cast<const char*>(a.SW3); }
    else {
      Wa = static_cast<const char*>(a.W) + (int64_t)g * a.N * Kdim * 2;
      if (MODE == MODE_GATEUP) Wb = static_cast<const char*>(a.W3) + (int64_t)g * a.N * Kdim * 2;
    }
    // per weight tile: byte address of this lane's piece at K = 0, and the step
    // per 32-wide K chunk (the MFMA A operand: row lane%16, K 8*(lane/16)..+8)
    const char* wsrc[4];
  #pragma unroll
    for (int n = 0; n < 4; ++n) {
      int row0;
      const char* base;
      if (MODE == MODE_GATEUP) { row0 = n0 + 32 * wave + 16 * (n & 1); base = n < 2 ? Wa : Wb; }
      else { row0 = n0 + 64 * wave + 16 * n; base = Wa; }
      if (PACKED) wsrc[n] = base + (int64_t)(row0 / 16) * 16 * 128 * 2 + lane * 16;
      else wsrc[n] = base + (int64_t)(row0 + (lane & 15)) * Kdim * 2 + 16 * (lane >> 4);
    }
    // byte offset of 32-wide K chunk kc (K = 32 kc) in a weight stream
    auto wk = [&](int kc) -> int64_t {
      if (PACKED) return (int64_t)(kc >> 2) * (a.N / 16) * 4096 + (kc & 3) * 1024;   // step-major
      return (int64_t)kc * 64;
    };

    // ---- activation tile (128 rows x 64 K per stage) through LDS, fragment order
    // thread t copies row t/8 + 32q, 16-byte column t%8 of the stage
    const int xc = tid & 7;
    const char* xsrc[4];
    int xdst[4];
  #pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (tid >> 3) + 32 * q;
      const int gr = m0 + r;                               // row within the group
      int64_t row = gr < c0 ? s0 + gr : (gr < R ? s1 + (gr - c0) : s0);   // pad rows read a valid row
      if (a.gather_src) {                                  // the token of rank gr (pad rows: rank 0)
        const int rank = gr < R ? gr : 0;
        row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
      }
      xsrc[q] = reinterpret_cast<const char*>(a.X + row * a.ldx) + 16 * xc;
      xdst[q] = (((r >> 4) * 2 + (xc >> 2)) * 64 + swz(16 * (xc & 3) + (r & 15), xc >> 2)) * 16;
    }

    // the tile's non-empty 16-row tiles, rounded up to 32-row sub-tiles
    const int rows_here = min(kTM, R - m0);
    const int mv = ((rows_here + 31) / 32) * 2;
    auto run = [&](auto mvc) {
      // Global loads run kTBanks - 1 stages ahead (per
      // stage: the activation pieces first, then the weights; vector-memory
      // counters drain in order, so staging the activations never waits for the
      // weights issued after them).
      constexpr int MV = decltype(mvc)::value;    // non-empty 16-row tiles (even)
      constexpr int XQ = MV / 2;                   // activation pieces per thread and stage
      u32x4 xr[kTBanks][XQ], wr[kTBanks][4][2];
      auto gload = [&](int bank, int stage) {
        const int k0 = kbeg + stage * kTK;
  #pragma unroll
        for (int q = 0; q < XQ; ++q) xr[bank][q] = *reinterpret_cast<const u32x4*>(xsrc[q] + (int64_t)k0 * 2);
  #pragma unroll
        for (int n = 0; n < 4; ++n)
  #pragma unroll
          for (int j = 0; j < 2; ++j)
            wr[bank][n][j] = *reinterpret_cast<const u32x4*>(wsrc[n] + wk(k0 / 32 + j));
      };
      auto lstore = [&](int bank, int buf) {
  #pragma unroll
        for (int q = 0; q < XQ; ++q) *reinterpret_cast<u32x4*>(xsm + buf * kXStage + xdst[q]) = xr[bank][q];
      };

      f32x4 acc[MV][4];
  #pragma unroll
      for (int m = 0; m < MV; ++m)
  #pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0, 0, 0, 0};

      // operand fragments of one 32-wide K step j of LDS buffer buf
      auto lread = [&](bf16x8* xf, int buf, int j) {
        const char* xb = xsm + buf * kXStage;
  #pragma unroll
        for (int m = 0; m < MV; ++m)
          xf[m] = *reinterpret_cast<const bf16x8*>(xb + ((m * 2 + j) * 64 + swz(lane, j)) * 16);
      };
      auto mma = [&](int bank, const bf16x8* xf, int j) {
  #pragma unroll
        for (int m = 0; m < MV; ++m)
  #pragma unroll
          for (int n = 0; n < 4; ++n)
            acc[m][n] = mfma16x16x32(__builtin_bit_cast(bf16x8, wr[bank][n][j]), xf[m], acc[m][n]);
      };

      // Operand reads are software-pipelined against the MFMAs: with one wave
      // per SIMD nothing else hides their latency.  Per stage st: the reads of
      // K step 1 are issued, then the global loads; K step 0's MFMAs run on
      // fragments read at the end of the previous stage; the next stage's
      // activations are stored to the other LDS buffer; K step 1's MFMAs run;
      // barrier; the next stage's K step 0 reads are issued at once.  Stages
      // past the end re-load the last stage (clamped) instead of branching
      // around loads; the extra LDS copy goes to the buffer not being read.
      bf16x8 xa[MV], xbv[MV];
      const int slast = nstages - 1;
  #pragma unroll
      for (int p = 0; p < kTBanks - 1; ++p) gload(p, min(p, slast));
      lstore(0, 0);
      __syncthreads();
      lread(xa, 0, 0);
      for (int s0 = 0; s0 < nstages; s0 += kTBanks) {
  #pragma unroll
        for (int u = 0; u < kTBanks; ++u) {
          const int st = s0 + u;
          if (st < nstages) {
            lread(xbv, st & 1, 1);
            gload((u + kTBanks - 1) % kTBanks, min(st + kTBanks - 1, slast));
            mma(u, xa, 0);
            lstore((u + 1) % kTBanks, (st + 1) & 1);   // that buffer was last read before the previous barrier
            mma(u, xbv, 1);
            __syncthreads();
            lread(xa, (st + 1) & 1, 0);                 // after the last stage: unused reads of written LDS
          }
        }
      }

      // ---- epilogue: acc[m][n] holds D[w-row 4*(lane/16)+j of tile n][token lane%16 of tile m]
      const int lr = lane & 15, lg = lane >> 4;
  #pragma unroll
      for (int m = 0; m < MV; ++m) {
        const int gr = m0 + m * 16 + lr;                    // row within the group
        if (gr >= R) continue;
        const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
        if (MODE == MODE_GATEUP) {
  #pragma unroll
          for (int n = 0; n < 2; ++n) {
            const f32x4 gt = acc[m][n], up = acc[m][n + 2];
            const int ncol = n0 + 32 * wave + 16 * n + 4 * lg;
            u32x2 o = {pack_bf16x2(silu_t(gt.x) * up.x, silu_t(gt.y) * up.y),
                       pack_bf16x2(silu_t(gt.z) * up.z, silu_t(gt.w) * up.w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
          }
        } else {
  #pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int ncol = n0 + 64 * wave + 16 * n + 4 * lg;
            if (a.out_f32) {
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol) = acc[m][n];
            } else {
              u32x2 o = {pack_bf16x2(acc[m][n].x, acc[m][n].y), pack_bf16x2(acc[m][n].z, acc[m][n].w)};
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
            }
          }
        }
      }
    };
    switch (mv) {
      case 2: run(IntC<2>{}); break;
      case 4: run(IntC<4>{}); break;
      case 6: run(IntC<6>{}); break;
      default: run(IntC<8>{}); break;
    }
  }
}

// ---- wide variant: 128 token rows x 512 weight rows per workgroup ----------
//
// Each wave owns all 128 token rows x 128 weight rows (8 x 8 MFMA tiles, the
// 256 accumulator registers of a wave running alone on its SIMD), so every
// activation fragment read from LDS feeds eight MFMAs instead of four: the
// LDS operand traffic per MFMA is half the narrow kernel's.  K advances in
// 32-wide steps (one MFMA K); the activation step (8 KiB, fragment order, one
// ds_read_b128 per 16-row tile) is double-buffered in LDS, and the global
// loads of weights and activations run kWBanks - 1 steps ahead through
// kWBanks register banks.
constexpr int kWN = 512;                 // weight rows per tile
constexpr int kWBanks = 3;
constexpr int kWStage = kTM * 32 * 2;    // 8 KiB: 128 rows x 32 K

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// OUTF32 (down projection only): fp32 partial planes of a K split, else bf16
// (a template argument: with both epilogues in one kernel the accumulators
// are copied out and spilled ahead of the branch)
template <int MODE, bool PACKED, bool OUTF32>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ffn_wide_kernel(TiledArgs ta) {
  const StreamArgs& a = ta.s;
  __shared__ __attribute__((aligned(16))) char xsm[2 * kWStage];

  TileWork tw;
  if (!decode_work(ta, tw)) return;
  const int g = tw.g, nt = tw.nt, c0 = tw.c0, R = tw.R;
  const int64_t s0 = tw.s0, s1 = tw.s1;
  const bool shared = tw.shared;
  // a work item is a kTileRows-row tile: its 128-row halves in turn
  for (int half = 0; half < kTileRows / kTM; ++half) {
    const int m0 = tw.mt * kTileRows + half * kTM;   // first row of this half within the group
    if (m0 >= R) break;
    if (half) __syncthreads();             // the previous half is done with the LDS

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int Kdim = a.Kdim;
    const int ks = blockIdx.z;
    const int kper = Kdim / a.ksplit;
    const int kc0 = ks * kper / 32;           // first 32-wide K chunk
    const int nsteps = kper / 32;

    // ---- weight rows: wave w owns eight 16-row weight tiles
    //   GATEUP: W1 rows n0 + 64w .. +64 (tiles 0..3) and the same W3 rows (tiles 4..7)
    //   DOWN:   W2 rows n0 + 128w .. +128
    const int n0 = MODE == MODE_GATEUP ? nt * (kWN / 2) : nt * kWN;
    const char* Wa;
    const char* Wb = nullptr;
    if (shared) { Wa = static_cast<const char*>(a.SW); Wb = static_cast<const char*>(a.SW3); }
    else {
      Wa = static_cast<const char*>(a.W) + (int64_t)g * a.N * Kdim * 2;
      if (MODE == MODE_GATEUP) Wb = static_cast<const char*>(a.W3) + (int64_t)g * a.N * Kdim * 2;
    }
    // buffer resources over one weight matrix (N x Kdim) and the activation rows
    const uint32_t wbytes = (uint32_t)a.N * Kdim * 2;
    const __amdgpu_buffer_rsrc_t wra = buffer_rsrc(Wa, wbytes);
    const __amdgpu_buffer_rsrc_t wrb = buffer_rsrc(MODE == MODE_GATEUP ? Wb : Wa, wbytes);
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(a.X, (uint32_t)ta.x_bytes);
    //   weight tile n: byte offset of this lane's piece at K = 0 within its matrix
    uint32_t woff[8];
  #pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int row0 = MODE == MODE_GATEUP ? n0 + 64 * wave + 16 * (n & 3) : n0 + 128 * wave + 16 * n;
      if (PACKED) woff[n] = (uint32_t)(row0 / 16) * 16 * 128 * 2 + lane * 16;
      else woff[n] = (uint32_t)(row0 + (lane & 15)) * Kdim * 2 + 16 * (lane >> 4);
    }
    auto wk = [&](int kc) -> uint32_t {    // byte offset of 32-wide K chunk kc
      if (PACKED) return (uint32_t)(kc >> 2) * (a.N / 16) * 4096 + (kc & 3) * 1024;   // step-major
      return (uint32_t)kc * 64;
    };

    // ---- activations: thread t stages 16-row tile wave + 4q, row t % 16, 16-byte
    // K column (t / 16) % 4 of each step, i.e. fragment slot t % 64 of that tile
    uint32_t xoff[2];
  #pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int gr = m0 + (wave + 4 * q) * 16 + (lane & 15);   // row within the group
      int64_t row = gr < c0 ? s0 + gr : (gr < R ? s1 + (gr - c0) : s0);   // pad rows read a valid row
      if (a.gather_src) {
        const int rank = gr < R ? gr : 0;
        row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
      }
      xoff[q] = (uint32_t)(row * a.ldx * 2) + 16 * (lane >> 4);
    }

    const int rows_here = min(kTM, R - m0);
    const int mv = ((rows_here + 31) / 32) * 2;
    auto run = [&](auto mvc) {
      constexpr int MV = decltype(mvc)::value;    // non-empty 16-row tiles (even)
      // weights and activations run kWBanks - 1 steps ahead (bank = step % kWBanks)
      u32x4 xr[kWBanks][2], wr[kWBanks][8];
      // (every wave stages both of its tiles, also the empty ones past MV, which
      // read a valid row: loads that depend on the wave would be branches, and
      // the compiler then waits for every outstanding load once per pass)
      auto gload_x = [&](int bank, int step) {
        const uint32_t so = (uint32_t)(kc0 + step) * 64;
  #pragma unroll
        for (int q = 0; q < 2; ++q) xr[bank][q] = buffer_load16(xrs, xoff[q], so);
      };
      auto gload_w = [&](int bank, int step) {
        const uint32_t so = wk(kc0 + step);
  #pragma unroll
        for (int n = 0; n < 8; ++n)
          wr[bank][n] = buffer_load16(MODE == MODE_GATEUP && n >= 4 ? wrb : wra, woff[n], so);
      };
      auto lstore = [&](int bank, int buf) {
  #pragma unroll
        for (int q = 0; q < 2; ++q)
          *reinterpret_cast<u32x4*>(xsm + buf * kWStage + ((wave + 4 * q) * 64 + lane) * 16) = xr[bank][q];
      };

      f32x4 acc[MV][8];
  #pragma unroll
      for (int m = 0; m < MV; ++m)
  #pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0, 0, 0, 0};

      // Per step st: the activations and weights of step st + kWBanks - 1 are
      // issued into the bank step st - 1 freed; the MFMAs of step st run on
      // bank st % kWBanks and LDS buffer st % 2; step st + 1's activations go to
      // the other buffer (last read before the previous barrier); barrier.
      // Steps past the end re-load the last step (clamped) instead of branching
      // around loads.
      const int slast = nsteps - 1;
  #pragma unroll
      for (int p = 0; p < kWBanks - 1; ++p) {
        gload_x(p, min(p, slast));
        gload_w(p, min(p, slast));
      }
      lstore(0, 0);
      __syncthreads();
      for (int sb = 0; sb < nsteps; sb += kWBanks) {
  #pragma unroll
        for (int u = 0; u < kWBanks; ++u) {
          const int st = sb + u;
          if (st < nsteps) {
            gload_x((u + kWBanks - 1) % kWBanks, min(st + kWBanks - 1, slast));
            gload_w((u + kWBanks - 1) % kWBanks, min(st + kWBanks - 1, slast));
            // (scheduling fences keep each step's loads, reads and MFMAs in their
            // step: hoisted across steps they outgrow the register file)
            __builtin_amdgcn_sched_barrier(0);
            const char* xb = xsm + (st & 1) * kWStage;
            bf16x8 xf[MV];
  #pragma unroll
            for (int m = 0; m < MV; ++m) xf[m] = *reinterpret_cast<const bf16x8*>(xb + (m * 64 + lane) * 16);
  #pragma unroll
            for (int m = 0; m < MV; ++m)
  #pragma unroll
              for (int n = 0; n < 8; ++n)
                acc[m][n] = mfma16x16x32(__builtin_bit_cast(bf16x8, wr[u][n]), xf[m], acc[m][n]);
            // order: the reads of tiles 0 and 1, then per tile m its 8 MFMAs
            // followed by the read of tile m + 2, so each read has a tile's
            // MFMAs (8 x 16 cycles) to land
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  #pragma unroll
            for (int m = 0; m < MV; ++m) {
              __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
              if (m + 2 < MV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            lstore((u + 1) % kWBanks, (st + 1) & 1);
            __syncthreads();
          }
        }
      }

      // ---- epilogue: acc[m][n] holds D[w-row 4*(lane/16)+j of tile n][token lane%16 of tile m]
      const int lr = lane & 15, lg = lane >> 4;
  #pragma unroll
      for (int m = 0; m < MV; ++m) {
        const int gr = m0 + m * 16 + lr;
        if (gr >= R) continue;
        const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
        if (MODE == MODE_GATEUP) {
  #pragma unroll
          for (int n = 0; n < 4; ++n) {
            const f32x4 gt = acc[m][n], up = acc[m][n + 4];
            const int ncol = n0 + 64 * wave + 16 * n + 4 * lg;
            u32x2 o = {pack_bf16x2(silu_t(gt.x) * up.x, silu_t(gt.y) * up.y),
                       pack_bf16x2(silu_t(gt.z) * up.z, silu_t(gt.w) * up.w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
          }
        } else {
  #pragma unroll
          for (int n = 0; n < 8; ++n) {
            const int ncol = n0 + 128 * wave + 16 * n + 4 * lg;
            if constexpr (OUTF32) {
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol) = acc[m][n];
            } else {
              u32x2 o = {pack_bf16x2(acc[m][n].x, acc[m][n].y), pack_bf16x2(acc[m][n].z, acc[m][n].w)};
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
            }
          }
        }
      }
    };
    switch (mv) {
      case 2: run(IntC<2>{}); break;
      case 4: run(IntC<4>{}); break;
      case 6: run(IntC<6>{}); break;
      default: run(IntC<8>{}); break;
    }
  }
}

// ---- wide tile with operands staged by direct-to-LDS loads ------------------
//
// The tile, the waves' outputs and the MFMA order are ffn_wide_kernel's (so
// the results are the same bit for bit), but weights and activations go from
// memory straight into a ring of kDStages LDS stages (buffer_load ... lds,
// each lane's 16 bytes landing at stage base + 16 * lane), so kDStages - 1
// 32-wide K steps are in flight without holding registers.  Each wave then
// reads its 8 weight fragments and the step's activation fragments from LDS
// (ds_read_b128 of 1 KiB lane-contiguous panels, free of bank conflicts).
// Fragment reads are software-pipelined: step st multiplies the fragments
// read from LDS during step st - 1 while reading those of step st + 1, so the
// LDS reads run under the MFMAs even at one wave per SIMD.  Per step: wait
// for the wave's own loads of stage st + 1 (vector-memory counters drain in
// order) and its fragment reads of step st, barrier (every wave's loads of
// stage st + 1 have landed and every wave has finished reading stage st - 1),
// issue the loads of step st + kDStages - 1 into stage st - 1, read stage
// st + 1, multiply.  Loads run kDStages - 2 steps ahead.  Packed weights only.
constexpr int kDStages = 4;
constexpr int kDW = kWN * 32 * 2;   // 32 KiB: 512 weight rows x 32 K
constexpr int kDX = kTM * 32 * 2;   // 8 KiB: 128 token rows x 32 K
constexpr int kDLoads = 10;         // loads per wave and step: 8 weight panels, 2 activation tiles

template <int MODE, bool OUTF32>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ffn_wdma_kernel(TiledArgs ta) {
  const StreamArgs& a = ta.s;
  __shared__ __attribute__((aligned(16))) char w0s[kDW];
  __shared__ __attribute__((aligned(16))) char w1s[kDW];
  __shared__ __attribute__((aligned(16))) char w2s[kDW];
  __shared__ __attribute__((aligned(16))) char w3s[kDW];
  __shared__ __attribute__((aligned(16))) char x0s[kDX];
  __shared__ __attribute__((aligned(16))) char x1s[kDX];
  __shared__ __attribute__((aligned(16))) char x2s[kDX];
  __shared__ __attribute__((aligned(16))) char x3s[kDX];

  TileWork tw;
  if (!decode_work(ta, tw)) return;
  const int g = tw.g, nt = tw.nt, c0 = tw.c0, R = tw.R;
  const int64_t s0 = tw.s0, s1 = tw.s1;
  const bool shared = tw.shared;
  // a work item is a kTileRows-row tile: its 128-row halves in turn
  for (int half = 0; half < kTileRows / kTM; ++half) {
    const int m0 = tw.mt * kTileRows + half * kTM;   // first row of this half within the group
    if (m0 >= R) break;
    if (half) __syncthreads();             // the previous half is done with the LDS

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Kdim = a.Kdim;
    const int ks = blockIdx.z;
    const int kper = Kdim / a.ksplit;
    const int kc0 = ks * kper / 32;
    const int nsteps = kper / 32;

    const int n0 = MODE == MODE_GATEUP ? nt * (kWN / 2) : nt * kWN;
    const char* Wa;
    const char* Wb = nullptr;
    if (shared) { Wa = static_cast<const char*>(a.SW); Wb = static_cast<const char*>(a.SW3); }
    else {
      Wa = static_cast<const char*>(a.W) + (int64_t)g * a.N * Kdim * 2;
      if (MODE == MODE_GATEUP) Wb = static_cast<const char*>(a.W3) + (int64_t)g * a.N * Kdim * 2;
    }
    const uint32_t wbytes = (uint32_t)a.N * Kdim * 2;
    // the weight panels this wave loads: p = 8 * wave + i; for gate/up panels
    // 0..15 are W1 rows n0 + 16 p, panels 16..31 the same rows of W3
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(MODE == MODE_GATEUP && wave >= 2 ? Wb : Wa, wbytes);
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(a.X, (uint32_t)ta.x_bytes);
    uint32_t pw[8];
  #pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = 8 * wave + i;
      const int row0 = MODE == MODE_GATEUP ? n0 + 16 * (p & 15) : n0 + 16 * p;
      pw[i] = (uint32_t)(row0 / 16) * 16 * 128 * 2 + lane * 16;
    }
    auto wk = [&](int kc) -> uint32_t { return (uint32_t)(kc >> 2) * (a.N / 16) * 4096 + (kc & 3) * 1024; };
    // activation tiles this wave loads: wave + 4 q (row m0 + 16 (wave + 4 q) + lane % 16)
    uint32_t xoff[2];
  #pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int gr = m0 + (wave + 4 * q) * 16 + (lane & 15);
      int64_t row = gr < c0 ? s0 + gr : (gr < R ? s1 + (gr - c0) : s0);   // pad rows read a valid row
      if (a.gather_src) {
        const int rank = gr < R ? gr : 0;
        row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
      }
      xoff[q] = (uint32_t)(row * a.ldx * 2) + 16 * (lane >> 4);
    }

    const int rows_here = min(kTM, R - m0);
    const int mv = ((rows_here + 31) / 32) * 2;
    auto run = [&](auto mvc) {
      constexpr int MV = decltype(mvc)::value;
      // loads of step st (clamped past the end: re-read, never multiplied) into stage S
      auto issue = [&](auto sc, int st) {
        constexpr int S = decltype(sc)::value;
        char* ws = S == 0 ? w0s : S == 1 ? w1s : S == 2 ? w2s : w3s;
        char* xs = S == 0 ? x0s : S == 1 ? x1s : S == 2 ? x2s : x3s;
        const int stc = st < nsteps ? st : nsteps - 1;
        const uint32_t wso = wk(kc0 + stc);
  #pragma unroll
        for (int i = 0; i < 8; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, ws + (8 * wave + i) * 1024, 16, pw[i], wso, 0, 0);
        const uint32_t xso = (uint32_t)(kc0 + stc) * 64;
  #pragma unroll
        for (int q = 0; q < 2; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, xs + (wave + 4 * q) * 1024, 16, xoff[q], xso, 0, 0);
      };
      f32x4 acc[MV][8];
  #pragma unroll
      for (int m = 0; m < MV; ++m)
  #pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
      // fragments of one stage: 8 weight panels, then MV activation tiles
      bf16x8 fa[8 + MV], fb[8 + MV];
      auto readf = [&](auto sc, bf16x8* f) {
        constexpr int S = decltype(sc)::value;
        const char* ws = S == 0 ? w0s : S == 1 ? w1s : S == 2 ? w2s : w3s;
        const char* xs = S == 0 ? x0s : S == 1 ? x1s : S == 2 ? x2s : x3s;
  #pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int p = MODE == MODE_GATEUP ? (n < 4 ? 4 * wave + n : 16 + 4 * wave + (n - 4)) : 8 * wave + n;
          f[n] = *reinterpret_cast<const bf16x8*>(ws + p * 1024 + lane * 16);
        }
  #pragma unroll
        for (int m = 0; m < MV; ++m) f[8 + m] = *reinterpret_cast<const bf16x8*>(xs + m * 1024 + lane * 16);
      };
      auto mma = [&](const bf16x8* f) {
  #pragma unroll
        for (int m = 0; m < MV; ++m)
  #pragma unroll
          for (int n = 0; n < 8; ++n) acc[m][n] = mfma16x16x32(f[n], f[8 + m], acc[m][n]);
      };
      // s_waitcnt immediates (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4
      // and lgkmcnt 11:8 left at their maxima
      constexpr int kVm0 = (kDStages - 2) * kDLoads;   // stage 0 landed, stages 1 and 2 may run
      constexpr int kVm = (kDStages - 3) * kDLoads;    // the next stage landed, the one after may run
      constexpr int kWait0 = (kVm0 & 15) | ((kVm0 >> 4) << 14) | 0x70 | 0xF00;
      constexpr int kWaitNext = (kVm & 15) | ((kVm >> 4) << 14) | 0x70 | 0xF00;
      issue(IntC<0>{}, 0);
      issue(IntC<1>{}, 1);
      issue(IntC<2>{}, 2);
      __builtin_amdgcn_s_waitcnt(kWait0);
      __builtin_amdgcn_s_barrier();
      readf(IntC<0>{}, fa);
      // step st: its fragments are in registers (read during the previous
      // step); read the next stage's fragments while its MFMAs run
      // (the scheduling barriers keep each step's MFMAs between its own
      // s_barrier and the next one: MFMAs touch no memory, and the scheduler
      // would otherwise sink them below the next wait)
      auto step = [&](auto nc, auto rc, bf16x8* cur, bf16x8* nxt, int st) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitNext);   // this wave's loads of stage st + 1 landed
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): fragments of step st are in registers
        __builtin_amdgcn_s_barrier();            // every wave's: stage st + 1 readable, stage st - 1 free
        issue(nc, st + kDStages - 1);
        if (st + 1 < nsteps) readf(rc, nxt);
        if (st < nsteps) mma(cur);
        __builtin_amdgcn_sched_barrier(0);
      };
      for (int sb = 0; sb < nsteps; sb += kDStages) {
        step(IntC<3>{}, IntC<1>{}, fa, fb, sb);
        step(IntC<0>{}, IntC<2>{}, fb, fa, sb + 1);
        step(IntC<1>{}, IntC<3>{}, fa, fb, sb + 2);
        step(IntC<2>{}, IntC<0>{}, fb, fa, sb + 3);
      }
      // no load may land in LDS after the workgroup has ended
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();

      // ---- epilogue: acc[m][n] holds D[w-row 4*(lane/16)+j of tile n][token lane%16 of tile m]
      const int lr = lane & 15, lg = lane >> 4;
  #pragma unroll
      for (int m = 0; m < MV; ++m) {
        const int gr = m0 + m * 16 + lr;
        if (gr >= R) continue;
        const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
        if (MODE == MODE_GATEUP) {
  #pragma unroll
          for (int n = 0; n < 4; ++n) {
            const f32x4 gt = acc[m][n], up = acc[m][n + 4];
            const int ncol = n0 + 64 * wave + 16 * n + 4 * lg;
            u32x2 o = {pack_bf16x2(silu_t(gt.x) * up.x, silu_t(gt.y) * up.y),
                       pack_bf16x2(silu_t(gt.z) * up.z, silu_t(gt.w) * up.w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
          }
        } else {
  #pragma unroll
          for (int n = 0; n < 8; ++n) {
            const int ncol = n0 + 128 * wave + 16 * n + 4 * lg;
            if constexpr (OUTF32) {
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol) = acc[m][n];
            } else {
              u32x2 o = {pack_bf16x2(acc[m][n].x, acc[m][n].y), pack_bf16x2(acc[m][n].z, acc[m][n].w)};
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
            }
          }
        }
      }
    };
    switch (mv) {
      case 2: run(IntC<2>{}); break;
      case 4: run(IntC<4>{}); break;
      case 6: run(IntC<6>{}); break;
      default: run(IntC<8>{}); break;
    }
  }
}

// ---- wide tile, weights straight to registers, activations through LDS --------
//
// The tile, the waves' outputs and the MFMA order are ffn_wdma_kernel's (so
// the results are the same bit for bit).  A weight fragment is read by one
// wave only, so weights skip LDS: each wave loads its 8 weight fragments of a
// step into one of two register banks, two steps ahead.  Only the activation
// tile, which all four waves read, goes through LDS, by direct-to-LDS loads
// into a ring of kHStages stages (three steps ahead); the MFMAs of each
// activation tile wait only for that tile's LDS read.  LDS traffic per step
// and workgroup falls from 104 KiB (40 KiB written, 64 KiB read) to 40 KiB.
// The launch guarantees nsteps % 4 == 0.  Packed weights only.
constexpr int kHStages = 4;

template <int MODE, bool OUTF32>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ffn_whyb_kernel(TiledArgs ta) {
  const StreamArgs& a = ta.s;
  __shared__ __attribute__((aligned(16))) char x0s[kDX];
  __shared__ __attribute__((aligned(16))) char x1s[kDX];
  __shared__ __attribute__((aligned(16))) char x2s[kDX];
  __shared__ __attribute__((aligned(16))) char x3s[kDX];

  TileWork tw;
  if (!decode_work(ta, tw)) return;
  const int g = tw.g, nt = tw.nt, c0 = tw.c0, R = tw.R;
  const int64_t s0 = tw.s0, s1 = tw.s1;
  const bool shared = tw.shared;
  // a work item is a kTileRows-row tile: its 128-row halves in turn
  for (int half = 0; half < kTileRows / kTM; ++half) {
    const int m0 = tw.mt * kTileRows + half * kTM;   // first row of this half within the group
    if (m0 >= R) break;
    if (half) __syncthreads();             // the previous half is done with the LDS

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Kdim = a.Kdim;
    const int ks = blockIdx.z;
    const int kper = Kdim / a.ksplit;
    const int kc0 = ks * kper / 32;
    const int nsteps = kper / 32;

    const int n0 = MODE == MODE_GATEUP ? nt * (kWN / 2) : nt * kWN;
    const char* Wa;
    const char* Wb = nullptr;
    if (shared) { Wa = static_cast<const char*>(a.SW); Wb = static_cast<const char*>(a.SW3); }
    else {
      Wa = static_cast<const char*>(a.W) + (int64_t)g * a.N * Kdim * 2;
      if (MODE == MODE_GATEUP) Wb = static_cast<const char*>(a.W3) + (int64_t)g * a.N * Kdim * 2;
    }
    const uint32_t wbytes = (uint32_t)a.N * Kdim * 2;
    const __amdgpu_buffer_rsrc_t wra = buffer_rsrc(Wa, wbytes);
    const __amdgpu_buffer_rsrc_t wrb = buffer_rsrc(MODE == MODE_GATEUP ? Wb : Wa, wbytes);
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(a.X, (uint32_t)ta.x_bytes);
    // weight fragment n of this wave: GATEUP n < 4 W1 rows n0 + 64 w + 16 n,
    // n >= 4 the same rows of W3; DOWN W2 rows n0 + 128 w + 16 n
    uint32_t pw[8];
  #pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int row0 = MODE == MODE_GATEUP ? n0 + 64 * wave + 16 * (n & 3) : n0 + 128 * wave + 16 * n;
      pw[n] = (uint32_t)(row0 / 16) * 16 * 128 * 2 + lane * 16;
    }
    auto wk = [&](int kc) -> uint32_t { return (uint32_t)(kc >> 2) * (a.N / 16) * 4096 + (kc & 3) * 1024; };
    uint32_t xoff[2];
  #pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int gr = m0 + (wave + 4 * q) * 16 + (lane & 15);
      int64_t row = gr < c0 ? s0 + gr : (gr < R ? s1 + (gr - c0) : s0);   // pad rows read a valid row
      if (a.gather_src) {
        const int rank = gr < R ? gr : 0;
        row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
      }
      xoff[q] = (uint32_t)(row * a.ldx * 2) + 16 * (lane >> 4);
    }

    const int rows_here = min(kTM, R - m0);
    const int mv = ((rows_here + 31) / 32) * 2;
    auto run = [&](auto mvc) {
      constexpr int MV = decltype(mvc)::value;
      // activation loads of step st (clamped past the end) into stage S
      auto issue_x = [&](auto sc, int st) {
        constexpr int S = decltype(sc)::value;
        char* xs = S == 0 ? x0s : S == 1 ? x1s : S == 2 ? x2s : x3s;
        const int stc = st < nsteps ? st : nsteps - 1;
        const uint32_t xso = (uint32_t)(kc0 + stc) * 64;
  #pragma unroll
        for (int q = 0; q < 2; ++q)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, xs + (wave + 4 * q) * 1024, 16, xoff[q], xso, 0, 0);
      };
      // weight fragments of step st (clamped) into a register bank
      auto load_w = [&](bf16x8* wb, int st) {
        const int stc = st < nsteps ? st : nsteps - 1;
        const uint32_t wso = wk(kc0 + stc);
  #pragma unroll
        for (int n = 0; n < 8; ++n)
          wb[n] = __builtin_bit_cast(bf16x8, buffer_load16(MODE == MODE_GATEUP && n >= 4 ? wrb : wra, pw[n], wso));
      };
      auto read_x = [&](auto sc, bf16x8* f) {
        constexpr int S = decltype(sc)::value;
        const char* xs = S == 0 ? x0s : S == 1 ? x1s : S == 2 ? x2s : x3s;
  #pragma unroll
        for (int m = 0; m < MV; ++m) f[m] = *reinterpret_cast<const bf16x8*>(xs + m * 1024 + lane * 16);
      };
      f32x4 acc[MV][8];
  #pragma unroll
      for (int m = 0; m < MV; ++m)
  #pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
      bf16x8 w0[8], w1[8];   // weight banks of steps st and st + 1
      bf16x8 xf[MV];         // activation fragments of step st
      // Issue order: A0 A1 W0 A2 W1 (A: a step's activation stage, W: its
      // weights), then per step st: A(st + 3), and after its MFMAs W(st + 2).
      // At the top of step st the loads issued after A(st) are at most W(st-1)
      // A(st+1) W(st) A(st+2) W(st+1), of which W(st-1) has already been
      // waited for: vmcnt(20) means stage st has landed (exactly so at st = 0).
      issue_x(IntC<0>{}, 0);
      issue_x(IntC<1>{}, 1);
      load_w(w0, 0);
      issue_x(IntC<2>{}, 2);
      load_w(w1, 1);
      constexpr int kVm = 2 * 8 + 2 * 2;
      constexpr int kWait = (kVm & 15) | ((kVm >> 4) << 14) | 0x70 | 0xF00;
      auto step = [&](auto sc, auto nc, bf16x8* wc, int st) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWait);       // this wave's loads of stage st landed
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): its reads of stage st - 1 are done
        __builtin_amdgcn_s_barrier();            // every wave's: stage st readable, stage st - 1 free
        issue_x(nc, st + kHStages - 1);
        read_x(sc, xf);
        __builtin_amdgcn_sched_barrier(0);       // every read issued before the first MFMA
  #pragma unroll
        for (int m = 0; m < MV; ++m)
  #pragma unroll
          for (int n = 0; n < 8; ++n) acc[m][n] = mfma16x16x32(wc[n], xf[m], acc[m][n]);
        // the bank's next weights only after its last MFMA (else a third bank)
        __builtin_amdgcn_sched_barrier(0);
        load_w(wc, st + 2);
        __builtin_amdgcn_sched_barrier(0);
      };
      for (int sb = 0; sb < nsteps; sb += 4) {
        step(IntC<0>{}, IntC<3>{}, w0, sb);
        step(IntC<1>{}, IntC<0>{}, w1, sb + 1);
        step(IntC<2>{}, IntC<1>{}, w0, sb + 2);
        step(IntC<3>{}, IntC<2>{}, w1, sb + 3);
      }
      // no load may land in LDS after the workgroup has ended
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();

      // ---- epilogue: acc[m][n] holds D[w-row 4*(lane/16)+j of tile n][token lane%16 of tile m]
      const int lr = lane & 15, lg = lane >> 4;
  #pragma unroll
      for (int m = 0; m < MV; ++m) {
        const int gr = m0 + m * 16 + lr;
        if (gr >= R) continue;
        const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
        if (MODE == MODE_GATEUP) {
  #pragma unroll
          for (int n = 0; n < 4; ++n) {
            const f32x4 gt = acc[m][n], up = acc[m][n + 4];
            const int ncol = n0 + 64 * wave + 16 * n + 4 * lg;
            u32x2 o = {pack_bf16x2(silu_t(gt.x) * up.x, silu_t(gt.y) * up.y),
                       pack_bf16x2(silu_t(gt.z) * up.z, silu_t(gt.w) * up.w)};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
          }
        } else {
  #pragma unroll
          for (int n = 0; n < 8; ++n) {
            const int ncol = n0 + 128 * wave + 16 * n + 4 * lg;
            if constexpr (OUTF32) {
              *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol) = acc[m][n];
            } else {
              u32x2 o = {pack_bf16x2(acc[m][n].x, acc[m][n].y), pack_bf16x2(acc[m][n].z, acc[m][n].w)};
              *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row * a.ldo + ncol) = o;
            }
          }
        }
      }
    };
    switch (mv) {
      case 2: run(IntC<2>{}); break;
      case 4: run(IntC<4>{}); break;
      case 6: run(IntC<6>{}); break;
      default: run(IntC<8>{}); break;
    }
  }
}

// ---- tall tile: 256 token rows x 256 weight rows, every wave all 256 rows ------
//
// A work item is a whole kTileRows-row tile, so the weights of an expert of up
// to 256 rows (the average prefill group) are read by one workgroup, once,
// where the 128-row kernels above read them once per 128-row half.  Each wave
// owns all 256 token rows x 64 weight rows (16 x 4 MFMA tiles, the 256
// accumulator registers of a wave alone on its SIMD), so a tile that is only
// partly full shortens every wave alike: no wave idles at the barriers while
// another computes.  The cost is operand traffic from LDS: every wave reads
// the whole activation tile (256 rows x 64 K = 32 KiB a 64-wide stage), each
// fragment feeding four MFMAs.
//  * Weights go straight to registers (each weight fragment is read by one
//    wave only): per 64-wide K stage 8 fragments (4 panels x two 32-wide
//    steps) into one of two banks, two stages ahead.
//  * Activations go by direct-to-LDS loads into a ring of kQStages stages of
//    32 KiB, three stages ahead: 16 row tiles x two 32-wide steps of 1 KiB
//    each in MFMA fragment order, each wave loading four row tiles.
//  * Per output element the K range is reduced in 32-wide MFMA steps in
//    ascending order with the same instruction as the other kernels, so the
//    results are the same bit for bit.
// The launch needs packed weights and a K range of whole blocks of four
// 64-wide stages.
constexpr int kQM = kTileRows;        // token rows per tile (256)
constexpr int kQMT = kQM / 16;        // 16-row MFMA tiles per tile
constexpr int kQStages = 4;           // LDS ring of 64-wide K stages
constexpr int kQStage = kQM * 64 * 2; // 32 KiB a stage
constexpr int kQN = 256;              // weight rows per tile
constexpr int kQAhead = 2;            // row tiles whose fragments are read ahead of their MFMAs
// cache policy of the weight loads (buffer instruction aux bits; 0 = the
// default, cached; 2 = nt on gfx950).  A group's row tiles read the same
// weights close together in time, and the later reads find them in L2 or in
// the memory-side cache only if the first read allocated them there.
#ifndef MOE_TALL_WEIGHT_POLICY
#define MOE_TALL_WEIGHT_POLICY 0
#endif
constexpr int kWeightPolicy = MOE_TALL_WEIGHT_POLICY;
static_assert(kQM == 256, "the tall tile is one work item");

struct NoHook {
  __device__ void operator()() const {}
};

// One work item: rows m0 = 256 mt .. of group g against weight-row tile nt.
// The activation ring is four LDS arrays, one per stage slot, rather than one
// array with offsets: the compiler then tells a direct-to-LDS load into one
// slot from a read of another and does not make the read wait for every
// load in flight.  at_loop_end() runs once the K loop is done, before the
// epilogue (the persistent schedule claims its next unit there, so the
// claim's latency overlaps the epilogue's arithmetic).
template <int MODE, bool OUTF32, typename Hook = NoHook>
__device__ __forceinline__ void tall_tile(const TiledArgs& ta, const TileWork& tw, char* x0s, char* x1s,
                                          char* x2s, char* x3s, Hook at_loop_end = Hook{}) {
  const StreamArgs& a = ta.s;
  const int g = tw.g, nt = tw.nt, c0 = tw.c0, R = tw.R;
  const int64_t s0 = tw.s0, s1 = tw.s1;
  const bool shared = tw.shared;
  const int m0 = tw.mt * kQM;                // first row of the tile within the group

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kdim = a.Kdim;
  const int ks = blockIdx.z;
  const int kper = Kdim / a.ksplit;
  const int kc0 = ks * kper / 32;            // first 32-wide K chunk
  const int nst = kper / 64;                 // 64-wide stages

  // weight panels of this wave: GATEUP W1 rows n0 + 32 w + 16 j (j = 0, 1) and
  // the same rows of W3 (fragments 2, 3); DOWN W2 rows n0 + 64 w + 16 j
  const int n0 = MODE == MODE_GATEUP ? nt * (kQN / 2) : nt * kQN;
  const char* Wa;
  const char* Wb = nullptr;
  if (shared) { Wa = static_cast<const char*>(a.SW); Wb = static_cast<const char*>(a.SW3); }
  else {
    Wa = static_cast<const char*>(a.W) + (int64_t)g * a.N * Kdim * 2;
    if (MODE == MODE_GATEUP) Wb = static_cast<const char*>(a.W3) + (int64_t)g * a.N * Kdim * 2;
  }
  const uint32_t wbytes = (uint32_t)a.N * Kdim * 2;
  const __amdgpu_buffer_rsrc_t wra = buffer_rsrc(Wa, wbytes);
  const __amdgpu_buffer_rsrc_t wrb = buffer_rsrc(MODE == MODE_GATEUP ? Wb : Wa, wbytes);
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(a.X, (uint32_t)ta.x_bytes);
  uint32_t pw[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row0 = MODE == MODE_GATEUP ? n0 + 32 * wave + 16 * (n & 1) : n0 + 64 * wave + 16 * n;
    pw[n] = (uint32_t)(row0 / 16) * 16 * 128 * 2 + lane * 16;
  }
  // byte offset of 32-wide K chunk kc in the packed (step-major) layout
  auto wk = [&](int kc) -> uint32_t { return (uint32_t)(kc >> 2) * (a.N / 16) * 4096 + (kc & 3) * 1024; };
  // activation row tiles this wave loads: wave + 4 q (row m0 + 16 (wave + 4 q) + lane % 16);
  // rows past the group read a valid row, never used
  uint32_t xoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int gr = m0 + (wave + 4 * q) * 16 + (lane & 15);
    int64_t row = gr < c0 ? s0 + gr : (gr < R ? s1 + (gr - c0) : s0);
    if (a.gather_src) {
      const int rank = gr < R ? gr : 0;
      row = shared ? rank : a.gather_src[a.gather_off[g] + rank];
    }
    xoff[q] = (uint32_t)(row * a.ldx * 2) + 16 * (lane >> 4);
  }

  const int rows_here = min(kQM, R - m0);
  const int mv = ((rows_here + 31) / 32) * 2;   // non-empty 16-row tiles, in pairs
  auto run = [&](auto mvc) -> void {
    constexpr int MV = decltype(mvc)::value;
    auto slot = [&](auto sc) -> char* {
      constexpr int S = decltype(sc)::value;
      return S == 0 ? x0s : S == 1 ? x1s : S == 2 ? x2s : x3s;
    };
    // activations of stage st (clamped past the end: re-read, never used) into ring slot S
    auto issue_x = [&](auto sc, int st) -> void {
      const int stc = st < nst ? st : nst - 1;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, slot(sc) + ((wave + 4 * q) * 2 + j) * 1024, 16, xoff[q],
                                                   (uint32_t)(kc0 + 2 * stc + j) * 64, 0, 0);
    };
    // one of the stage's 16 loads of this wave: pieces 0..7 activations (row
    // tile wave + 4 (i / 2), step i % 2) into LDS slot S, 8..15 weights
    // (panel (i - 8) / 2, step i % 2) into bank b
    auto issue_piece = [&](int i, auto sc, bf16x8* b, int st) -> void {
      const int stc = st < nst ? st : nst - 1;
      const int j = i & 1;
      if (i < 8) {
        const int q = i >> 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, slot(sc) + ((wave + 4 * q) * 2 + j) * 1024, 16, xoff[q],
                                                 (uint32_t)(kc0 + 2 * stc + j) * 64, 0, 0);
      } else {
        const int n = (i - 8) >> 1;
        b[2 * n + j] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(MODE == MODE_GATEUP && n >= 2 ? wrb : wra, (int)pw[n],
                                                           (int)wk(kc0 + 2 * stc + j), kWeightPolicy));
      }
    };
    // weights of stage st (clamped) into a bank: fragment 2 n + j = panel n,
    // step j (cache policy kWeightPolicy)
    auto load_w = [&](bf16x8* wb, int st) -> void {
      const int stc = st < nst ? st : nst - 1;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wb[2 * n + j] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(MODE == MODE_GATEUP && n >= 2 ? wrb : wra,
                                                             (int)pw[n], (int)wk(kc0 + 2 * stc + j), kWeightPolicy));
    };
    f32x4 acc[MV][4];
#pragma unroll
    for (int m = 0; m < MV; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    // weight banks: stage st multiplies bank st % 4 while the weights of
    // stages st + 1 .. st + 3 are in flight in the others
    bf16x8 wbank[kQStages][8];
    // Issue order A0 W0 A1 W1 A2 W2, then during stage st the 16 loads of
    // stage st + 3, one after each row tile's MFMAs (A: a stage's 8
    // activation loads into LDS, W: this wave's 8 weight loads): spread over
    // the stage, a load never waits long to issue while the MFMAs stand
    // behind it (a wave issues in order; a burst of 16 at the top of a stage
    // filled the address unit's queue and stalled the wave for hundreds of
    // cycles).  At the top of stage st the loads issued after stage st's are
    // those of st + 1 and st + 2, so vmcnt(32) means this wave's loads of
    // stage st (both kinds) have landed; the barrier then makes every
    // wave's activation loads of stage st visible.
    issue_x(IntC<0>{}, 0);
    load_w(wbank[0], 0);
    issue_x(IntC<1>{}, 1);
    load_w(wbank[1], 1);
    issue_x(IntC<2>{}, 2);
    load_w(wbank[2], 2);
    constexpr int kVm = 32;
    constexpr int kWait = (kVm & 15) | ((kVm >> 4) << 14) | 0x70 | 0xF00;
    auto stage = [&](auto sc, auto nc, int st) -> void {
      constexpr int S = decltype(sc)::value;
      constexpr int NS = decltype(nc)::value;
      bf16x8* wc = wbank[S];
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWait);       // this wave's loads of stage st landed
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): its reads of stage st - 1 are done
      __builtin_amdgcn_s_barrier();            // every wave's: stage st readable, slot of st - 1 free
      // row tile m's two fragments are read while tile m - kQAhead's MFMAs
      // run; the scheduling fences keep the reads from all moving ahead (32
      // fragments would not fit in the registers beside the accumulators)
      const char* xs = slot(sc);
      bf16x8 xf[kQAhead + 1][2];
#pragma unroll
      for (int m = 0; m < kQAhead; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          xf[m][j] = *reinterpret_cast<const bf16x8*>(xs + (m * 2 + j) * 1024 + lane * 16);
      // 16 row-tile slots: the MFMAs of the tiles present, and one load of
      // stage st + 3 per slot (into LDS slot NS and the bank of stage st - 1,
      // both free now)
#pragma unroll
      for (int m = 0; m < kQMT; ++m) {
        if (m < MV) {
          if (m + kQAhead < MV) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              xf[(m + kQAhead) % (kQAhead + 1)][j] =
                  *reinterpret_cast<const bf16x8*>(xs + ((m + kQAhead) * 2 + j) * 1024 + lane * 16);
          }
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8* x = xf[m % (kQAhead + 1)];
          // both 32-wide steps of every panel, the first step of all four first
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int n = 0; n < 4; ++n) mfma_acc(acc[m][n], wc[2 * n + j], x[j]);
        }
        issue_piece(m, nc, wbank[NS], st + kQStages - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the loop may end after this stage: the compiler places moves of
      // accumulators at the loop exit, before any code after the loop, and it
      // cannot see that these registers are still being written by the
      // products above, so the wait states go here
      if constexpr (S == kQStages - 1) acc_fence();
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int sb = 0; sb < nst; sb += kQStages) {
      stage(IntC<0>{}, IntC<3>{}, sb);
      stage(IntC<1>{}, IntC<0>{}, sb + 1);
      stage(IntC<2>{}, IntC<1>{}, sb + 2);
      stage(IntC<3>{}, IntC<2>{}, sb + 3);
    }
    // no load may land in LDS after the workgroup has ended
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    acc_fence();
    at_loop_end();

    // ---- epilogue: acc[m][n] holds D[w-row 4*(lane/16)+j of panel n][token lane%16 of tile m]
    const int lr = lane & 15, lg = lane >> 4;
    if constexpr (OUTF32) {
      // fp32 partial planes (a K split): each lane stores its own 16 bytes
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        const int gr = m0 + m * 16 + lr;
        if (gr >= R) continue;
        const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int ncol = n0 + 64 * wave + 16 * n + 4 * lg;
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ks * a.split_stride + row * a.ldo + ncol) = acc[m][n];
        }
      }
    } else {
      // bf16 outputs go through LDS (the ring is free now): every lane writes
      // its values unconditionally, then the workgroup stores whole 16-byte
      // pieces of the valid rows.  Per-row conditional stores straight from
      // the accumulators split the code into a block per row tile, and the
      // compiler then moved every accumulator at the join.
      // LDS tile: row r (0..MV*16-1) of kOutCols bf16 in ring slot r / kSlotRows,
      // 16-byte pieces rotated by the row against bank conflicts
      constexpr int kOutCols = MODE == MODE_GATEUP ? kQN / 2 : kQN;   // h: 128, y: 256 columns
      constexpr int kPieces = kOutCols / 8;                            // 16-byte pieces per row
      constexpr int kSlotRows = kQStage / (kOutCols * 2);              // rows per 32 KiB slot
      auto piece_ptr = [&](int r, int pc) -> uint16_t* {
        const int sl = r / kSlotRows;
        char* base = sl == 0 ? x0s : sl == 1 ? x1s : sl == 2 ? x2s : x3s;
        return reinterpret_cast<uint16_t*>(base) + (r % kSlotRows) * kOutCols + ((pc + r) % kPieces) * 8;
      };
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        // one row tile at a time: read all at once, the accumulators would
        // need as many ordinary registers again
        __builtin_amdgcn_sched_barrier(0);
        const int r = m * 16 + lr;
        if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const f32x4 gt = acc[m][n], up = acc[m][n + 2];
            const int col = 32 * wave + 16 * n + 4 * lg;        // within the tile's 128 columns
            const u32x2 o = {pack_bf16x2(silu_t(gt.x) * up.x, silu_t(gt.y) * up.y),
                             pack_bf16x2(silu_t(gt.z) * up.z, silu_t(gt.w) * up.w)};
            *reinterpret_cast<u32x2*>(piece_ptr(r, col / 8) + col % 8) = o;
          }
        } else {
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int col = 64 * wave + 16 * n + 4 * lg;
            const u32x2 o = {pack_bf16x2(acc[m][n].x, acc[m][n].y), pack_bf16x2(acc[m][n].z, acc[m][n].w)};
            *reinterpret_cast<u32x2*>(piece_ptr(r, col / 8) + col % 8) = o;
          }
        }
      }
      __syncthreads();
      const int rows = min(rows_here, MV * 16);
      for (int i = tid; i < rows * kPieces; i += kTThreads) {
        const int r = i / kPieces, pc = i % kPieces;
        const int gr = m0 + r;
        const int64_t row = gr < c0 ? s0 + gr : s1 + (gr - c0);
        const u32x4 v = *reinterpret_cast<const u32x4*>(piece_ptr(r, pc));
        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.out) + row * a.ldo + n0 + pc * 8) = v;
      }
      __syncthreads();             // the next item's loads refill this LDS
    }
  };
  switch (mv) {
    case 2: run(IntC<2>{}); break;
    case 4: run(IntC<4>{}); break;
    case 6: run(IntC<6>{}); break;
    case 8: run(IntC<8>{}); break;
    case 10: run(IntC<10>{}); break;
    case 12: run(IntC<12>{}); break;
    case 14: run(IntC<14>{}); break;
    default: run(IntC<16>{}); break;
  }
}

// PERSIST: the claim schedule of claim_units(), one workgroup per compute
// unit; else one workgroup per work item (decode_work).
template <int MODE, bool OUTF32, bool PERSIST>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ffn_tall_kernel(TiledArgs ta) {
  __shared__ __attribute__((aligned(16))) char x0s[kQStage];
  __shared__ __attribute__((aligned(16))) char x1s[kQStage];
  __shared__ __attribute__((aligned(16))) char x2s[kQStage];
  __shared__ __attribute__((aligned(16))) char x3s[kQStage];
  static_assert(kQStages == 4, "four ring slots");
  if constexpr (!PERSIST) {
    TileWork tw;
    if (!decode_work(ta, tw)) return;
    tall_tile<MODE, OUTF32>(ta, tw, x0s, x1s, x2s, x3s);
  } else {
    const int ntn = ta.s.N / (MODE == MODE_GATEUP ? kQN / 2 : kQN);   // weight tiles per row tile
    claim_units<kTThreads>(ta.s, ta.tile_off, ta.claim, ntn, [&](const TileWork& tw, auto at_loop_end) {
      tall_tile<MODE, OUTF32>(ta, tw, x0s, x1s, x2s, x3s, at_loop_end);
    });
  }
}

// The tall kernel: packed weights, N in whole tiles, a K range of whole blocks
// of four 64-wide stages, 32-bit buffer offsets.
bool tall_supported(int mode, const TiledArgs& a) {
  if (a.s.N % (mode == MODE_GATEUP ? kQN / 2 : kQN)) return false;
  const int kper = a.s.Kdim / a.s.ksplit;
  if (kper % (64 * kQStages) || kper <= 0) return false;
  return (int64_t)a.s.N * a.s.Kdim * 2 < (int64_t(1) << 31) && a.x_bytes > 0 &&
         a.x_bytes < (int64_t(1) << 31);
}

// compute units of the current device (0 if the query fails), asked once per device
int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

bool tiled_supported(int mode, int fp8, int N, int Kdim, int ksplit) {
  if (fp8) return false;
  if (mode == MODE_GATEUP) { if (N % 128) return false; }
  else if (N % kTN) return false;
  return (Kdim / ksplit) % kTK == 0;
}

// The wide kernel addresses one weight matrix and the activation rows through
// 32-bit buffer offsets: both must stay below 2 GiB.
bool wide_supported(int mode, const TiledArgs& a) {
  if (a.s.N % (mode == MODE_GATEUP ? kWN / 2 : kWN)) return false;
  if ((a.s.Kdim / a.s.ksplit) % 32) return false;   // whole 32-wide steps (a pass may end early)
  return (int64_t)a.s.N * a.s.Kdim * 2 < (int64_t(1) << 31) && a.x_bytes > 0 &&
         a.x_bytes < (int64_t(1) << 31);
}

// Which kernel takes a launch.  a.variant (moe_desc_t.debug_flags) can force
// one; where the forced one does not apply to the shape the choice falls to
// the next one down.  Packed weights: by default the tall tile where it
// applies, then the hybrid tile (weights to registers, activations by
// direct-to-LDS loads) where the K range is whole blocks of four 32-wide
// steps, else the all-LDS one; row-major weights: the register-staged wide
// tile; shapes the wide tile does not divide: the narrow one.
int tiled_choice(const TiledArgs& a, int packed, int mode) {
  if (packed && (a.variant == 0 || a.variant == MOE_DEBUG_TILED_TALL) && tall_supported(mode, a))
    return MOE_DEBUG_TILED_TALL;
  const bool wide = wide_supported(mode, a) && a.variant != MOE_DEBUG_TILED_NARROW;
  if (!wide) return MOE_DEBUG_TILED_NARROW;
  if (!packed || a.variant == MOE_DEBUG_TILED_WIDE_REGS) return MOE_DEBUG_TILED_WIDE_REGS;
  if (a.variant != MOE_DEBUG_TILED_WIDE_LDS && (a.s.Kdim / a.s.ksplit) % 128 == 0) return MOE_DEBUG_TILED_WIDE_HYB;
  return MOE_DEBUG_TILED_WIDE_LDS;
}

const char* tiled_kernel_name(int choice) {
  switch (choice) {
    case MOE_DEBUG_TILED_NARROW: return "ffn_tiled_kernel";
    case MOE_DEBUG_TILED_WIDE_REGS: return "ffn_wide_kernel";
    case MOE_DEBUG_TILED_WIDE_LDS: return "ffn_wdma_kernel";
    case MOE_DEBUG_TILED_WIDE_HYB: return "ffn_whyb_kernel";
    case MOE_DEBUG_TILED_TALL: return "ffn_tall_kernel";
  }
  return "none";
}

hipError_t launch_ffn_tiled(const TiledArgs& a, int fp8, int packed, int mode, int max_tiles, hipStream_t s) {
  if (!tiled_supported(mode, fp8, a.s.N, a.s.Kdim, a.s.ksplit)) return hipErrorInvalidValue;
  if (max_tiles <= 0) return hipSuccess;
  const int choice = tiled_choice(a, packed, mode);
  if (choice == MOE_DEBUG_TILED_TALL) {
    const int ntn = a.s.N / (mode == MODE_GATEUP ? kQN / 2 : kQN);
    // the persistent schedule (one workgroup per compute unit, work claimed
    // through the route table's counters) where there are counters, no K
    // split, and the order fits its LDS; else one workgroup per work item
    const int cus = device_cus();
    if (a.claim && a.s.ksplit == 1 && a.s.E_phys <= kPlanGroups && cus >= kClaimLists) {
      const dim3 grid(cus);
      if (mode == MODE_GATEUP) hipLaunchKernelGGL((ffn_tall_kernel<MODE_GATEUP, false, true>), grid, dim3(kTThreads), 0, s, a);
      else if (a.s.out_f32) hipLaunchKernelGGL((ffn_tall_kernel<MODE_DOWN, true, true>), grid, dim3(kTThreads), 0, s, a);
      else hipLaunchKernelGGL((ffn_tall_kernel<MODE_DOWN, false, true>), grid, dim3(kTThreads), 0, s, a);
      return hipGetLastError();
    }
    const dim3 grid(ntn, max_tiles + 8, a.s.ksplit);
    if (mode == MODE_GATEUP) hipLaunchKernelGGL((ffn_tall_kernel<MODE_GATEUP, false, false>), grid, dim3(kTThreads), 0, s, a);
    else if (a.s.out_f32) hipLaunchKernelGGL((ffn_tall_kernel<MODE_DOWN, true, false>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_tall_kernel<MODE_DOWN, false, false>), grid, dim3(kTThreads), 0, s, a);
    return hipGetLastError();
  }
  const bool wide = choice != MOE_DEBUG_TILED_NARROW;
  // grid.y covers the static bound on row tiles (the live count is read on the
  // device) plus 8, so that the XCD remap's largest linear id, which can pass
  // the live work count by up to 7, always has a workgroup
  const int wn = wide ? (mode == MODE_GATEUP ? kWN / 2 : kWN) : (mode == MODE_GATEUP ? 128 : kTN);
  const dim3 grid(a.s.N / wn, max_tiles + 8, a.s.ksplit);
  if (choice == MOE_DEBUG_TILED_WIDE_HYB) {
    if (mode == MODE_GATEUP) hipLaunchKernelGGL((ffn_whyb_kernel<MODE_GATEUP, false>), grid, dim3(kTThreads), 0, s, a);
    else if (a.s.out_f32) hipLaunchKernelGGL((ffn_whyb_kernel<MODE_DOWN, true>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_whyb_kernel<MODE_DOWN, false>), grid, dim3(kTThreads), 0, s, a);
    return hipGetLastError();
  }
  if (choice == MOE_DEBUG_TILED_WIDE_LDS) {
    if (mode == MODE_GATEUP) hipLaunchKernelGGL((ffn_wdma_kernel<MODE_GATEUP, false>), grid, dim3(kTThreads), 0, s, a);
    else if (a.s.out_f32) hipLaunchKernelGGL((ffn_wdma_kernel<MODE_DOWN, true>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_wdma_kernel<MODE_DOWN, false>), grid, dim3(kTThreads), 0, s, a);
    return hipGetLastError();
  }
  if (wide) {
    if (mode == MODE_GATEUP) {
      if (packed) hipLaunchKernelGGL((ffn_wide_kernel<MODE_GATEUP, true, false>), grid, dim3(kTThreads), 0, s, a);
      else hipLaunchKernelGGL((ffn_wide_kernel<MODE_GATEUP, false, false>), grid, dim3(kTThreads), 0, s, a);
    } else if (a.s.out_f32) {
      if (packed) hipLaunchKernelGGL((ffn_wide_kernel<MODE_DOWN, true, true>), grid, dim3(kTThreads), 0, s, a);
      else hipLaunchKernelGGL((ffn_wide_kernel<MODE_DOWN, false, true>), grid, dim3(kTThreads), 0, s, a);
    } else {
      if (packed) hipLaunchKernelGGL((ffn_wide_kernel<MODE_DOWN, true, false>), grid, dim3(kTThreads), 0, s, a);
      else hipLaunchKernelGGL((ffn_wide_kernel<MODE_DOWN, false, false>), grid, dim3(kTThreads), 0, s, a);
    }
  } else if (mode == MODE_GATEUP) {
    if (packed) hipLaunchKernelGGL((ffn_tiled_kernel<MODE_GATEUP, true>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<MODE_GATEUP, false>), grid, dim3(kTThreads), 0, s, a);
  } else {
    if (packed) hipLaunchKernelGGL((ffn_tiled_kernel<MODE_DOWN, true>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<MODE_DOWN, false>), grid, dim3(kTThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
