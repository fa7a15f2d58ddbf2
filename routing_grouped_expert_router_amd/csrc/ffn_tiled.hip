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
//    streaming kernel.
//  * A group's last row tile is usually partly empty (groups are 28..961
//    rows at the prefill workload): the tile is run with only its non-empty
//    32-row sub-tiles (a compile-time count, one instance per count), so no
//    MFMA, LDS read or activation load is spent on whole pad sub-tiles.
//  * Each output element accumulates its K range in 32-wide MFMA steps in
//    ascending order, exactly as the streaming kernel does, so the split of
//    groups between the two kernels does not change any bit of the result.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <int V>
struct IntC { static constexpr int value = V; };

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

template <int MODE, bool PACKED>
__global__ __launch_bounds__(kTThreads) void ffn_tiled_kernel(TiledArgs ta) {
  const StreamArgs& a = ta.s;
  __shared__ __attribute__((aligned(16))) char xsm[2 * kXStage];   // activation tile, 2 stages

  // ---- work item.  The hardware deals workgroups round-robin over the 8 XCDs
  // (linear id L goes to XCD L % 8).  The live work list -- tile_off's
  // ceil(rows/128) tiles per group times the weight-row tiles -- is cut into 8
  // contiguous chunks, one per XCD, ordered (group, weight tile, row tile), so
  // the workgroups an XCD runs together share one group's weight and
  // activation tiles in that XCD's L2.
  const int ngroups = a.E_phys + 1;
  const int ntiles_n = gridDim.x;
  const int64_t work = (int64_t)ta.tile_off[ngroups] * ntiles_n;
  const int64_t L = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t chunk = (work + 7) / 8;
  const int64_t k_in = L / 8;
  if (k_in >= chunk) return;
  const int64_t wi = (L % 8) * chunk + k_in;
  if (wi >= work) return;
  int lo = 0, hi = ngroups;                  // largest g with tile_off[g] * ntiles_n <= wi
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)ta.tile_off[mid] * ntiles_n <= wi) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mtiles = ta.tile_off[g + 1] - ta.tile_off[g];
  const int64_t o = wi - (int64_t)ta.tile_off[g] * ntiles_n;
  const int nt = int(o / mtiles);            // weight-row tile
  const int mt = int(o % mtiles);            // row tile within the group
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
  const int R = c0 + c1;
  if (R <= ta.min_rows) return;           // the streaming kernel owns this group
  const int m0 = mt * kTM;                 // first row of the tile within the group

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

bool tiled_supported(int mode, int fp8, int N, int Kdim, int ksplit) {
  if (fp8) return false;
  if (mode == MODE_GATEUP) { if (N % 128) return false; }
  else if (N % kTN) return false;
  return (Kdim / ksplit) % kTK == 0;
}

hipError_t launch_ffn_tiled(const TiledArgs& a, int fp8, int packed, int mode, int max_tiles, hipStream_t s) {
  if (!tiled_supported(mode, fp8, a.s.N, a.s.Kdim, a.s.ksplit)) return hipErrorInvalidValue;
  if (max_tiles <= 0) return hipSuccess;
  // grid.y covers the static bound on row tiles (the live count is read on the
  // device) plus 8, so that the XCD remap's largest linear id, which can pass
  // the live work count by up to 7, always has a workgroup
  const dim3 grid(mode == MODE_GATEUP ? a.s.N / 128 : a.s.N / kTN, max_tiles + 8, a.s.ksplit);
  if (mode == MODE_GATEUP) {
    if (packed) hipLaunchKernelGGL((ffn_tiled_kernel<MODE_GATEUP, true>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<MODE_GATEUP, false>), grid, dim3(kTThreads), 0, s, a);
  } else {
    if (packed) hipLaunchKernelGGL((ffn_tiled_kernel<MODE_DOWN, true>), grid, dim3(kTThreads), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<MODE_DOWN, false>), grid, dim3(kTThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
