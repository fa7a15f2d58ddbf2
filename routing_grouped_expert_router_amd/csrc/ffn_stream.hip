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
#include "stream_dev.hpp"

namespace moe {

// grid (N / 64, b_rows + E_phys + n_shared, ksplit); region B exists only
// when region A takes fewer than four tiles per pass.
// fp8 single-tile launches run two waves per SIMD (three measured slower
// with the gate/up scales held in registers)
template <bool FP8, int MTA>
constexpr int min_waves() { return (FP8 && MTA == 1) ? 2 : 1; }

// XLK: region A keeps its activations in LDS (dynamic shared memory sized by
// the launch to cover both the K range and region B's tiles).
template <bool FP8, int MODE, int MTA, bool PACKED, bool XLK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves<FP8, MTA>() * !XLK + XLK)))
void ffn_stream_kernel(StreamArgs a) {
  constexpr int TB = tiles_b<FP8>();
  constexpr int LDS = XLK ? 1 : lds_elems<(MTA < 4 && MTA < TB) ? TB : MTA>();
  __shared__ __attribute__((aligned(16))) uint16_t xs_static[LDS];
  extern __shared__ __attribute__((aligned(16))) uint16_t xs_dynamic[];
  uint16_t* xs_raw = XLK ? xs_dynamic : xs_static;
  const int ks = blockIdx.z;
  int y = blockIdx.y;
  if constexpr (MTA < 4) {
    if (y < a.b_rows) {
      const int sh = a.b_rows - a.E_phys;   // n_shared * shared_chunks rows of the shared expert
      if (y < sh) stream_group<FP8, MODE, TB, PACKED, banks_b<FP8, MODE>(), false>(a, a.E_phys, ks, y, a.shared_chunks,
                                                                          a.max_rows, a.b_max_rows, xs_raw, blockIdx.x);
      else stream_group<FP8, MODE, TB, PACKED, banks_b<FP8, MODE>(), true>(a, y - sh, ks, 0, 1, a.max_rows,
                                                                   a.b_max_rows, xs_raw, blockIdx.x);
      return;
    }
    y -= a.b_rows;
  }
  if constexpr (XLK || FP8) {
    // fp8 launches are never compacted (stream_compacts): the loop below
    // costs their variants the registers of a wave per SIMD
    if constexpr (XLK)
      stream_group<FP8, MODE, 1, PACKED, banks_xl<FP8>(), true, true>(a, y, ks, 0, 1, 0, a.max_rows, xs_raw, blockIdx.x);
    else
      stream_group<FP8, MODE, MTA, PACKED, banks_a<FP8, MODE>(), true>(a, y, ks, 0, 1, 0, a.max_rows, xs_raw, blockIdx.x);
    return;
  }
  // compact rows (a.compact_rows > 0): row y takes the y-th, (y + rows)-th,
  // ... slots with tokens, found by one forward scan of the counts (few
  // tokens, so far fewer launched rows than slots); the rows after them are
  // the shared expert.  One call site of the group body (three inlined
  // copies raised the register count and halved the occupancy).
  const int rows = a.compact_rows;
  int p = 0, k = -1, j = y;
  auto next_slot = [&]() -> int {
    for (; p < a.E_phys; ++p)
      if (a.counts[p] > 0 && ++k == j) return p;
    return -1;
  };
  int g = rows == 0 ? y : (y >= rows ? a.E_phys + (y - rows) : next_slot());
  while (g >= 0) {
    stream_group<FP8, MODE, MTA, PACKED, banks_a<FP8, MODE>(), true>(a, g, ks, 0, 1, 0, a.max_rows, xs_raw, blockIdx.x);
    if (rows == 0 || y >= rows) return;
    ++p;
    j += rows;
    g = next_slot();
    if (g >= 0) __syncthreads();         // the previous group is done with the LDS
  }
}

// fp8 down projections with one row tile per pass and a K range of at most
// kXlSteps steps keep their activations in LDS (measured: pays for fp8 with
// K = 2048, costs time for bf16)
bool stream_uses_xl(int fp8, int mode, int mt, const StreamArgs& a) {
  return fp8 && mode == MODE_DOWN && mt == 1 && a.Kdim / kKS / a.ksplit <= kXlSteps;
}

template <bool FP8, int MODE, bool PACKED>
static hipError_t launch_mt(const StreamArgs& a, int mt, dim3 grid, hipStream_t s) {
  if constexpr (MODE == MODE_DOWN && FP8) {
    const int steps = a.Kdim / kKS / a.ksplit;
    if (stream_uses_xl(FP8, MODE, mt, a)) {
      // bytes: the K range's activation pieces, and region B's LDS tiles
      constexpr int TB = tiles_b<FP8>();
      const size_t lds = std::max<size_t>((size_t)steps * 256 * 16, sizeof(uint16_t) * lds_elems<TB>());
      hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 1, PACKED, true>), grid, dim3(kThreads), lds, s, a);
      return hipGetLastError();
    }
  }
  switch (mt) {
    case 1: hipLaunchKernelGGL((ffn_stream_kernel<FP8, MODE, 1, PACKED, false>), grid, dim3(kThreads), 0, s, a); break;
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

bool stream_compacts(int fp8) { return !fp8; }

hipError_t launch_ffn_stream(const StreamArgs& a, int fp8, int packed, int mode, int mt, dim3 grid,
                             hipStream_t s) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (a.compact_rows != 0 && !stream_compacts(fp8)) return hipErrorInvalidValue;
  if (a.nblk < 1 || a.nblk > 8 || (int64_t)grid.x * 64 * a.nblk != a.N) return hipErrorInvalidValue;
  if (mt == 4 && a.b_rows != 0) return hipErrorInvalidValue;
  if (a.b_rows != 0 && a.b_rows < a.E_phys) return hipErrorInvalidValue;
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
