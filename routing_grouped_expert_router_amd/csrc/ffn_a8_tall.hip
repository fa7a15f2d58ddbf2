// W8A8 expert projections for large groups (prefill) on gfx950: fp8
// (E4M3FN) weights and activations, fp8 MFMA, per-128 block scales, the
// block sums promoted to fp32 ("推理 INFRA 方法论(5)", DeepGEMM section: FP8
// operands with per-128 scales, each 128-wide K block summed on the matrix
// unit and accumulated in fp32 after scaling; prefill groups in the
// contiguous layout with large tiles).
//
//  * Work item: 256 token rows of one group x a walk of 1..8 consecutive
//    weight tiles of 128 rows (MODE_GATEUP: 64 rows of W1 and the same 64
//    rows of W3, so SiLU(g) * u pairs sit in one lane; MODE_DOWN: 128 rows of
//    W2), from the persistent claim schedule of tile_sched.hpp.  The walk's
//    tiles run as one pipeline, so a short K range (the down projection's)
//    pays the item's set-up and the pipeline's fill once per walk; each
//    tile's outputs are stored straight from the accumulators once its last
//    K block is in.  Each of the four waves owns all 256 token rows x 32
//    weight rows (two 16-row panels: W1 and W3 of the same rows, or two of
//    W2), 16 x 2 MFMA tiles of 16 x 16, so a partly full tile shortens every
//    wave alike.
//  * K runs in 128-wide stages.  Per (row tile, panel) and stage one
//    v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales gives the block
//    sum, which is multiplied by the weight block's scale times the token's
//    and added to an fp32 accumulator, K blocks in ascending order: the
//    streaming W8A8 kernel's arithmetic, operand for operand, so both give
//    the same bits.
//  * Activation codes (32 KiB a stage, 16-byte pieces in MFMA lane order) go
//    by direct-to-LDS loads into a ring of four stages, three ahead; every
//    wave reads all 16 row tiles' fragments from it, each feeding its two
//    panels' products.  Each row's activation scales for four stages load
//    as one 16-byte piece into one of two alternating LDS buffers.
//  * Weights go straight to registers (each fragment is read by one wave),
//    four banks, three stages ahead.  The weight-block scales of the walk's
//    tiles (a row of K blocks per matrix and tile) go to LDS by direct loads
//    at the item's start.
//  * A stage's 12 loads per wave (13 when it also loads a scale block) are
//    issued one after each row tile's products, so they never queue in a
//    burst behind the MFMAs, and each tile's promotion runs under the next
//    tile's products; the products' results stay in ordinary VGPRs, where
//    the promotion's VALU instructions read them.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_sched.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int kAThreads = 256;
constexpr int kAM = kTileRows;              // token rows per work item
constexpr int kAMT = kAM / 16;              // 16-row MFMA tiles per item
constexpr int kAN = 128;                    // weight rows per weight tile
constexpr int kAStages = 4;                 // LDS ring slots of 128-wide K stages
constexpr int kAXBytes = kAM * 128;         // a ring slot: a stage's activation codes (32 KiB)
constexpr int kAScaleBlock = 4;             // K stages whose activation scales load together
constexpr int kAMaxKb = 128;                // K blocks a weight-scale row in LDS holds
constexpr int kAMaxWalk = 8;                // weight tiles one item walks, at most
constexpr int kALoads = 12;                 // loads per wave and stage: 8 codes, 4 weights (+1 scales
                                            // at every kAScaleBlock-th stage)
constexpr int kAAhead = 2;                  // row tiles whose fragments are read ahead of their products
constexpr int kPromoteValu = 10;            // VALU instructions of a tile's promotion
static_assert(kAM == 256 && kAMT == 16, "an item is 16 row tiles");
static_assert(kALoads + 1 <= kAMT, "a stage's loads fit its row-tile steps");
static_assert(kAScaleBlock == kAStages, "a scale block is one pass of the ring");
static_assert(kAMaxKb == 128, "two 64-word halves per weight-scale row, one per wave");

__device__ __forceinline__ float a8t_silu(float g) { return g / (1.0f + __expf(-g)); }

// a pointer every lane holds the same value of, in scalar registers (a
// buffer resource built from a value the compiler takes for divergent is
// used through a loop over its distinct values)
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ i32x8 join8(const u32x4 lo, const u32x4 hi) {
  return __builtin_bit_cast(i32x8, u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
}

// One work item: rows m0 = 256 mt .. of group tw.g against the ta.walk
// weight tiles tw.nt * walk .. (tw.nt + 1) * walk - 1, run as one pipeline of
// walk * (Kdim / 128) stages: stage st multiplies weight tile st / nkb at K
// block st % nkb, and a tile's outputs are stored straight from the
// accumulators once its last K block is in, while the next tile's first
// loads are in flight.  at_loop_end() runs once the last stage is done,
// before the last tile's stores.
template <int MODE, typename Hook>
__device__ __forceinline__ void a8_tall_tile(const A8TallArgs& ta, const TileWork& tw, char* r0, char* r1,
                                             char* r2, char* r3, float* xs0, float* xs1, float* wsc,
                                             Hook at_loop_end) {
  constexpr bool GU = MODE == MODE_GATEUP;
  const A8Args& a = ta.s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int g = tw.g, c0 = tw.c0, R = tw.R;
  const int64_t s0 = tw.s0, s1 = tw.s1;
  const int m0 = tw.mt * kAM;                  // first row of the item within the group
  const int N = a.N, Kdim = a.Kdim, nkb = Kdim / 128;
  const int walk = ta.walk;
  constexpr int kTileOut = GU ? kAN / 2 : kAN;           // output columns (weight rows) of a weight tile
  const int n0 = tw.nt * walk * kTileOut;                // first output column of the item

  const uint8_t* Wa;
  const uint8_t* Wb;
  const float* Sa;
  const float* Sb;
  if (tw.shared) {
    Wa = a.SW; Wb = GU ? a.SW3 : a.SW;
    Sa = a.SS; Sb = GU ? a.SS3 : a.SS;
  } else {
    Wa = a.W + (int64_t)g * N * Kdim;
    Wb = GU ? a.W3 + (int64_t)g * N * Kdim : Wa;
    Sa = a.S + (int64_t)g * (N / 128) * nkb;
    Sb = GU ? a.S3 + (int64_t)g * (N / 128) * nkb : Sa;
  }
  const __amdgpu_buffer_rsrc_t wra = buffer_rsrc(uniform_ptr(Wa), (uint32_t)N * Kdim);
  const __amdgpu_buffer_rsrc_t wrb = buffer_rsrc(uniform_ptr(Wb), (uint32_t)N * Kdim);
  const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(uniform_ptr(a.X), (uint32_t)(ta.x_rows * a.ldx));
  const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(uniform_ptr(a.XS), (uint32_t)(ta.x_rows * nkb * 4));
  // this wave's two 16-row weight panels (packed layout: per K block, panel
  // p's 2 KiB at p * 2048, lane l's 16 bytes of half j at j * 1024 + 16 l)
  const int pn0 = GU ? (n0 + 16 * wave) / 16 : (n0 + 32 * wave) / 16;
  const int pn1 = GU ? pn0 : pn0 + 1;
  const uint32_t pw[2] = {(uint32_t)pn0 * 2048 + lane * 16, (uint32_t)pn1 * 2048 + lane * 16};
  const uint32_t kbytes = (uint32_t)N * 128;   // one K block of the packed layout
  constexpr uint32_t kTileBytes = kTileOut / 16 * 2048;  // the next weight tile's panels, same K block

  // activation rows: the four row tiles of codes this wave loads (wave + 4 q;
  // lane: row lr, K bytes 16 lg + 64 j), then the row whose scales it loads
  // (row 64 wave + lane: 16 bytes, the scales of kAScaleBlock consecutive K
  // stages).  Rows past the group read a valid row, never used.  The gather
  // indices load together, under one wait.
  int rk[5];
#pragma unroll
  for (int q = 0; q < 4; ++q) rk[q] = m0 + (wave + 4 * q) * 16 + lr;
  rk[4] = m0 + 64 * wave + lane;
  int64_t rw[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) rk[i] = rk[i] < R ? rk[i] : 0;
  if (a.gather_src && !tw.shared) {
    const int32_t* gs = a.gather_src + a.gather_off[g];
#pragma unroll
    for (int i = 0; i < 5; ++i) rw[i] = gs[rk[i]];
  } else if (a.gather_src) {
#pragma unroll
    for (int i = 0; i < 5; ++i) rw[i] = rk[i];
  } else {
#pragma unroll
    for (int i = 0; i < 5; ++i) rw[i] = rk[i] < c0 ? s0 + rk[i] : s1 + (rk[i] - c0);
  }
  uint32_t xoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) xoff[q] = (uint32_t)(rw[q] * a.ldx) + 16 * lg;
  const uint32_t soff = (uint32_t)(rw[4] * nkb * 4);

  const int rows_here = min(kAM, R - m0);
  const int mv = ((rows_here + 31) / 32) * 2;   // non-empty 16-row tiles, in pairs
  auto run = [&](auto mvc) -> void {
    constexpr int MV = decltype(mvc)::value;
    auto slot = [&](auto sc) -> char* {
      constexpr int S = decltype(sc)::value;
      return S == 0 ? r0 : S == 1 ? r1 : S == 2 ? r2 : r3;
    };
    // load i of stage st (clamped past the end: re-read, never used):
    // 0..7 codes of row tile wave + 4 (i / 2), half i % 2, into ring slot
    // sl; 8..11 weights of panel (i - 8) / 2, half (i - 8) % 2, into bank b;
    // 12 (stages st % kAScaleBlock == 0) the activation scales of stages
    // st .. st + 3 into the scale buffer sb: word 4 r + k is row r, stage
    // st + k, so lane (lr) finds row tile m's scale at word 4 (16 m + lr) + k
    u32x4 wb[kAStages][2][2];
    // (wt, kb): weight tile of the walk and K block of the stage (past the
    // walk's end: its last stage again)
    auto issue = [&](int i, char* sl, u32x4 (*b)[2], float* sb, int wt, int kb) -> void {
      if (i < 8) {
        const int q = i >> 1, j = i & 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, sl + ((wave + 4 * q) * 2 + j) * 1024, 16, xoff[q],
                                                 (uint32_t)kb * 128 + 64 * j, 0, 0);
      } else if (i < kALoads) {
        const int n = (i - 8) >> 1, j = (i - 8) & 1;
        b[n][j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(n ? wrb : wra, (int)pw[n],
                                                         (int)(wt * kTileBytes + kb * kbytes + j * 1024), 0));
      } else {
        const int blk = kb / kAScaleBlock * kAScaleBlock;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, sb + wave * 256, 16, soff, (uint32_t)blk * 4, 0, 0);
      }
    };
    f32x4 acc[MV][2];
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[m][0] = acc[m][1] = f32x4{0, 0, 0, 0};
    // prologue: stages 0..2, weights first (a wait the compiler places
    // before the first load into a register then covers the previous
    // item's stores only), and after stage 0's weights the weight-block
    // scales of every tile of the walk, direct loads of 64 words:
    // wsc[2 kAMaxKb t + k] of W1 (W2) and wsc[2 kAMaxKb t + kAMaxKb + k] of
    // W3 for tile t (for the down projection the W2 row again in the W3
    // half); wave w loads matrix w / 2, words 64 (w % 2) .. of every tile,
    // kAMaxWalk loads whatever the walk (tiles past it load the last one
    // again), so the compiler's load counts stay fixed
#pragma unroll
    for (int i = 8; i < kALoads; ++i) issue(i, r0, wb[0], xs0, 0, 0);
    {
      const int mat = (wave >> 1) & 1, c = (wave & 1) * 64;
      const __amdgpu_buffer_rsrc_t sr = buffer_rsrc(uniform_ptr(GU && mat ? Sb : Sa), (uint32_t)(N / 128) * nkb * 4);
#pragma unroll
      for (int t = 0; t < kAMaxWalk; ++t) {
        const int tc = t < walk ? t : walk - 1;
        const uint32_t o = (uint32_t)(((n0 + tc * kTileOut) / 128) * nkb + min(c + lane, nkb - 1)) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, wsc + 2 * kAMaxKb * t + mat * kAMaxKb + c, 4, o, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(i, r0, wb[0], xs0, 0, 0);
    issue(kALoads, r0, wb[0], xs0, 0, 0);       // the scales of stages 0..3
    __builtin_amdgcn_sched_barrier(0);          // each stage's loads before the next stage's
#pragma unroll
    for (int i = 8; i < kALoads; ++i) issue(i, r1, wb[1], xs0, 0, 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(i, r1, wb[1], xs0, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 8; i < kALoads; ++i) issue(i, r2, wb[2], xs0, 0, 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(i, r2, wb[2], xs0, 0, 2);
    __builtin_amdgcn_sched_barrier(0);
    // Stage st's loads are issued during stage st - 3 (slot S - 1 mod 4),
    // kALoads of them, one more for stages st % 4 == 0 (issued from slot 1).
    // At the top of stage st the loads issued after stage st's are those of
    // st + 1 and st + 2, so vmcnt(their count) means this wave's loads of
    // stage st (and, before stage 0, the weight scales) have landed.
    auto stage = [&](auto sc, auto nc, int wt, int kb, float* rsb, float* lsb) -> void {
      constexpr int S = decltype(sc)::value;
      constexpr int kVm = 2 * kALoads + ((S + 1) % kAScaleBlock == 0) + ((S + 2) % kAScaleBlock == 0);
      constexpr int kWait = (kVm & 15) | ((kVm >> 4) << 14) | 0x70 | 0xF00;
      constexpr bool kScaleLoad = (S + kAStages - 1) % kAScaleBlock == 0;   // stage st + 3 starts a block
      u32x4 (*wc)[2] = wb[S];
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWait);       // this wave's loads of stage st landed
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): its reads of stage st - 1 are done
      __builtin_amdgcn_s_barrier();            // every wave's: stage st readable, slot of st - 1 free
      const char* xs = slot(sc);
      const i32x8 w0 = join8(wc[0][0], wc[0][1]), w1 = join8(wc[1][0], wc[1][1]);
      // the stage whose loads this one issues: three K blocks on, maybe in
      // the next weight tile, clamped to the walk's last stage
      int la_kb = kb + kAStages - 1, la_wt = wt;
      if (la_kb >= nkb) { la_kb -= nkb; ++la_wt; }
      if (la_wt >= walk) { la_wt = walk - 1; la_kb = nkb - 1; }
      const float sw0 = wsc[2 * kAMaxKb * wt + kb], sw1 = GU ? wsc[2 * kAMaxKb * wt + kAMaxKb + kb] : sw0;
      // activation scale of row tile m (this lane's token) at stage st,
      // read just before its promotion
      auto xscale = [&](int m) -> float { return rsb[4 * (16 * m + lr) + S]; };
      auto frag = [&](int m) -> i32x8 {
        return join8(*reinterpret_cast<const u32x4*>(xs + (m * 2) * 1024 + lane * 16),
                     *reinterpret_cast<const u32x4*>(xs + (m * 2 + 1) * 1024 + lane * 16));
      };
      i32x8 xf[kAAhead + 1];
#pragma unroll
      for (int m = 0; m < kAAhead && m < MV; ++m) xf[m] = frag(m);
      f32x4 dp0, dp1;                          // block sums of the previous row tile
      const f32x4 zero = {0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < kAMT; ++m) {
        if (m < MV) {
          if (m + kAAhead < MV) xf[(m + kAAhead) % (kAAhead + 1)] = frag(m + kAAhead);
          const i32x8 x = xf[m % (kAAhead + 1)];
          const f32x4 d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w0, x, zero, 0, 0, 0, 127, 0, 127);
          const f32x4 d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w1, x, zero, 0, 0, 0, 127, 0, 127);
          if (m > 0) {
            const float sxp = xscale(m - 1);
            acc[m - 1][0] += dp0 * (sw0 * sxp);
            acc[m - 1][1] += dp1 * (sw1 * sxp);
          }
          dp0 = d0;
          dp1 = d1;
        }
        if (m < kALoads || (kScaleLoad && m == kALoads))
          issue(m, slot(nc), wb[decltype(nc)::value], lsb, la_wt, la_kb);
      }
      const float sxl = xscale(MV - 1);
      acc[MV - 1][0] += dp0 * (sw0 * sxl);
      acc[MV - 1][1] += dp1 * (sw1 * sxl);
      // The stage is one scheduling region laid out as a pipeline: the
      // scale reads, then per row tile its fragment reads (two tiles ahead),
      // its two products each followed by VALU work -- the promotion of the
      // tile before, whose products have finished by then -- and one of the
      // next stage's loads.  (Left to itself the compiler put each tile's
      // promotion right behind its own products, so the wave waited for the
      // matrix core and then kept it idle through the promotion.)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + 2 * kAAhead, 0);   // DS reads
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        if (m + kAAhead < MV) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // fragment, scale
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, kPromoteValu / 2, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kPromoteValu / 2, 0);
        if (m < kALoads || (kScaleLoad && m == kALoads))
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // acc[m][n] holds D[row 4 lg + i of panel n][token lr of tile m] of
    // weight tile wt: bf16 outputs straight from the accumulators, 8 bytes
    // a lane, rows past the group not stored.  (The stores are younger than
    // every load a later stage top waits for, so those waits still hold.)
    auto store_tile = [&](int wt) -> void {
      uint16_t* out = static_cast<uint16_t*>(a.out) + n0 + wt * kTileOut;
#pragma unroll
      for (int m = 0; m < MV; ++m) {
        const int gr = m0 + m * 16 + lr;
        if (gr < R) {
          uint16_t* o = out + (gr < c0 ? s0 + gr : s1 + (gr - c0)) * a.ldo;
          if constexpr (GU) {
            const f32x4 gt = acc[m][0], up = acc[m][1];
            *reinterpret_cast<u32x2*>(o + 16 * wave + 4 * lg) =
                u32x2{pack_bf16x2(a8t_silu(gt.x) * up.x, a8t_silu(gt.y) * up.y),
                      pack_bf16x2(a8t_silu(gt.z) * up.z, a8t_silu(gt.w) * up.w)};
          } else {
#pragma unroll
            for (int n = 0; n < 2; ++n)
              *reinterpret_cast<u32x2*>(o + 32 * wave + 16 * n + 4 * lg) =
                  u32x2{pack_bf16x2(acc[m][n].x, acc[m][n].y), pack_bf16x2(acc[m][n].z, acc[m][n].w)};
          }
        }
      }
    };
    // two scale blocks per pass, so that each stage's scale buffers are
    // fixed: stages sb .. sb + 3 read xs0 while slot 1 loads the next
    // block into xs1, and the other way round; a weight tile ends at a pass
    // end (nkb is a multiple of the pass)
    for (int wt = 0; wt < walk; ++wt) {
      for (int kb = 0; kb < nkb; kb += 2 * kAStages) {
        stage(IntC<0>{}, IntC<3>{}, wt, kb, xs0, xs1);
        stage(IntC<1>{}, IntC<0>{}, wt, kb + 1, xs0, xs1);
        stage(IntC<2>{}, IntC<1>{}, wt, kb + 2, xs0, xs1);
        stage(IntC<3>{}, IntC<2>{}, wt, kb + 3, xs0, xs1);
        stage(IntC<0>{}, IntC<3>{}, wt, kb + 4, xs1, xs0);
        stage(IntC<1>{}, IntC<0>{}, wt, kb + 5, xs1, xs0);
        stage(IntC<2>{}, IntC<1>{}, wt, kb + 6, xs1, xs0);
        stage(IntC<3>{}, IntC<2>{}, wt, kb + 7, xs1, xs0);
      }
      if (wt + 1 < walk) {                     // a weight tile other than the last is complete
        store_tile(wt);
#pragma unroll
        for (int m = 0; m < MV; ++m) acc[m][0] = acc[m][1] = f32x4{0, 0, 0, 0};
      }
    }
    // no load may land in LDS once the next item's loads refill it
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    at_loop_end();
    store_tile(walk - 1);
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

template <int MODE>
__global__ __launch_bounds__(kAThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ffn_a8_tall_kernel(A8TallArgs ta) {
  __shared__ __attribute__((aligned(16))) char r0[kAXBytes];
  __shared__ __attribute__((aligned(16))) char r1[kAXBytes];
  __shared__ __attribute__((aligned(16))) char r2[kAXBytes];
  __shared__ __attribute__((aligned(16))) char r3[kAXBytes];
  __shared__ __attribute__((aligned(16))) float xs0[kAM * kAScaleBlock];   // activation scales of
  __shared__ __attribute__((aligned(16))) float xs1[kAM * kAScaleBlock];   // alternate stage blocks
  __shared__ __attribute__((aligned(16))) float wsc[2 * kAMaxKb * kAMaxWalk];
  const int ntn = ta.s.N / (MODE == MODE_GATEUP ? kAN / 2 : kAN) / ta.walk;   // walks per row tile
  claim_units<kAThreads>(ta.s, ta.tile_off, ta.claim, ntn, [&](const TileWork& tw, auto at_loop_end) {
    a8_tall_tile<MODE>(ta, tw, r0, r1, r2, r3, xs0, xs1, wsc, at_loop_end);
  });
}

// Whole 128-row output tiles (64 for gate/up), walks that divide their
// number, a K range of whole blocks of eight 128-wide stages that the scale
// rows in LDS hold, no K split, the route table's claim counters, and 32-bit
// buffer offsets.
bool a8_tall_supported(int mode, const A8TallArgs& a) {
  const A8Args& s = a.s;
  const int wn = mode == MODE_GATEUP ? kAN / 2 : kAN;
  if (s.N <= 0 || s.N % wn || s.N % 128 || s.Kdim <= 0 || s.Kdim % (128 * 2 * kAStages) || s.Kdim / 128 > kAMaxKb)
    return false;
  if (s.ksplit != 1 || s.out_f32 || s.ldx < s.Kdim || s.ldx % 16) return false;
  if (a.walk < 1 || a.walk > kAMaxWalk || (s.N / wn) % a.walk) return false;
  if (!a.claim || !a.tile_off || s.E_phys > kPlanGroups || a.x_rows <= 0) return false;
  const int64_t lim = int64_t(1) << 31;
  return (int64_t)s.N * s.Kdim < lim && a.x_rows * s.ldx < lim && a.x_rows * (s.Kdim / 128) * 4 < lim;
}

hipError_t launch_ffn_a8_tall(const A8TallArgs& a, int mode, hipStream_t s) {
  const int cus = device_cus();
  if (!a8_tall_supported(mode, a) || cus < kClaimLists) return hipErrorInvalidValue;
  const dim3 grid(cus);
  if (mode == MODE_GATEUP) hipLaunchKernelGGL((ffn_a8_tall_kernel<MODE_GATEUP>), grid, dim3(kAThreads), 0, s, a);
  else hipLaunchKernelGGL((ffn_a8_tall_kernel<MODE_DOWN>), grid, dim3(kAThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
