// gemm_tile_mma: tiled fp16/bf16 -> fp32 GEMM on CDNA4 MFMA.
//
// Each workgroup owns one BM x BN output tile.  The K loop streams 64-deep
// slabs of A and B through a double-buffered, swizzled LDS tile (the next slab
// is in flight while the current one feeds the MFMAs), the fp32 accumulators
// stay in registers for the whole loop, and the tile is stored once at the end
// (Warp issue #1965, "Proposed change" and "Design consequences").
#include <type_traits>

#include "gemm_core.hpp"

namespace mfl {

// ---------------------------------------------------------------------------
// Generic path: any operand orders, any M, N, K (ragged edges masked).  The
// next slab is staged in registers, then written to the LDS buffer not being
// read.
template <int BM, int BN, int BK, int WGM, int WGN, int SHAPE, int DT, bool AK, bool BKC, bool EDGE>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_tile_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ B,
                                                                   float* __restrict__ C, int64_t lda, int64_t ldb,
                                                                   int64_t ldc, int M, int N, int K, int tiles_m,
                                                                   int tiles_n, int accumulate) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MN = Shape<SHAPE>::MN;
  constexpr int TM = WM / MN, TN = WN / MN;
  static_assert(TM * MN == WM && TN * MN == WN, "wave tile must be a multiple of the MFMA tile");
  constexpr int STAGE = (BM + BN) * BK;
  using Acc = typename Shape<SHAPE>::Acc;

  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, &tm, &tn);
  const int row0 = tm * BM, col0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr0 = (wave / WGN) * WM, wc0 = (wave % WGN) * WN;
  // K-strided operands are staged k-major (TileLoader) and read with the
  // transpose read; the k-major layout is that of the 16x16x32 instruction.
  static_assert(SHAPE == 0 || (AK && BKC), "k-major tiles take the 16x16x32 instruction");
  using RA = std::conditional_t<AK, FragOffsets<SHAPE, BK>, KmFrag<SHAPE, BM, WM, TM>>;
  using RB = std::conditional_t<BKC, FragOffsets<SHAPE, BK>, KmFrag<SHAPE, BN, WN, TN>>;
  const RA fa(wr0, lane);
  const RB fb(wc0, lane);

  Acc acc[TM][TN];
  zero_acc<SHAPE, TM, TN>(acc);

  TileLoader<BM, BK, NT, AK, EDGE> la;
  TileLoader<BN, BK, NT, BKC, EDGE> lb;
  const int KT = (K + BK - 1) / BK;
  if (KT > 0) {
    la.load(A, lda, row0, 0, M, K, tid);
    lb.load(B, ldb, col0, 0, N, K, tid);
    la.store(lds, tid);
    lb.store(lds + BM * BK, tid);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = (kt & 1) * STAGE, nxt = STAGE - cur;
      const bool more = kt + 1 < KT;
      if (more) {
        la.load(A, lda, row0, (kt + 1) * BK, M, K, tid);
        lb.load(B, ldb, col0, (kt + 1) * BK, N, K, tid);
      }
      mma_slab<SHAPE, DT, TM, TN, BK>(lds + cur, lds + cur + BM * BK, fa, fb, acc);
      if (more) {
        la.store(lds + nxt, tid);
        lb.store(lds + nxt + BM * BK, tid);
      }
      __syncthreads();
    }
  }
  store_acc<SHAPE, TM, TN, EDGE>(C, ldc, row0 + wr0, col0 + wc0, M, N, lane, acc, accumulate);
}

template <int BM, int BN, int BK, int WGM, int WGN, int SHAPE, int DT, bool AK, bool BKC, bool EDGE>
static int launch_gemm(const void* a, int64_t lda, const void* b, int64_t ldb, float* c, int64_t ldc, int M, int N,
                       int K, int accumulate, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, BK, WGM, WGN, SHAPE, DT, AK, BKC, EDGE>), dim3(tiles_m * tiles_n),
                     dim3(WGM * WGN * 64), 0, stream, (const uint16_t*)a, (const uint16_t*)b, c, lda, ldb, ldc, M, N,
                     K, tiles_m, tiles_n, accumulate);
  return launch_status();
}

// ---------------------------------------------------------------------------
// Fast path: any operand order; ragged M, N, K through the EDGE variant.
// Global -> LDS moves use the CDNA4 direct-to-LDS buffer load (DmaOperand: one
// wave instruction writes 64 x 16 bytes to consecutive LDS addresses, with no
// staging registers, the layout applied on the source side).  Per-lane state is
// one 32-bit offset per operand; the row step of each load instruction and the
// K step are uniform scalar offsets.  Sixteen waves (four per SIMD, 64 x 64
// outputs each) let one wave's MFMAs run while another waits on LDS or on the
// barrier; at 256 x 256 x 64 the fragment traffic (conflict free) stays below
// the MFMA time.
//
// STAGES-deep ring of LDS stages: stage kt+STAGES-1 is requested while stage kt
// feeds the MFMAs.  One barrier per K step both publishes stage kt (every
// wave's loads for it have landed) and retires stage kt-1, whose buffer the
// new request reuses.  AKM / BKM: A column-major / B row-major (k-major slabs,
// fragments read with the transpose read).  EDGE: M or N is not a multiple of
// the tile, or K not of 64 — the last tile row / column loads zeros (or
// neighbouring storage) past the edge and stores only the elements inside C,
// and the last K slab zeroes the fragments of K positions past K.
template <int BM, int BN, int WGM, int WGN, int SHAPE, int DT, int STAGES, bool AKM, bool BKM, bool EDGE, int CARRY>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_fast_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ B,
                                                                   float* __restrict__ C, uint32_t lda, uint32_t ldb,
                                                                   uint32_t ldc, int M, int N, int K, int tiles_m,
                                                                   int tiles_n, int accumulate) {
  constexpr int BK = 64;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MN = Shape<SHAPE>::MN;
  constexpr int TM = WM / MN, TN = WN / MN;
  constexpr int STAGE = (BM + BN) * BK;
  using DA = DmaOperand<SHAPE, BM, NW, AKM, EDGE>;
  using DB = DmaOperand<SHAPE, BN, NW, BKM, EDGE>;
  constexpr int LOADS = DA::INSTR + DB::INSTR;
  static_assert(STAGES >= 2 && (STAGES - 2) * LOADS < 64, "vmcnt range");
  using Acc = typename Shape<SHAPE>::Acc;
  using RA = std::conditional_t<AKM, KmFrag<SHAPE, BM, WM, TM>, FragOffsets<SHAPE, BK>>;
  using RB = std::conditional_t<BKM, KmFrag<SHAPE, BN, WN, TN>, FragOffsets<SHAPE, BK>>;

  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, &tm, &tn);
  const int row0 = tm * BM, col0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr0 = (wave / WGN) * WM, wc0 = (wave % WGN) * WN;

  const DA da(A, lda, row0, K, wave, lane, M - row0);
  const DB db(B, ldb, col0, K, wave, lane, N - col0);
  auto issue = [&](int stage, int k0) {
    da.issue(lds + stage * STAGE, wave, k0);
    db.issue(lds + stage * STAGE + BM * BK, wave, k0);
  };

  const RA fa(wr0, lane);
  const RB fb(wc0, lane);
  Acc acc[TM][TN];
  zero_acc<SHAPE, TM, TN>(acc);
  u32x4 ca[CARRY > 0 ? CARRY : 1], cb[TN];  // fragments of the MFMAs carried over a barrier

  const int KT = (K + BK - 1) / BK;  // a multiple of BK unless EDGE
  // With a k-major operand the next stage's loads are issued after the
  // fragment reads of this stage's first MFMA K step: the compiler makes an
  // LDS transpose read that follows a direct-to-LDS load wait for that load to
  // land (it cannot tell the two buffers apart), so loads issued right after
  // the barrier would hold up the step's first reads for their whole latency.
  // Issued there, they still have most of the step to land.
  constexpr bool LATE = AKM || BKM;
  // With more than two stages the k-major fragments are read by transpose reads
  // the compiler does not track (mma_slab_tr_asm), so the next stage is issued
  // right after the barrier and stays in flight through the step: 2048^3 with
  // 128 x 128 tiles, k-major A and/or B, 22.3-23.2 us against 30.3-32.6 us.
  constexpr bool TRASM = (AKM || BKM) && STAGES > 2 && CARRY == 0;
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
    if (st < KT) issue(st, st * BK);
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads for stage kt are done when at most the later stages'
    // loads are still in flight; near the end fewer later stages exist
    if (kt + STAGES - 2 < KT)
      wait_vmcnt<(STAGES - 2) * LOADS>();
    else
      wait_vmcnt<0>();
    // Beyond two stages the barrier must leave the later stages' loads in
    // flight, which __syncthreads (its fence waits for every load) would not.
    if constexpr (STAGES > 2)
      lds_barrier();
    else
      __syncthreads();
    if constexpr (TRASM) {
      if (kt + STAGES - 1 < KT) issue((kt + STAGES - 1) % STAGES, (kt + STAGES - 1) * BK);
      const int cur = (kt % STAGES) * STAGE;
      mma_slab_tr_asm<SHAPE, DT, TM, TN, BK, AKM, BKM, EDGE>(lds + cur, lds + cur + BM * BK, fa, fb, acc,
                                                             K - kt * BK);
    } else if constexpr (!LATE) {
      if (kt + STAGES - 1 < KT) issue((kt + STAGES - 1) % STAGES, (kt + STAGES - 1) * BK);
      const int cur = (kt % STAGES) * STAGE;
      if constexpr (CARRY > 0)
        mma_slab_carry<SHAPE, DT, TM, TN, BK, CARRY, EDGE>(lds + cur, lds + cur + BM * BK, fa, fb, acc, ca, cb,
                                                            kt > 0, K - kt * BK);
      else
        mma_slab<SHAPE, DT, TM, TN, BK, EDGE>(lds + cur, lds + cur + BM * BK, fa, fb, acc, K - kt * BK);
    } else {
      const int cur = (kt % STAGES) * STAGE;
      const auto late = [&] {
        if (kt + STAGES - 1 < KT) issue((kt + STAGES - 1) % STAGES, (kt + STAGES - 1) * BK);
      };
      if constexpr (CARRY > 0)
        mma_slab_carry_then<SHAPE, DT, TM, TN, BK, CARRY, EDGE>(lds + cur, lds + cur + BM * BK, fa, fb, acc, ca, cb,
                                                                 kt > 0, K - kt * BK, late);
      else
        mma_slab_then<SHAPE, DT, TM, TN, BK, EDGE>(lds + cur, lds + cur + BM * BK, fa, fb, acc, K - kt * BK, late);
    }
  }
  if constexpr (CARRY > 0)
    if (KT > 0) mma_carried<SHAPE, DT, TM, TN, CARRY>(ca, cb, acc);
  // The store buffer starts at this wave's tile origin and spans its WM rows
  // (EDGE: only the rows inside C).
  const int wrows = EDGE ? max(0, min(WM, M - (row0 + wr0))) : WM;
  const rsrc_t rc = make_rsrc(C + (int64_t)(row0 + wr0) * ldc + col0 + wc0, (uint32_t)wrows * ldc * 4u);
  const int ncols = N - (col0 + wc0);
  if (accumulate)
    store_acc_rsrc<SHAPE, TM, TN, true, EDGE>(rc, ldc, lane, acc, ncols);
  else
    store_acc_rsrc<SHAPE, TM, TN, false, EDGE>(rc, ldc, lane, acc, ncols);
}

template <int BM, int BN, int WGM, int WGN, int SHAPE, int DT, bool AKM, bool BKM, int STAGES = 2>
static int launch_fast(const void* a, int64_t lda, const void* b, int64_t ldb, float* c, int64_t ldc, int M, int N,
                       int K, int accumulate, hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n), block(WGM * WGN * 64);
  const auto A = (const uint16_t*)a;
  const auto B = (const uint16_t*)b;
  // Whole 256 x 256 tiles (16 waves) with the 16x16x32 instruction carry two of
  // a wave's four fragment rows of each slab's last MFMA K step over the next
  // barrier (measured +1.4 % at 4096^3; the EDGE variant has no registers left
  // for the carried fragments and does not carry); whole 192 x 192 tiles carry
  // one row.
  constexpr int CARRY = SHAPE != 0 ? 0 : (BM == 256 && BN == 256) ? 2 : (BM == 192 && BN == 192) ? 1 : 0;
  if (M % BM == 0 && N % BN == 0 && K % 64 == 0)
    hipLaunchKernelGGL((gemm_fast_kernel<BM, BN, WGM, WGN, SHAPE, DT, STAGES, AKM, BKM, false, CARRY>), grid, block, 0,
                       stream, A, B, c, (uint32_t)lda, (uint32_t)ldb, (uint32_t)ldc, M, N, K, tiles_m, tiles_n,
                       accumulate);
  else
    hipLaunchKernelGGL((gemm_fast_kernel<BM, BN, WGM, WGN, SHAPE, DT, STAGES, AKM, BKM, true, 0>), grid, block, 0,
                       stream, A, B, c, (uint32_t)lda, (uint32_t)ldb, (uint32_t)ldc, M, N, K, tiles_m, tiles_n,
                       accumulate);
  return launch_status();
}

// ---------------------------------------------------------------------------
template <int DT, bool AK, bool BKC>
static int launch_generic(const void* a, int64_t lda, const void* b, int64_t ldb, float* c, int64_t ldc, int M, int N,
                          int K, int accumulate, hipStream_t s) {
  if (M % 128 == 0 && N % 128 == 0 && K % 64 == 0)
    return launch_gemm<128, 128, 64, 2, 2, 0, DT, AK, BKC, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  return launch_gemm<128, 128, 64, 2, 2, 0, DT, AK, BKC, true>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
}

// The buffer offsets of the fast path are 32-bit.  A K-contiguous operand's
// buffer is one tile panel (rows x ld elements, rows = 256 at most); a k-major
// operand's buffer spans all K rows (K x ld elements); C's is 256 rows of ldc.
static bool fast_fits(bool kmajor, int64_t ld, int64_t K) {
  const int64_t lim = (int64_t)1 << 32;
  return kmajor ? K * ld * 2 < lim : 256 * ld * 2 < lim;
}

// Wave quantisation.  256 x 256 tiles run one workgroup per CU, so a tile count
// just above a multiple of 256 leaves a last round with most CUs idle.  With at
// least two full rounds and a partial one, the first m1 tile-rows run as whole
// rounds of 256-tiles and the remaining rows as a second launch of 128 x 128
// tiles (two workgroups per CU), which must fit one round (at most 512 tiles).
// m1 is one tile-row below the most that fits the full rounds (one more if the
// rest would not fit one round).  Measured, K-contiguous operands: 6144^3
// +9 %, 7168^3 +9 %, 10240 x 4096 x 4096 +4 %; k-major A and/or B: 6144^3
// +7-9 %, 7168^3 +2-5 %.  Each output element sees the
// same MFMA sequence whatever the tile size, so the two launches give the same
// bits as one.  Returns m1, or 0 for a single launch.
static int quantisation_split_rows(int M, int N) {
  const int tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int64_t T = (int64_t)tm * tn, F = T / 256;
  if (F < 2 || T % 256 == 0) return 0;
  const auto small = [&](int64_t m1) { return ((M - 256 * m1 + 127) / 128) * (int64_t)((N + 127) / 128); };
  int64_t m1 = 256 * F / tn - 1;
  if (small(m1) > 512) ++m1;
  if (m1 < 1 || m1 >= tm || m1 * tn > 256 * F || small(m1) > 512) return 0;
  return (int)m1;
}

template <int DT, bool AKM, bool BKM>
static int dispatch_fast(int shape, const void* a, int64_t lda, const void* b, int64_t ldb, float* c, int64_t ldc,
                         int M, int N, int K, int accumulate, hipStream_t s) {
  // The largest tile that still gives the chip at least 128 workgroups:
  // 256 x 256 (16 waves of 64 x 64; 192 x 192 when that fills one round
  // better, below), 128 x 128 (4 waves of 64 x 64), or for small problems
  // with K-contiguous operands 64 x 64 or 32 x 32 (4 waves each, below), where
  // a single big tile would leave all but a few CUs idle.  Sizes that are not
  // tile multiples run the EDGE variant of the same kernel.
  const auto count = [&](int t) { return (int64_t)((M + t - 1) / t) * ((N + t - 1) / t); };
  const bool s32 = shape == MFL_MFMA_32X32X16;
  if (const int m1 = quantisation_split_rows(M, N)) {
    const int M1 = 256 * m1;
    // rows M1.. of A: M1 rows in (row-major) or M1 elements in (column-major)
    const auto a2 = (const uint16_t*)a + (AKM ? (int64_t)M1 : (int64_t)M1 * lda);
    float* c2 = c + (int64_t)M1 * ldc;
    const int r = s32 ? launch_fast<256, 256, 4, 4, 1, DT, AKM, BKM>(a, lda, b, ldb, c, ldc, M1, N, K, accumulate, s)
                      : launch_fast<256, 256, 4, 4, 0, DT, AKM, BKM>(a, lda, b, ldb, c, ldc, M1, N, K, accumulate, s);
    if (r != MFL_OK) return r;
    return s32 ? launch_fast<128, 128, 2, 2, 1, DT, AKM, BKM>(a2, lda, b, ldb, c2, ldc, M - M1, N, K, accumulate, s)
               : launch_fast<128, 128, 2, 2, 0, DT, AKM, BKM>(a2, lda, b, ldb, c2, ldc, M - M1, N, K, accumulate, s);
  }
  // One partial round of 256 x 256 tiles (128-255 of them, e.g. 3072^3: 144)
  // leaves CUs idle; when 192 x 192 tiles (12 waves of 64 x 48, three per SIMD)
  // cover C in one round they run on more CUs: 3072^3 50 us against 60 us
  // (256 workgroups against 144).  The 192-wide slab is K-contiguous only, and
  // a 48-wide wave tile needs the 16x16x32 instruction.  Above one round the
  // extra rounds cost more than the fill gains (3328^3: 96 us against 67 us).
  if constexpr (!AKM && !BKM)
    if (!s32 && count(256) >= 128 && count(256) < 256 && count(192) <= 256)
      return launch_fast<192, 192, 3, 4, 0, DT, false, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  if (count(256) >= 128)
    return s32 ? launch_fast<256, 256, 4, 4, 1, DT, AKM, BKM>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s)
               : launch_fast<256, 256, 4, 4, 0, DT, AKM, BKM>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  // 128 x 128 tiles.  At most one per CU: 16 waves of 32 x 32 and three LDS
  // stages (2048^3 20.5 us against 24.4 us with 4 waves of 64 x 64 and two
  // stages; 1536^3 14.5 against 18.1).  More tiles: 4 waves and two stages, so
  // that two workgroups share a CU (2560^3 35.7 us against 43.1).
  if (count(128) >= 128 || AKM || BKM) {
    if (s32) return launch_fast<128, 128, 2, 2, 1, DT, AKM, BKM>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    if (count(128) <= 256)
      return launch_fast<128, 128, 4, 4, 0, DT, AKM, BKM, 3>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    return launch_fast<128, 128, 2, 2, 0, DT, AKM, BKM>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  }
  // Small problems: 64 x 64 tiles with 4 waves of 32 x 32, or, with the
  // 16x16x32 instruction, 32 x 32 tiles (4 waves of 16 x 16) when 64-tiles
  // would give fewer than 128 workgroups.  Measured (bf16, kernel time): 1024^3
  // 6.7 us against 7.4 us for 64 x 64 tiles with 2 waves; 512^3 3.8 us on
  // 32 x 32 tiles against 4.2 / 4.7 us on 64 x 64 tiles with 4 / 2 waves.
  if constexpr (!AKM && !BKM) {
    if (s32) return launch_fast<64, 64, 2, 2, 1, DT, false, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    if (count(64) >= 128)
      return launch_fast<64, 64, 2, 2, 0, DT, false, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    return launch_fast<32, 32, 2, 2, 0, DT, false, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  }
  return MFL_EUNSUPPORTED;  // not reached: k-major operands always take a 128 or 256 tile
}

// Whether dispatch_fast takes these sizes: K a multiple of 8 (whole 16-byte
// chunks along K), and an M (N) that a k-major A (B) tile can clamp on a
// 16-byte chunk boundary.
static bool fast_sizes(bool akm, bool bkm, int M, int N, int K) {
  return K % 8 == 0 && K > 0 && (!akm || M % 8 == 0) && (!bkm || N % 8 == 0);
}

template <int DT>
static int dispatch(int shape, const void* a, int64_t lda, int oa, const void* b, int64_t ldb, int ob, float* c,
                    int64_t ldc, int M, int N, int K, int accumulate, hipStream_t s) {
  const bool akm = oa == MFL_COL_MAJOR, bkm = ob == MFL_ROW_MAJOR;
  if (fast_sizes(akm, bkm, M, N, K) && fast_fits(akm, lda, K) && fast_fits(bkm, ldb, K) &&
      256 * ldc * 4 < ((int64_t)1 << 32)) {
    if (!akm && !bkm) return dispatch_fast<DT, false, false>(shape, a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    if (!akm) return dispatch_fast<DT, false, true>(shape, a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    if (!bkm) return dispatch_fast<DT, true, false>(shape, a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
    return dispatch_fast<DT, true, true>(shape, a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  }
  if (!akm && !bkm) return launch_generic<DT, true, true>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  if (!akm) return launch_generic<DT, true, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  if (!bkm) return launch_generic<DT, false, true>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
  return launch_generic<DT, false, false>(a, lda, b, ldb, c, ldc, M, N, K, accumulate, s);
}

// Validates one 16-bit operand of `rows` x `cols` (logical) stored in `order`.
static int check16(const void* p, int64_t rows, int64_t cols, int64_t ld, int order) {
  if (order != MFL_ROW_MAJOR && order != MFL_COL_MAJOR) return MFL_EINVAL;
  if (rows == 0 || cols == 0) return MFL_OK;
  if (!p || !aligned16(p) || ld <= 0 || ld % 8 != 0) return MFL_EINVAL;
  const int64_t inner = order == MFL_ROW_MAJOR ? cols : rows;
  const int64_t outer = order == MFL_ROW_MAJOR ? rows : cols;
  if (ld < inner) return MFL_EINVAL;
  if (outer > INT64_MAX / ld) return MFL_EOVERFLOW;
  return MFL_OK;
}

}  // namespace mfl

using namespace mfl;

extern "C" int gemm_tile_mma_shape(int shape, int dtype, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda,
                                   int order_a, const void* b, int64_t ldb, int order_b, float* c, int64_t ldc,
                                   int accumulate, void* stream) {
  if (shape != MFL_MFMA_16X16X32 && shape != MFL_MFMA_32X32X16) return MFL_EINVAL;
  if (dtype != MFL_F16 && dtype != MFL_BF16) return MFL_EINVAL;
  if (m < 0 || n < 0 || k < 0 || (accumulate != 0 && accumulate != 1)) return MFL_EINVAL;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return MFL_EUNSUPPORTED;
  int st;
  if ((st = check16(a, m, k, lda, order_a)) != MFL_OK) return st;
  if ((st = check16(b, k, n, ldb, order_b)) != MFL_OK) return st;
  if (m == 0 || n == 0) return MFL_OK;
  if (!c || ((uintptr_t)c & 3) || ldc < n) return MFL_EINVAL;
  if (m > INT64_MAX / ldc) return MFL_EOVERFLOW;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MFL_BF16)
    return dispatch<MFL_BF16>(shape, a, lda, order_a, b, ldb, order_b, c, ldc, (int)m, (int)n, (int)k, accumulate, s);
  return dispatch<MFL_F16>(shape, a, lda, order_a, b, ldb, order_b, c, ldc, (int)m, (int)n, (int)k, accumulate, s);
}

extern "C" int gemm_tile_mma(int dtype, int64_t m, int64_t n, int64_t k, const void* a, int64_t lda, int order_a,
                             const void* b, int64_t ldb, int order_b, float* c, int64_t ldc, int accumulate,
                             void* stream) {
  return gemm_tile_mma_shape(MFL_MFMA_16X16X32, dtype, m, n, k, a, lda, order_a, b, ldb, order_b, c, ldc, accumulate,
                             stream);
}
