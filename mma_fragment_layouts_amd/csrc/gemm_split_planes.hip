// Split-precision fp32 GEMM from pre-split 16-bit planes (Strata PR #800, "The
// fix": hi and lo products in separate accumulator chains, added in plain fp32
// at the end).
//
// The split-on-load kernel (gemm_split.hpp) converts every fp32 tile it loads,
// so each element of A is split once per column tile of C (and each element of
// B once per row tile): at 4096^3 that is 32 conversions per element and about
// three vector instructions per MFMA.  Here each operand is split once into hi
// and lo planes in HBM (one elementwise pass), and the GEMM streams the four
// 16-bit planes with the direct-to-LDS buffer loads of the dense fast path.
//
// Tile: 128 x 128 x 64, 8 waves of 64 x 32 outputs (two per SIMD), so that
// three chains of accumulators (96 registers) fit beside the operand fragments.
// Per MFMA K step a wave reads 4 + 4 A fragments and 2 + 2 B fragments for 24
// MFMAs.  For every accumulator the MFMAs arrive in the same order as in the
// split-on-load kernel (K steps ascending; within one, hh, hl, lh, ll), and the
// chains are summed the same way, so both kernels give bit-identical results.
#include <type_traits>

#include "gemm_split.hpp"

namespace mfl {

// AKM / BKM: A column-major / B row-major — those planes are staged k-major
// and read with the transpose read, as in the dense fast path; the MFMAs and
// their order do not change, so every operand order gives the same bits.
// EDGE: M or N is not a multiple of 128, or K not of 64 — as in the dense fast
// path, the last tiles load zeros (or neighbouring storage) past the edges, the
// fragments of K positions past K are zeroed in the last slab, and only the
// elements inside C are stored.
// 128 x 128 tiles, 16 waves of 32 x 32 (four per SIMD): at 4096^3 with 3 chains
// 306 us against 322 us for 8 waves of 64 x 32, bit-identical.
constexpr int kPlanesWGM = 4, kPlanesWGN = 4;

template <int DT, class P, bool AKM, bool BKM, bool EDGE>
__global__ __launch_bounds__(kPlanesWGM* kPlanesWGN * 64) void gemm_split_planes_kernel(const uint16_t* __restrict__ Ah,
                                                                const uint16_t* __restrict__ Al,
                                                                const uint16_t* __restrict__ Bh,
                                                                const uint16_t* __restrict__ Bl, float* __restrict__ C,
                                                                uint32_t lda, uint32_t ldb, uint32_t ldc, int M, int N,
                                                                int K, int tiles_m, int tiles_n, int accumulate) {
  static_assert(P::SA && P::SB, "the planes path splits both operands");
  constexpr int SHAPE = 0, BM = 128, BN = 128, BK = 64, WGM = kPlanesWGM, WGN = kPlanesWGN, NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MN = Shape<SHAPE>::MN;
  constexpr int TM = WM / MN, TN = WN / MN;
  constexpr int PLANE = BM * BK;                   // one plane's slab (BM == BN), 16-bit elements
  constexpr int STAGE = 4 * PLANE;                 // A_hi | A_lo | B_hi | B_lo
  static_assert(BM == BN, "planes share one slab size");
  using DA = DmaOperand<SHAPE, BM, NW, AKM, EDGE>;
  using DB = DmaOperand<SHAPE, BN, NW, BKM, EDGE>;
  static_assert(2 * (DA::INSTR + DB::INSTR) < 64, "vmcnt range");
  using RA = std::conditional_t<AKM, KmFrag<SHAPE, BM, WM, TM>, FragOffsets<SHAPE, BK>>;
  using RB = std::conditional_t<BKM, KmFrag<SHAPE, BN, WN, TN>, FragOffsets<SHAPE, BK>>;
  using Acc = typename Shape<SHAPE>::Acc;

  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, &tm, &tn);
  const int row0 = tm * BM, col0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr0 = (wave / WGN) * WM, wc0 = (wave % WGN) * WN;

  const DA dah(Ah, lda, row0, K, wave, lane, M - row0), dal(Al, lda, row0, K, wave, lane, M - row0);
  const DB dbh(Bh, ldb, col0, K, wave, lane, N - col0), dbl(Bl, ldb, col0, K, wave, lane, N - col0);
  auto issue = [&](int stage, int k0) {
    uint16_t* st = lds + stage * STAGE;
    dah.issue(st, wave, k0);
    dal.issue(st + PLANE, wave, k0);
    dbh.issue(st + 2 * PLANE, wave, k0);
    dbl.issue(st + 3 * PLANE, wave, k0);
  };

  const RA fa(wr0, lane);
  const RB fb(wc0, lane);
  Acc acc[P::CHAINS][TM][TN];
#pragma unroll
  for (int ch = 0; ch < P::CHAINS; ++ch) zero_acc<SHAPE, TM, TN>(acc[ch]);

  const int KT = (K + BK - 1) / BK;  // a multiple of BK unless EDGE
  // A k-major plane's fragments are read by transpose reads the compiler does
  // not track (frag_read_tr_asm): a tracked one would wait for the next
  // stage's loads, issued right after the barrier, to land.  4096^3, 3
  // chains, A column-major and B row-major, one machine: 416-417 us per call
  // against 438-441 us with tracked reads and the loads issued after each
  // step's first reads (K-contiguous planes 381-383 us).
  constexpr bool TRASM = AKM || BKM;
  constexpr int KS = BK / Shape<SHAPE>::K;
  // One slab with k-major plane(s): every fragment of a K step read, waited
  // for, then the step's MFMAs (same products and order as below).
  auto slab_tr = [&](const uint16_t* st, int kvalid) {
    uint32_t ba = 0, bb = 0;
    if constexpr (AKM) ba = lds_address(st + fa.off);
    if constexpr (BKM) bb = lds_address(st + 2 * PLANE + fb.off);
    static_for<KS>([&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      u32x4 ah[TM], al[TM], bh[TN], bl[TN];
      static_for<TM>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (AKM) {
          ah[i] = frag_read_tr_asm<SHAPE, kk, i>(ba);
          al[i] = frag_read_tr_asm<SHAPE, kk, i>(ba + 2 * PLANE);
        } else {
          ah[i] = frag_read(st, fa, kk, i);
          al[i] = frag_read(st + PLANE, fa, kk, i);
        }
      });
      static_for<TN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (BKM) {
          bh[j] = frag_read_tr_asm<SHAPE, kk, j>(bb);
          bl[j] = frag_read_tr_asm<SHAPE, kk, j>(bb + 2 * PLANE);
        } else {
          bh[j] = frag_read(st + 2 * PLANE, fb, kk, j);
          bl[j] = frag_read(st + 3 * PLANE, fb, kk, j);
        }
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if constexpr (AKM) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          asm volatile("" : "+v"(ah[i]));
          asm volatile("" : "+v"(al[i]));
        }
      }
      if constexpr (BKM) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          asm volatile("" : "+v"(bh[j]));
          asm volatile("" : "+v"(bl[j]));
        }
      }
      if constexpr (EDGE) {
        if (kvalid < BK && kk * Shape<SHAPE>::K + 8 * (lane / MN) >= kvalid) {
#pragma unroll
          for (int i = 0; i < TM; ++i) ah[i] = al[i] = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < TN; ++j) bh[j] = bl[j] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int p = 0; p < P::NPROD; ++p)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const u32x4 av = P::a_lo(p) ? al[i] : ah[i];
            const u32x4 bv = P::b_lo(p) ? bl[j] : bh[j];
            acc[P::chain(p)][i][j] = mfma<SHAPE, DT>(av, bv, acc[P::chain(p)][i][j]);
          }
    });
  };
  if (KT > 0) issue(0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    // this wave's loads of stage kt have landed; after the barrier every
    // wave's have, and stage kt-1 (the buffer refilled next) is retired
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 1 < KT) issue((kt + 1) & 1, (kt + 1) * BK);
    const uint16_t* st = lds + (kt & 1) * STAGE;
    if constexpr (TRASM) {
      slab_tr(st, K - kt * BK);
      continue;
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 ah[TM], al[TM], bh[TN], bl[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        ah[i] = frag_read(st, fa, kk, i);
        al[i] = frag_read(st + PLANE, fa, kk, i);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bh[j] = frag_read(st + 2 * PLANE, fb, kk, j);
        bl[j] = frag_read(st + 3 * PLANE, fb, kk, j);
      }
      if constexpr (EDGE) {
        // K positions 8*(lane/16) .. +7 of MFMA step kk (the operand numeral);
        // the bound is wave-uniform, so only the last slab of a K tail branches
        const int kvalid = K - kt * BK;
        if (kvalid < BK && kk * Shape<SHAPE>::K + 8 * (lane / MN) >= kvalid) {
#pragma unroll
          for (int i = 0; i < TM; ++i) ah[i] = al[i] = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < TN; ++j) bh[j] = bl[j] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int p = 0; p < P::NPROD; ++p)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const u32x4 av = P::a_lo(p) ? al[i] : ah[i];
            const u32x4 bv = P::b_lo(p) ? bl[j] : bh[j];
            acc[P::chain(p)][i][j] = mfma<SHAPE, DT>(av, bv, acc[P::chain(p)][i][j]);
          }
    }
  }
  // Chains in plain fp32, the small ones first: c0 + (c1 + c2).
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (P::CHAINS == 3) acc[1][i][j] = acc[1][i][j] + acc[2][i][j];
      if constexpr (P::CHAINS >= 2) acc[0][i][j] = acc[0][i][j] + acc[1][i][j];
    }
  // The store buffer spans this wave's rows inside C (EDGE: only those < M).
  const int wrows = EDGE ? max(0, min(WM, M - (row0 + wr0))) : WM;
  const rsrc_t rc = make_rsrc(C + (int64_t)(row0 + wr0) * ldc + col0 + wc0, (uint32_t)wrows * ldc * 4u);
  const int ncols = N - (col0 + wc0);
  if (accumulate)
    store_acc_rsrc<SHAPE, TM, TN, true, EDGE>(rc, ldc, lane, acc[0], ncols);
  else
    store_acc_rsrc<SHAPE, TM, TN, false, EDGE>(rc, ldc, lane, acc[0], ncols);
}

template <int DT, class P, bool AKM, bool BKM>
static int launch_planes(const uint16_t* ah, const uint16_t* al, const uint16_t* bh, const uint16_t* bl, float* c,
                         int64_t lda, int64_t ldb, int64_t ldc, int M, int N, int K, int accumulate, hipStream_t s) {
  const int tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  const dim3 grid(tiles_m * tiles_n), block(kPlanesWGM * kPlanesWGN * 64);
  if (M % 128 == 0 && N % 128 == 0 && K % 64 == 0)
    hipLaunchKernelGGL((gemm_split_planes_kernel<DT, P, AKM, BKM, false>), grid, block, 0, s, ah, al, bh, bl, c,
                       (uint32_t)lda, (uint32_t)ldb, (uint32_t)ldc, M, N, K, tiles_m, tiles_n, accumulate);
  else
    hipLaunchKernelGGL((gemm_split_planes_kernel<DT, P, AKM, BKM, true>), grid, block, 0, s, ah, al, bh, bl, c,
                       (uint32_t)lda, (uint32_t)ldb, (uint32_t)ldc, M, N, K, tiles_m, tiles_n, accumulate);
  return launch_status();
}

template <int DT, bool AKM, bool BKM>
static int dispatch_planes(int chains, bool lolo, const uint16_t* ah, const uint16_t* al, const uint16_t* bh,
                           const uint16_t* bl, float* c, int64_t lda, int64_t ldb, int64_t ldc, int M, int N, int K,
                           int accumulate, hipStream_t s) {
#define MFL_PLANES(CH, LL)                                                                                       \
  return launch_planes<DT, Products<true, true, CH, LL>, AKM, BKM>(ah, al, bh, bl, c, lda, ldb, ldc, M, N, K, \
                                                                   accumulate, s)
  if (lolo) {
    if (chains == 1) MFL_PLANES(1, true);
    if (chains == 2) MFL_PLANES(2, true);
    MFL_PLANES(3, true);
  }
  if (chains == 1) MFL_PLANES(1, false);
  if (chains == 2) MFL_PLANES(2, false);
  MFL_PLANES(3, false);
#undef MFL_PLANES
}

template <int DT>
static int dispatch_planes_orders(bool akm, bool bkm, int chains, bool lolo, const uint16_t* ah, const uint16_t* al,
                                  const uint16_t* bh, const uint16_t* bl, float* c, int64_t lda, int64_t ldb,
                                  int64_t ldc, int M, int N, int K, int accumulate, hipStream_t s) {
  if (!akm && !bkm)
    return dispatch_planes<DT, false, false>(chains, lolo, ah, al, bh, bl, c, lda, ldb, ldc, M, N, K, accumulate, s);
  if (!akm)
    return dispatch_planes<DT, false, true>(chains, lolo, ah, al, bh, bl, c, lda, ldb, ldc, M, N, K, accumulate, s);
  if (!bkm)
    return dispatch_planes<DT, true, false>(chains, lolo, ah, al, bh, bl, c, lda, ldb, ldc, M, N, K, accumulate, s);
  return dispatch_planes<DT, true, true>(chains, lolo, ah, al, bh, bl, c, lda, ldb, ldc, M, N, K, accumulate, s);
}

static int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Storage rows of an operand: A (m x k) has m rows of lda when row-major and k
// rows when column-major; B (k x n) has n rows of ldb when column-major and k
// rows when row-major.  The planes have the operand's storage shape.
static int64_t rows_a(int64_t m, int64_t k, int order_a) { return order_a == MFL_ROW_MAJOR ? m : k; }
static int64_t rows_b(int64_t n, int64_t k, int order_b) { return order_b == MFL_COL_MAJOR ? n : k; }
static int64_t inner_a(int64_t m, int64_t k, int order_a) { return order_a == MFL_ROW_MAJOR ? k : m; }
static int64_t inner_b(int64_t n, int64_t k, int order_b) { return order_b == MFL_COL_MAJOR ? k : n; }

static int64_t planes_bytes(int64_t m, int64_t n, int64_t k, int64_t lda, int order_a, int64_t ldb, int order_b) {
  return 2 * align256(rows_a(m, k, order_a) * lda * 2) + 2 * align256(rows_b(n, k, order_b) * ldb * 2);
}

// The planes path takes both operands split, K a multiple of 8 (whole 16-byte
// chunks along K), an M (N) that a k-major A (B) tile can clamp on a 16-byte
// chunk boundary, rows of the planes 16-byte aligned, and 32-bit buffer
// offsets: a K-contiguous operand's buffer is one 128-row panel, a k-major
// operand's spans all k rows.  M and N need not be tile multiples.
static bool planes_apply(int64_t m, int64_t n, int64_t k, int64_t lda, int order_a, int mode_a, int64_t ldb,
                         int order_b, int mode_b, int64_t ldc) {
  const int64_t lim = (int64_t)1 << 32;
  if (mode_a != MFL_SPLIT || mode_b != MFL_SPLIT) return false;
  if (m <= 0 || n <= 0 || k <= 0 || k % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0) return false;
  if ((order_a == MFL_COL_MAJOR && m % 8 != 0) || (order_b == MFL_ROW_MAJOR && n % 8 != 0)) return false;
  const int64_t pa = order_a == MFL_ROW_MAJOR ? 128 : k, pb = order_b == MFL_COL_MAJOR ? 128 : k;
  return pa * lda * 2 < lim && pb * ldb * 2 < lim && 64 * ldc * 4 < lim;
}

}  // namespace mfl

using namespace mfl;

extern "C" int split_fp32(int dtype, const float* x, void* hi, void* lo, int64_t n, void* stream);

extern "C" int gemm_split_fp32_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t lda, int order_a, int mode_a,
                                               int64_t ldb, int order_b, int mode_b, int64_t ldc, int64_t* bytes) {
  if (!bytes || m < 0 || n < 0 || k < 0 || lda < 0 || ldb < 0 || ldc < 0) return MFL_EINVAL;
  if ((order_a != MFL_ROW_MAJOR && order_a != MFL_COL_MAJOR) || (order_b != MFL_ROW_MAJOR && order_b != MFL_COL_MAJOR))
    return MFL_EINVAL;
  if ((mode_a != MFL_ROUND && mode_a != MFL_SPLIT) || (mode_b != MFL_ROUND && mode_b != MFL_SPLIT)) return MFL_EINVAL;
  if (!planes_apply(m, n, k, lda, order_a, mode_a, ldb, order_b, mode_b, ldc)) {
    *bytes = 0;  // the split-on-load kernel runs; it needs no workspace
    return MFL_OK;
  }
  if (rows_a(m, k, order_a) > INT64_MAX / 4 / lda || rows_b(n, k, order_b) > INT64_MAX / 4 / ldb) return MFL_EOVERFLOW;
  *bytes = planes_bytes(m, n, k, lda, order_a, ldb, order_b);
  return MFL_OK;
}

extern "C" int gemm_split_fp32(int piece, int64_t m, int64_t n, int64_t k, const float* a, int64_t lda, int order_a,
                               int mode_a, const float* b, int64_t ldb, int order_b, int mode_b, int chains, int lolo,
                               float* c, int64_t ldc, int accumulate, void* stream);

extern "C" int gemm_split_fp32_ws(int piece, int64_t m, int64_t n, int64_t k, const float* a, int64_t lda, int order_a,
                                  int mode_a, const float* b, int64_t ldb, int order_b, int mode_b, int chains,
                                  int lolo, float* c, int64_t ldc, int accumulate, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
  if (!planes_apply(m, n, k, lda, order_a, mode_a, ldb, order_b, mode_b, ldc))
    return gemm_split_fp32(piece, m, n, k, a, lda, order_a, mode_a, b, ldb, order_b, mode_b, chains, lolo, c, ldc,
                           accumulate, stream);
  // Same argument checks as gemm_split_fp32 for what the planes path can meet.
  if (piece != MFL_F16 && piece != MFL_BF16) return MFL_EINVAL;
  if ((lolo != 0 && lolo != 1) || (accumulate != 0 && accumulate != 1)) return MFL_EINVAL;
  if (chains < 1 || chains > 3 || chains > 3 + lolo) return MFL_EINVAL;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return MFL_EUNSUPPORTED;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || ((uintptr_t)c & 3)) return MFL_EINVAL;
  const int64_t ra = rows_a(m, k, order_a), rb = rows_b(n, k, order_b);
  if (lda < inner_a(m, k, order_a) || ldb < inner_b(n, k, order_b) || ldc < n) return MFL_EINVAL;
  if (ra > INT64_MAX / 4 / lda || rb > INT64_MAX / 4 / ldb || m > INT64_MAX / ldc) return MFL_EOVERFLOW;
  if (!workspace || ((uintptr_t)workspace & 255) ||
      workspace_bytes < planes_bytes(m, n, k, lda, order_a, ldb, order_b))
    return MFL_EINVAL;
  char* w = (char*)workspace;
  uint16_t* ah = (uint16_t*)w;
  uint16_t* al = (uint16_t*)(w + align256(ra * lda * 2));
  uint16_t* bh = (uint16_t*)(w + 2 * align256(ra * lda * 2));
  uint16_t* bl = (uint16_t*)(w + 2 * align256(ra * lda * 2) + align256(rb * ldb * 2));
  // Split exactly the elements each operand's storage spans,
  // (rows - 1) * ld + inner: the last row need not be padded.
  int st;
  if ((st = split_fp32(piece, a, ah, al, (ra - 1) * lda + inner_a(m, k, order_a), stream)) != MFL_OK) return st;
  if ((st = split_fp32(piece, b, bh, bl, (rb - 1) * ldb + inner_b(n, k, order_b), stream)) != MFL_OK) return st;
  const bool akm = order_a == MFL_COL_MAJOR, bkm = order_b == MFL_ROW_MAJOR;
  hipStream_t s = (hipStream_t)stream;
  if (piece == MFL_BF16)
    return dispatch_planes_orders<MFL_BF16>(akm, bkm, chains, lolo, ah, al, bh, bl, c, lda, ldb, ldc, (int)m, (int)n,
                                            (int)k, accumulate, s);
  return dispatch_planes_orders<MFL_F16>(akm, bkm, chains, lolo, ah, al, bh, bl, c, lda, ldb, ldc, (int)m, (int)n,
                                         (int)k, accumulate, s);
}
