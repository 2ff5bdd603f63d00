// Split-precision fp32 GEMM on 16-bit MFMA (Strata PR #800, "What's going on"
// and "The fix").
//
// An fp32 operand in split mode is carried as hi = RNE16(x) plus
// lo = RNE16(x - hi); an operand in round mode is rounded once.  Each K step
// contributes the products hi*hi, hi*lo, lo*hi (those the modes provide) and
// optionally lo*lo.  The page's fix keeps the small products out of the
// accumulator that holds the large hi*hi sum: here the products go into
// CHAINS separate register accumulators,
//   CHAINS = 1: every product into one accumulator (the single-chain variant);
//   CHAINS = 2: hi*hi | all correction products;
//   CHAINS = 3: hi*hi | hi*lo | lo*hi (+ lo*lo);
// which are added in plain fp32 once, after the K loop: c0 + (c1 + c2).
//
// The split happens on load: fp32 tiles are read from global memory (16-byte
// loads), converted in registers, and the hi and lo parts are written to
// separate swizzled LDS tiles; the MFMA loop then reads 16-bit fragments
// exactly as the 16-bit GEMM does.
#pragma once
#include "gemm_core.hpp"

namespace mfl {

// Product set of one K step, as a compile-time descriptor.
template <bool SA_, bool SB_, int CHAINS_, bool LOLO_>
struct Products {
  static constexpr bool SA = SA_, SB = SB_, LOLO = LOLO_ && SA_ && SB_;
  static constexpr int CHAINS = CHAINS_;
  static constexpr int NPROD = 1 + (SB ? 1 : 0) + (SA ? 1 : 0) + (LOLO ? 1 : 0);
  static_assert(CHAINS >= 1 && CHAINS <= NPROD && CHAINS <= 3, "chains must not exceed the products");
  // product p in order: hh, [hl], [lh], [ll]; which operand halves it uses
  static constexpr bool a_lo(int p) { return (SB ? (p == 2 || p == 3) : (p == 1)); }
  static constexpr bool b_lo(int p) { return SB && (p == 1 || p == 3); }
  // chain of product p: 0 for hh; corrections go to chain 1 (two chains) or to
  // chains 1, 2, 2 (three chains)
  static constexpr int chain(int p) { return CHAINS == 1 || p == 0 ? 0 : (CHAINS == 2 ? 1 : (p == 1 ? 1 : 2)); }
};

// Loads one R x BK fp32 operand tile per stage and writes its 16-bit hi (and
// lo) parts to swizzled LDS tiles.  KC: K contiguous (element (r,k) at
// base[(r0+r)*ld + k0+k]); otherwise K strided (base[(k0+k)*ld + r0+r]).
// Each thread moves chunks of 8 values (two 16-byte loads).  EDGE: K positions
// past k_end, and (K strided) rows past rows_total, are zero; a vector that
// straddles the edge is read element by element, so no read leaves the
// operand's storage.  K-contiguous rows past rows_total repeat the last row and
// are never stored.
template <int R, int BK, int NT, bool KC, bool EDGE, bool SPLIT, int DT>
struct SplitLoader {
  static constexpr int CHUNKS = R * BK / 8;
  static constexpr int PER = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly among threads");
  f32x4 reg[PER][2];

  __device__ __forceinline__ void load(const float* __restrict__ base, int64_t ld, int r0, int k0, int rows_total,
                                       int k_end, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KC) {
        const int r = idx / (BK / 8), c = idx % (BK / 8);
        const int gr = EDGE ? min(r0 + r, rows_total - 1) : r0 + r;
        const int kf = k0 + c * 8;
        const float* p = base + (int64_t)gr * ld + kf;
        if (!EDGE || kf + 8 <= k_end) {
          reg[i][0] = *reinterpret_cast<const f32x4*>(p);
          reg[i][1] = *reinterpret_cast<const f32x4*>(p + 4);
        } else {  // K positions past k_end are zero and never read
          reg[i][0] = gload4_partial(p, k_end - kf);
          reg[i][1] = gload4_partial(p + 4, k_end - kf - 4);
        }
      } else {
        const int k = idx / (R / 8), rc = idx % (R / 8);
        const int gk = k0 + k, gr = r0 + rc * 8;
        const float* p = base + (int64_t)gk * ld + gr;
        if (!EDGE || (gk < k_end && gr + 8 <= rows_total)) {
          reg[i][0] = *reinterpret_cast<const f32x4*>(p);
          reg[i][1] = *reinterpret_cast<const f32x4*>(p + 4);
        } else if (gk < k_end) {  // rows past rows_total are zero and never read
          reg[i][0] = gload4_partial(p, rows_total - gr);
          reg[i][1] = gload4_partial(p + 4, rows_total - gr - 4);
        } else {
          reg[i][0] = z;
          reg[i][1] = z;
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* hi, uint16_t* lo, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NT;
      uint16_t h[8], l[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = reg[i][e >> 2][e & 3];
        h[e] = to16<DT>(x);
        if constexpr (SPLIT) l[e] = to16<DT>(x - from16<DT>(h[e]));
      }
      if constexpr (KC) {
        const int r = idx / (BK / 8), c = idx % (BK / 8);
        u32x4 v;
        __builtin_memcpy(&v, h, 16);
        lds_write16(hi, lds_chunk<BK>(r, c), v);
        if constexpr (SPLIT) {
          __builtin_memcpy(&v, l, 16);
          lds_write16(lo, lds_chunk<BK>(r, c), v);
        }
      } else {
        // k-major tile (the kmaj_chunk layout of the 16x16x32 instruction, as
        // the direct-to-LDS k-major slabs): the 8 rows rc*8 .. +7 at K row k
        // are one 16-byte chunk
        const int k = idx / (R / 8), rc = idx % (R / 8);
        u32x4 v;
        __builtin_memcpy(&v, h, 16);
        lds_write16(hi, lds_elemKM<0>(k, rc * 8), v);
        if constexpr (SPLIT) {
          __builtin_memcpy(&v, l, 16);
          lds_write16(lo, lds_elemKM<0>(k, rc * 8), v);
        }
      }
    }
  }
};

// Grid: x = output tiles, y = K slices.  Slice z covers K range
// [z*k_per_split, min(K, (z+1)*k_per_split)) and writes its result to
// C + z*c_split_stride (split K is used by the attention pair's second GEMM).
template <int BM, int BN, int WGM, int WGN, int DT, class P, bool AK, bool BKC, bool EDGE>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_split_kernel(const float* __restrict__ A,
                                                                    const float* __restrict__ B,
                                                                    float* __restrict__ C, int64_t lda, int64_t ldb,
                                                                    int64_t ldc, int M, int N, int K, int tiles_m,
                                                                    int tiles_n, int k_per_split,
                                                                    int64_t c_split_stride, int accumulate) {
  constexpr int BK = 64, SHAPE = 0;
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MN = Shape<SHAPE>::MN;
  constexpr int TM = WM / MN, TN = WN / MN;
  constexpr int TA = BM * BK, TB = BN * BK;
  constexpr int STAGE = TA * (P::SA ? 2 : 1) + TB * (P::SB ? 2 : 1);
  using Acc = typename Shape<SHAPE>::Acc;

  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, &tm, &tn);
  const int row0 = tm * BM, col0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr0 = (wave / WGN) * WM, wc0 = (wave % WGN) * WN;
  const int k_begin = blockIdx.y * k_per_split;
  const int k_end = min(K, k_begin + k_per_split);
  C += (int64_t)blockIdx.y * c_split_stride;

  // stage layout: A_hi | [A_lo] | B_hi | [B_lo]
  auto a_hi = [&](int s) { return lds + s * STAGE; };
  auto a_lo = [&](int s) { return lds + s * STAGE + TA; };
  auto b_hi = [&](int s) { return lds + s * STAGE + TA * (P::SA ? 2 : 1); };
  auto b_lo = [&](int s) { return lds + s * STAGE + TA * (P::SA ? 2 : 1) + TB; };

  // K-contiguous operands: swizzled row tiles read 16 bytes at a time;
  // K-strided ones: k-major tiles read with the transpose read.
  using RA = std::conditional_t<AK, FragOffsets<SHAPE, BK>, KmFrag<SHAPE, BM, WM, TM>>;
  using RB = std::conditional_t<BKC, FragOffsets<SHAPE, BK>, KmFrag<SHAPE, BN, WN, TN>>;
  const RA fa(wr0, lane);
  const RB fb(wc0, lane);
  Acc acc[P::CHAINS][TM][TN];
#pragma unroll
  for (int ch = 0; ch < P::CHAINS; ++ch) zero_acc<SHAPE, TM, TN>(acc[ch]);

  SplitLoader<BM, BK, NT, AK, EDGE, P::SA, DT> la;
  SplitLoader<BN, BK, NT, BKC, EDGE, P::SB, DT> lb;
  const int KT = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;
  if (KT > 0) {
    la.load(A, lda, row0, k_begin, M, k_end, tid);
    lb.load(B, ldb, col0, k_begin, N, k_end, tid);
    la.store(a_hi(0), a_lo(0), tid);
    lb.store(b_hi(0), b_lo(0), tid);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) {
        la.load(A, lda, row0, k_begin + (kt + 1) * BK, M, k_end, tid);
        lb.load(B, ldb, col0, k_begin + (kt + 1) * BK, N, k_end, tid);
      }
#pragma unroll
      for (int kk = 0; kk < FragOffsets<SHAPE, BK>::KSTEPS; ++kk) {
        u32x4 ah[TM], al[TM], bh[TN], bl[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          ah[i] = frag_read(a_hi(cur), fa, kk, i);
          if constexpr (P::SA) al[i] = frag_read(a_lo(cur), fa, kk, i);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          bh[j] = frag_read(b_hi(cur), fb, kk, j);
          if constexpr (P::SB) bl[j] = frag_read(b_lo(cur), fb, kk, j);
        }
        // Product-major order: between two products on one accumulator there
        // are TM*TN independent MFMAs, and within one accumulator the K step's
        // products arrive in the order hh, hl, lh, ll.
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
      if (more) {
        la.store(a_hi(cur ^ 1), a_lo(cur ^ 1), tid);
        lb.store(b_hi(cur ^ 1), b_lo(cur ^ 1), tid);
      }
      __syncthreads();
    }
  }
  // Sum the chains in plain fp32, the small ones first: c0 + (c1 + c2).
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (P::CHAINS == 3) acc[1][i][j] = acc[1][i][j] + acc[2][i][j];
      if constexpr (P::CHAINS >= 2) acc[0][i][j] = acc[0][i][j] + acc[1][i][j];
    }
  store_acc<SHAPE, TM, TN, EDGE>(C, ldc, row0 + wr0, col0 + wc0, M, N, lane, acc[0], accumulate);
}

// Launch helper used by the C ABI and by the attention pair.
// 128 x 128 tiles, 16 waves of 32 x 32 (four per SIMD; the tile's two LDS
// stages take 128 KiB, so one workgroup per CU): at 4096^3 with 3 chains
// 410 us against 439 us for 8 waves of 64 x 32 and 522 us for 4 of 64 x 64,
// bit-identical.
template <int DT, class P, bool AK, bool BKC>
inline int launch_split(const float* a, int64_t lda, const float* b, int64_t ldb, float* c, int64_t ldc, int M, int N,
                        int K, int splits, int k_per_split, int64_t c_split_stride, int accumulate, hipStream_t s) {
  constexpr int BM = 128, BN = 128, WGM = 4, WGN = 4;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const dim3 grid(tiles_m * tiles_n, splits), block(WGM * WGN * 64);
  if constexpr (AK && BKC) {
    const bool exact = M % BM == 0 && N % BN == 0 && k_per_split % 64 == 0 && K % k_per_split == 0;
    if (exact) {
      hipLaunchKernelGGL((gemm_split_kernel<BM, BN, WGM, WGN, DT, P, AK, BKC, false>), grid, block, 0, s, a, b, c,
                         lda, ldb, ldc, M, N, K, tiles_m, tiles_n, k_per_split, c_split_stride, accumulate);
      return launch_status();
    }
  }
  hipLaunchKernelGGL((gemm_split_kernel<BM, BN, WGM, WGN, DT, P, AK, BKC, true>), grid, block, 0, s, a, b, c, lda,
                     ldb, ldc, M, N, K, tiles_m, tiles_n, k_per_split, c_split_stride, accumulate);
  return launch_status();
}

// Selects the product set at run time.  Instantiated per (DT, orders) in
// separate translation units so that the kernels build in parallel.
template <int DT, bool AK, bool BKC>
int dispatch_split_modes(bool sa, bool sb, int chains, bool lolo, const float* a, int64_t lda, const float* b,
                         int64_t ldb, float* c, int64_t ldc, int M, int N, int K, int splits, int k_per_split,
                         int64_t c_split_stride, int accumulate, hipStream_t s) {
#define MFL_LAUNCH(SA, SB, CH, LL)                                                                            \
  return launch_split<DT, Products<SA, SB, CH, LL>, AK, BKC>(a, lda, b, ldb, c, ldc, M, N, K, splits, k_per_split, \
                                                             c_split_stride, accumulate, s)
  if (sa && sb) {
    if (lolo) {
      if (chains == 1) MFL_LAUNCH(true, true, 1, true);
      if (chains == 2) MFL_LAUNCH(true, true, 2, true);
      if (chains == 3) MFL_LAUNCH(true, true, 3, true);
    } else {
      if (chains == 1) MFL_LAUNCH(true, true, 1, false);
      if (chains == 2) MFL_LAUNCH(true, true, 2, false);
      if (chains == 3) MFL_LAUNCH(true, true, 3, false);
    }
  } else if (sa) {
    if (chains == 1) MFL_LAUNCH(true, false, 1, false);
    if (chains == 2) MFL_LAUNCH(true, false, 2, false);
  } else if (sb) {
    if (chains == 1) MFL_LAUNCH(false, true, 1, false);
    if (chains == 2) MFL_LAUNCH(false, true, 2, false);
  } else {
    if (chains == 1) MFL_LAUNCH(false, false, 1, false);
  }
#undef MFL_LAUNCH
  return MFL_EINVAL;
}

#define MFL_DECLARE_SPLIT(DT, AK, BKC)                                                                               \
  extern template int dispatch_split_modes<DT, AK, BKC>(bool, bool, int, bool, const float*, int64_t, const float*, \
                                                         int64_t, float*, int64_t, int, int, int, int, int, int64_t,  \
                                                         int, hipStream_t)
#define MFL_INSTANTIATE_SPLIT(DT, AK, BKC)                                                                    \
  template int dispatch_split_modes<DT, AK, BKC>(bool, bool, int, bool, const float*, int64_t, const float*, \
                                                  int64_t, float*, int64_t, int, int, int, int, int, int64_t,  \
                                                  int, hipStream_t)
#define MFL_FOR_ORDERS(X, DT) X(DT, true, true); X(DT, true, false); X(DT, false, true); X(DT, false, false)
MFL_FOR_ORDERS(MFL_DECLARE_SPLIT, MFL_F16);
MFL_FOR_ORDERS(MFL_DECLARE_SPLIT, MFL_BF16);

}  // namespace mfl
