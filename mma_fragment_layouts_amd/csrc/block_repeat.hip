// gemm_block_repeat: the block-GEMM repeat workload of Warp issue #1965
// ("Spike" section).  Every workgroup loads one A tile (TM x TK) and one B tile
// (TK x TN) into LDS once, then runs `repeats` back-to-back TM x TN x TK block
// MMAs into one register accumulator, reading the operand fragments from LDS on
// every repeat (as a block-level GEMM call does), and stores the tile once.
// With no HBM traffic in the loop, it measures the LDS -> MFMA path itself.
//
// LDS_API = true is the issue's other arm, the shared-memory pointer API
// ("Description": A, B and C are plain shared-memory tiles and every call
// computes C = A*B + C in place): A and B sit in LDS unswizzled, and on every
// repeat each wave reads its part of C from an fp32 LDS tile into registers,
// runs the block MMA and writes C back, with a workgroup barrier between calls.
// It exists to measure the two costs the issue names — bank conflicts of
// fragment reads from plain layouts, and the C round trip — on this hardware.
// In the register arm a repeat of one MFMA K step (TK = 32) reads the next
// repeat's fragments while its MFMAs issue; deeper repeats overlap inside the
// repeat instead.
#include "gemm_core.hpp"

namespace mfl {

template <int TM_, int TN_, int TK, int WGM, int WGN, int SHAPE, int DT, bool LDS_API>
__global__ __launch_bounds__(WGM* WGN * 64) void block_repeat_kernel(const uint16_t* __restrict__ A,
                                                                      const uint16_t* __restrict__ B,
                                                                      float* __restrict__ C, int64_t ldc,
                                                                      int tiles_m, int tiles_n, int repeats) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = TM_ / WGM, WN = TN_ / WGN;
  constexpr int MN = Shape<SHAPE>::MN;
  constexpr int FM = WM / MN, FN = WN / MN;
  static_assert(FM * MN == WM && FN * MN == WN, "wave tile must be a multiple of the MFMA tile");
  using Acc = typename Shape<SHAPE>::Acc;

  constexpr int C_ELEMS = LDS_API ? TM_ * TN_ * 2 : 0;  // fp32 C tile, in 16-bit units
  __shared__ __attribute__((aligned(16))) uint16_t lds[(TM_ + TN_) * TK + C_ELEMS];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, &tm, &tn);
  const int row0 = tm * TM_, col0 = tn * TN_;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr0 = (wave / WGN) * WM, wc0 = (wave % WGN) * WN;
  Acc acc[FM][FN];
  zero_acc<SHAPE, FM, FN>(acc);

  if constexpr (!LDS_API) {
    {
      TileLoader<TM_, TK, NT, true, false> la;
      TileLoader<TN_, TK, NT, true, false> lb;
      la.load(A, TK, row0, 0, 0, TK, tid);
      lb.load(B, TK, col0, 0, 0, TK, tid);
      la.store(lds, tid);
      lb.store(lds + TM_ * TK, tid);
    }
    __syncthreads();
    const FragOffsets<SHAPE, TK> fa(wr0, lane), fb(wc0, lane);
    constexpr int KS = TK / Shape<SHAPE>::K;  // MFMA K steps per repeat
    if constexpr (KS > 1) {
      for (int r = 0; r < repeats; ++r) {
        // Each repeat is a separate block GEMM: its fragments come from LDS
        // again (the memory clobber keeps the compiler from reusing registers).
        // Within a repeat the reads of K step kk+1 overlap the MFMAs of kk.
        asm volatile("" ::: "memory");
        mma_slab<SHAPE, DT, FM, FN, TK>(lds, lds + TM_ * TK, fa, fb, acc);
      }
    } else {
      // One MFMA K step per repeat: the next repeat's fragments are read from
      // LDS (after the clobber, so they are read again) into the other of two
      // register sets while this repeat's MFMAs issue.  Same MFMAs, same order.
      u32x4 xa[2][FM], xb[2][FN];
      auto rd = [&](int f) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < FM; ++i) xa[f][i] = frag_read(lds, fa, 0, i);
#pragma unroll
        for (int j = 0; j < FN; ++j) xb[f][j] = frag_read(lds + TM_ * TK, fb, 0, j);
      };
      auto mm = [&](int f) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma<SHAPE, DT>(xa[f][i], xb[f][j], acc[i][j]);
      };
      if (repeats > 0) rd(0);
      int r = 0;
      for (; r + 1 < repeats; r += 2) {
        rd(1);
        mm(0);
        if (r + 2 < repeats) rd(0);
        mm(1);
      }
      if (r < repeats) mm(0);
    }
  } else {
    // Plain tiles: A rows (row-major, K contiguous), B columns (K contiguous),
    // 16-byte chunk c of row r at r*TK + 8c; C fp32 row-major TM x TN.
    constexpr int ACH = TM_ * TK / 8, CH = (TM_ + TN_) * TK / 8;
    for (int c = tid; c < CH; c += NT) {
      const bool isa = c < ACH;
      const int cc = isa ? c : c - ACH;
      const int r = cc / (TK / 8), k8 = cc % (TK / 8);
      const uint16_t* src = (isa ? A + (int64_t)(row0 + r) * TK : B + (int64_t)(col0 + r) * TK) + k8 * 8;
      *reinterpret_cast<u32x4*>(lds + (isa ? 0 : TM_ * TK) + r * TK + k8 * 8) = *reinterpret_cast<const u32x4*>(src);
    }
    float* cl = reinterpret_cast<float*>(lds + (TM_ + TN_) * TK);
    constexpr AccLayout L = acc_layout(SHAPE);
    auto c_at = [&](int fm, int fn, int j) {
      return (wr0 + fm * MN + acc_row(L, lane, j)) * TN_ + wc0 + fn * MN + acc_col(L, lane, j);
    };
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int j = 0; j < L.per_lane; ++j) cl[c_at(fm, fn, j)] = 0.f;
    __syncthreads();
    const FragOffsets<SHAPE, TK> fa(wr0, lane, typename FragOffsets<SHAPE, TK>::Plain{}),
        fb(wc0, lane, typename FragOffsets<SHAPE, TK>::Plain{});
    for (int r = 0; r < repeats; ++r) {
      // one shared-memory-API call: C in from LDS, C += A B, C back to LDS
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int j = 0; j < L.per_lane; ++j) acc[fm][fn][j] = cl[c_at(fm, fn, j)];
      mma_slab<SHAPE, DT, FM, FN, TK>(lds, lds + TM_ * TK, fa, fb, acc);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int j = 0; j < L.per_lane; ++j) cl[c_at(fm, fn, j)] = acc[fm][fn][j];
      __syncthreads();
    }
  }
  store_acc<SHAPE, FM, FN, false>(C, ldc, row0 + wr0, col0 + wc0, 0, 0, lane, acc, 0);
}

template <int TM_, int TN_, int TK, int WGM, int WGN, int DT, bool LDS_API>
static int launch_repeat(const void* a, const void* b, float* c, int M, int N, int repeats, hipStream_t s) {
  const int tiles_m = M / TM_, tiles_n = N / TN_;
  hipLaunchKernelGGL((block_repeat_kernel<TM_, TN_, TK, WGM, WGN, 0, DT, LDS_API>), dim3(tiles_m * tiles_n),
                     dim3(WGM * WGN * 64), 0, s, (const uint16_t*)a, (const uint16_t*)b, c, (int64_t)N, tiles_m,
                     tiles_n, repeats);
  return launch_status();
}

template <int DT, bool LDS_API>
static int dispatch_repeat(int tm, int tn, int tk, int threads, const void* a, const void* b, float* c, int M, int N,
                           int repeats, hipStream_t s) {
  if (tm == 64 && tn == 64 && tk == 64) {
    if (threads == 64) return launch_repeat<64, 64, 64, 1, 1, DT, LDS_API>(a, b, c, M, N, repeats, s);
    if (threads == 128) return launch_repeat<64, 64, 64, 2, 1, DT, LDS_API>(a, b, c, M, N, repeats, s);
    if (threads == 256) return launch_repeat<64, 64, 64, 2, 2, DT, LDS_API>(a, b, c, M, N, repeats, s);
  } else if (tm == 32 && tn == 32 && tk == 32) {
    if (threads == 128) return launch_repeat<32, 32, 32, 2, 1, DT, LDS_API>(a, b, c, M, N, repeats, s);
  } else if (tm == 128 && tn == 128 && tk == 32) {
    if (threads == 128) return launch_repeat<128, 128, 32, 2, 1, DT, LDS_API>(a, b, c, M, N, repeats, s);
    if (threads == 256) return launch_repeat<128, 128, 32, 2, 2, DT, LDS_API>(a, b, c, M, N, repeats, s);
  }
  return MFL_EUNSUPPORTED;
}

static bool supported(int tm, int tn, int tk, int threads) {
  return (tm == 64 && tn == 64 && tk == 64 && (threads == 64 || threads == 128 || threads == 256)) ||
         (tm == 32 && tn == 32 && tk == 32 && threads == 128) ||
         (tm == 128 && tn == 128 && tk == 32 && (threads == 128 || threads == 256));
}

}  // namespace mfl

using namespace mfl;

template <bool LDS_API>
static int block_repeat_entry(int dtype, int tm, int tn, int tk, int threads, int repeats, int64_t m, int64_t n,
                              const void* a, const void* b, float* c, void* stream) {
  if (dtype != MFL_F16 && dtype != MFL_BF16) return MFL_EINVAL;
  if (tm <= 0 || tn <= 0 || tk <= 0 || threads <= 0 || repeats < 0 || m < 0 || n < 0) return MFL_EINVAL;
  if (!supported(tm, tn, tk, threads)) return MFL_EUNSUPPORTED;
  if (m % tm != 0 || n % tn != 0) return MFL_EUNSUPPORTED;
  if (m > INT32_MAX || n > INT32_MAX || (m / tm) * (n / tn) > INT32_MAX) return MFL_EUNSUPPORTED;
  if (m == 0 || n == 0) return MFL_OK;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || ((uintptr_t)c & 3)) return MFL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MFL_BF16)
    return dispatch_repeat<MFL_BF16, LDS_API>(tm, tn, tk, threads, a, b, c, (int)m, (int)n, repeats, s);
  return dispatch_repeat<MFL_F16, LDS_API>(tm, tn, tk, threads, a, b, c, (int)m, (int)n, repeats, s);
}

extern "C" int gemm_block_repeat(int dtype, int tm, int tn, int tk, int threads, int repeats, int64_t m, int64_t n,
                                 const void* a, const void* b, float* c, void* stream) {
  return block_repeat_entry<false>(dtype, tm, tn, tk, threads, repeats, m, n, a, b, c, stream);
}

extern "C" int gemm_block_repeat_lds_api(int dtype, int tm, int tn, int tk, int threads, int repeats, int64_t m,
                                         int64_t n, const void* a, const void* b, float* c, void* stream) {
  return block_repeat_entry<true>(dtype, tm, tn, tk, threads, repeats, m, n, a, b, c, stream);
}
