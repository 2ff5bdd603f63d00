// gemm_block_repeat: the block-GEMM repeat workload of Warp issue #1965
// ("Spike" section).  Every workgroup loads one A tile (TM x TK) and one B tile
// (TK x TN) into LDS once, then runs `repeats` back-to-back TM x TN x TK block
// MMAs into one register accumulator, reading the operand fragments from LDS on
// every repeat (as a block-level GEMM call does), and stores the tile once.
// With no HBM traffic in the loop, it measures the LDS -> MFMA path itself.
#include "gemm_core.hpp"

namespace mfl {

template <int TM_, int TN_, int TK, int WGM, int WGN, int SHAPE, int DT>
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

  __shared__ __attribute__((aligned(16))) uint16_t lds[(TM_ + TN_) * TK];

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, 4, &tm, &tn);
  const int row0 = tm * TM_, col0 = tn * TN_;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr0 = (wave / WGN) * WM, wc0 = (wave % WGN) * WN;

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
  Acc acc[FM][FN];
  zero_acc<SHAPE, FM, FN>(acc);
  for (int r = 0; r < repeats; ++r) {
    // Each repeat is a separate block GEMM: its fragments come from LDS again.
    asm volatile("" ::: "memory");
    mma_slab<SHAPE, DT, FM, FN, TK>(lds, lds + TM_ * TK, fa, fb, acc);
  }
  store_acc<SHAPE, FM, FN, false>(C, ldc, row0 + wr0, col0 + wc0, 0, 0, lane, acc, 0);
}

template <int TM_, int TN_, int TK, int WGM, int WGN, int DT>
static int launch_repeat(const void* a, const void* b, float* c, int M, int N, int repeats, hipStream_t s) {
  const int tiles_m = M / TM_, tiles_n = N / TN_;
  hipLaunchKernelGGL((block_repeat_kernel<TM_, TN_, TK, WGM, WGN, 0, DT>), dim3(tiles_m * tiles_n),
                     dim3(WGM * WGN * 64), 0, s, (const uint16_t*)a, (const uint16_t*)b, c, (int64_t)N, tiles_m,
                     tiles_n, repeats);
  return launch_status();
}

template <int DT>
static int dispatch_repeat(int tm, int tn, int tk, int threads, const void* a, const void* b, float* c, int M, int N,
                           int repeats, hipStream_t s) {
  if (tm == 64 && tn == 64 && tk == 64) {
    if (threads == 64) return launch_repeat<64, 64, 64, 1, 1, DT>(a, b, c, M, N, repeats, s);
    if (threads == 128) return launch_repeat<64, 64, 64, 2, 1, DT>(a, b, c, M, N, repeats, s);
    if (threads == 256) return launch_repeat<64, 64, 64, 2, 2, DT>(a, b, c, M, N, repeats, s);
  } else if (tm == 32 && tn == 32 && tk == 32) {
    if (threads == 128) return launch_repeat<32, 32, 32, 2, 1, DT>(a, b, c, M, N, repeats, s);
  } else if (tm == 128 && tn == 128 && tk == 32) {
    if (threads == 128) return launch_repeat<128, 128, 32, 2, 1, DT>(a, b, c, M, N, repeats, s);
    if (threads == 256) return launch_repeat<128, 128, 32, 2, 2, DT>(a, b, c, M, N, repeats, s);
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

extern "C" int gemm_block_repeat(int dtype, int tm, int tn, int tk, int threads, int repeats, int64_t m, int64_t n,
                                 const void* a, const void* b, float* c, void* stream) {
  if (dtype != MFL_F16 && dtype != MFL_BF16) return MFL_EINVAL;
  if (tm <= 0 || tn <= 0 || tk <= 0 || threads <= 0 || repeats < 0 || m < 0 || n < 0) return MFL_EINVAL;
  if (!supported(tm, tn, tk, threads)) return MFL_EUNSUPPORTED;
  if (m % tm != 0 || n % tn != 0) return MFL_EUNSUPPORTED;
  if (m > INT32_MAX || n > INT32_MAX || (m / tm) * (n / tn) > INT32_MAX) return MFL_EUNSUPPORTED;
  if (m == 0 || n == 0) return MFL_OK;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || ((uintptr_t)c & 3)) return MFL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == MFL_BF16) return dispatch_repeat<MFL_BF16>(tm, tn, tk, threads, a, b, c, (int)m, (int)n, repeats, s);
  return dispatch_repeat<MFL_F16>(tm, tn, tk, threads, a, b, c, (int)m, (int)n, repeats, s);
}
