// C ABI of the accumulator-fragment layout (host), the strided epilogue store
// and the single-MFMA probe (device), status strings.
//
// cuda-oxide PR #474, section "API": acc_coords, acc_offset, acc_matrix_offset
// (None on overflow) and acc_decode, here for the CDNA4 accumulator layouts and
// written against the numeral in layout.hpp.
#include "common.hpp"

using namespace mfl;

namespace {

bool valid_shape(int shape) { return shape == MFL_MFMA_16X16X32 || shape == MFL_MFMA_32X32X16; }

bool valid_point(int shape, int lane, int j) {
  const AccLayout& L = acc_layout(shape);
  return lane >= 0 && lane < L.lanes && j >= 0 && j < L.per_lane;
}

// One wave: write lane-major accumulator values through the layout.
template <int SHAPE>
__global__ __launch_bounds__(64) void acc_store_kernel(const float* __restrict__ acc, float* __restrict__ C,
                                                      int64_t row0, int64_t col0, int64_t ldc) {
  constexpr AccLayout L = acc_layout(SHAPE);
  const int lane = threadIdx.x;
#pragma unroll
  for (int j = 0; j < L.per_lane; ++j)
    C[(row0 + acc_row(L, lane, j)) * ldc + col0 + acc_col(L, lane, j)] = acc[lane * L.per_lane + j];
}

// One wave, one MFMA, zero accumulator in; raw registers out lane-major.
template <int SHAPE, int DT>
__global__ __launch_bounds__(64) void mfma_probe_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                                       const float* __restrict__ c_in, float* __restrict__ out) {
  const int lane = threadIdx.x;
  const u32x4 av = *reinterpret_cast<const u32x4*>(a + lane * 8);
  const u32x4 bv = *reinterpret_cast<const u32x4*>(b + lane * 8);
  typename Shape<SHAPE>::Acc c;
#pragma unroll
  for (int j = 0; j < Shape<SHAPE>::J; ++j) c[j] = c_in ? c_in[lane * Shape<SHAPE>::J + j] : 0.f;
  c = mfma<SHAPE, DT>(av, bv, c);
#pragma unroll
  for (int j = 0; j < Shape<SHAPE>::J; ++j) out[lane * Shape<SHAPE>::J + j] = c[j];
}

}  // namespace

extern "C" const char* mfl_status_string(int status) {
  switch (status) {
    case MFL_OK: return "MFL_OK";
    case MFL_EINVAL: return "MFL_EINVAL: invalid argument";
    case MFL_EOVERFLOW: return "MFL_EOVERFLOW: result does not fit";
    case MFL_EUNSUPPORTED: return "MFL_EUNSUPPORTED: not implemented for these arguments";
    case MFL_EHIP: return "MFL_EHIP: HIP launch failed";
    default: return "unknown mfl status";
  }
}

extern "C" int mfl_version(void) { return 100; }

extern "C" int mfl_acc_info(int shape, int* lanes, int* per_lane, int* rows, int* cols) {
  if (!valid_shape(shape) || !lanes || !per_lane || !rows || !cols) return MFL_EINVAL;
  const AccLayout& L = acc_layout(shape);
  *lanes = L.lanes;
  *per_lane = L.per_lane;
  *rows = L.rows;
  *cols = L.cols;
  return MFL_OK;
}

extern "C" int acc_coords(int shape, int lane, int j, int* row, int* col) {
  if (!valid_shape(shape) || !row || !col || !valid_point(shape, lane, j)) return MFL_EINVAL;
  const AccLayout& L = acc_layout(shape);
  *row = acc_row(L, lane, j);
  *col = acc_col(L, lane, j);
  return MFL_OK;
}

extern "C" int acc_offset(int shape, int lane, int j, int* offset) {
  if (!valid_shape(shape) || !offset || !valid_point(shape, lane, j)) return MFL_EINVAL;
  *offset = mfl::acc_offset(acc_layout(shape), lane, j);
  return MFL_OK;
}

extern "C" int acc_decode(int shape, int offset, int* lane, int* j) {
  if (!valid_shape(shape) || !lane || !j) return MFL_EINVAL;
  const AccLayout& L = acc_layout(shape);
  if (offset < 0 || offset >= L.rows * L.cols) return MFL_EINVAL;
  mfl::acc_decode(L, offset, lane, j);
  return MFL_OK;
}

extern "C" int acc_matrix_offset(int shape, int lane, int j, int64_t row0, int64_t col0, int64_t ld, int64_t* out) {
  if (!valid_shape(shape) || !out || !valid_point(shape, lane, j)) return MFL_EINVAL;
  if (row0 < 0 || col0 < 0 || ld <= 0) return MFL_EINVAL;
  const AccLayout& L = acc_layout(shape);
  int64_t r, c, rl, o;
  if (__builtin_add_overflow(col0, (int64_t)acc_col(L, lane, j), &c)) return MFL_EOVERFLOW;
  if (c >= ld) return MFL_EOVERFLOW;  // would spill into the next row
  if (__builtin_add_overflow(row0, (int64_t)acc_row(L, lane, j), &r)) return MFL_EOVERFLOW;
  if (__builtin_mul_overflow(r, ld, &rl)) return MFL_EOVERFLOW;
  if (__builtin_add_overflow(rl, c, &o)) return MFL_EOVERFLOW;
  *out = o;
  return MFL_OK;
}

extern "C" int acc_store_strided(int shape, const float* acc, float* c, int64_t row0, int64_t col0, int64_t ldc,
                                 void* stream) {
  if (!valid_shape(shape) || !acc || !c || row0 < 0 || col0 < 0 || ldc <= 0) return MFL_EINVAL;
  const AccLayout& L = acc_layout(shape);
  // The tile's last element, (row0 + rows - 1) * ldc + col0 + cols - 1, must fit.
  int64_t rlast, t;
  if (col0 > ldc - L.cols) return MFL_EOVERFLOW;
  if (__builtin_add_overflow(row0, (int64_t)(L.rows - 1), &rlast) || __builtin_mul_overflow(rlast, ldc, &t) ||
      __builtin_add_overflow(t, col0 + L.cols - 1, &t))
    return MFL_EOVERFLOW;
  hipStream_t s = (hipStream_t)stream;
  if (shape == MFL_MFMA_16X16X32)
    hipLaunchKernelGGL(acc_store_kernel<0>, dim3(1), dim3(64), 0, s, acc, c, row0, col0, ldc);
  else
    hipLaunchKernelGGL(acc_store_kernel<1>, dim3(1), dim3(64), 0, s, acc, c, row0, col0, ldc);
  return launch_status();
}

extern "C" int mfma_probe(int shape, int dtype, const void* a_frag, const void* b_frag, const float* c_in, float* acc,
                          void* stream) {
  if (!valid_shape(shape) || (dtype != MFL_F16 && dtype != MFL_BF16)) return MFL_EINVAL;
  if (!a_frag || !b_frag || !acc || !aligned16(a_frag) || !aligned16(b_frag)) return MFL_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* a = (const uint16_t*)a_frag;
  const uint16_t* b = (const uint16_t*)b_frag;
  if (shape == MFL_MFMA_16X16X32 && dtype == MFL_BF16)
    hipLaunchKernelGGL((mfma_probe_kernel<0, MFL_BF16>), dim3(1), dim3(64), 0, s, a, b, c_in, acc);
  else if (shape == MFL_MFMA_16X16X32)
    hipLaunchKernelGGL((mfma_probe_kernel<0, MFL_F16>), dim3(1), dim3(64), 0, s, a, b, c_in, acc);
  else if (dtype == MFL_BF16)
    hipLaunchKernelGGL((mfma_probe_kernel<1, MFL_BF16>), dim3(1), dim3(64), 0, s, a, b, c_in, acc);
  else
    hipLaunchKernelGGL((mfma_probe_kernel<1, MFL_F16>), dim3(1), dim3(64), 0, s, a, b, c_in, acc);
  return launch_status();
}
