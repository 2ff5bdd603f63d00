// C ABI of the accumulator- and operand-fragment layouts (host), the strided
// epilogue store, the strided operand load and the single-MFMA probe (device),
// status strings.
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

bool valid_operand(int operand) { return operand == MFL_OPERAND_A || operand == MFL_OPERAND_B; }

bool valid_operand_point(int shape, int lane, int i) {
  const AccLayout& L = operand_layout(shape);
  return lane >= 0 && lane < L.lanes && i >= 0 && i < L.per_lane;
}

// (row, col) of operand element i of `lane` as the operand is written: (m, k)
// for A, (k, n) for B, from the K-contiguous numeral offset mn*K + k.
MFL_HD constexpr void operand_rc(const AccLayout& L, int operand, int lane, int i, int* row, int* col) {
  const int off = mfl::acc_offset(L, lane, i);
  const int mn = off / L.cols, k = off % L.cols;
  *row = operand == MFL_OPERAND_A ? mn : k;
  *col = operand == MFL_OPERAND_A ? k : mn;
}

// One wave: gather each lane's 8 operand elements from a strided matrix.
template <int SHAPE>
__global__ __launch_bounds__(64) void operand_load_kernel(const uint16_t* __restrict__ m, int64_t row0, int64_t col0,
                                                         int64_t ld, int order, int operand,
                                                         uint16_t* __restrict__ frag) {
  constexpr AccLayout L = operand_layout(SHAPE);
  const int lane = threadIdx.x;
#pragma unroll
  for (int i = 0; i < L.per_lane; ++i) {
    int r, c;
    operand_rc(L, operand, lane, i, &r, &c);
    const int64_t idx = order == MFL_ROW_MAJOR ? (row0 + r) * ld + col0 + c : (col0 + c) * ld + row0 + r;
    frag[lane * L.per_lane + i] = m[idx];
  }
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
    case MFL_ESCRATCH: return "MFL_ESCRATCH: needs more than the static scratch array holds";
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

extern "C" int mfl_operand_info(int shape, int operand, int* lanes, int* per_lane, int* rows, int* cols) {
  if (!valid_shape(shape) || !valid_operand(operand) || !lanes || !per_lane || !rows || !cols) return MFL_EINVAL;
  const AccLayout& L = operand_layout(shape);  // rows = MN, cols = K
  *lanes = L.lanes;
  *per_lane = L.per_lane;
  *rows = operand == MFL_OPERAND_A ? L.rows : L.cols;
  *cols = operand == MFL_OPERAND_A ? L.cols : L.rows;
  return MFL_OK;
}

extern "C" int operand_coords(int shape, int operand, int lane, int i, int* row, int* col) {
  if (!valid_shape(shape) || !valid_operand(operand) || !row || !col || !valid_operand_point(shape, lane, i))
    return MFL_EINVAL;
  operand_rc(operand_layout(shape), operand, lane, i, row, col);
  return MFL_OK;
}

extern "C" int operand_offset(int shape, int operand, int lane, int i, int* offset) {
  if (!valid_shape(shape) || !valid_operand(operand) || !offset || !valid_operand_point(shape, lane, i))
    return MFL_EINVAL;
  *offset = mfl::acc_offset(operand_layout(shape), lane, i);
  return MFL_OK;
}

extern "C" int operand_decode(int shape, int operand, int offset, int* lane, int* i) {
  if (!valid_shape(shape) || !valid_operand(operand) || !lane || !i) return MFL_EINVAL;
  const AccLayout& L = operand_layout(shape);
  if (offset < 0 || offset >= L.rows * L.cols) return MFL_EINVAL;
  mfl::acc_decode(L, offset, lane, i);
  return MFL_OK;
}

extern "C" int operand_matrix_offset(int shape, int operand, int lane, int i, int64_t row0, int64_t col0, int64_t ld,
                                     int order, int64_t* out) {
  if (!valid_shape(shape) || !valid_operand(operand) || !out || !valid_operand_point(shape, lane, i)) return MFL_EINVAL;
  if (row0 < 0 || col0 < 0 || ld <= 0 || (order != MFL_ROW_MAJOR && order != MFL_COL_MAJOR)) return MFL_EINVAL;
  int r, c;
  operand_rc(operand_layout(shape), operand, lane, i, &r, &c);
  // outer / inner: the strided and the contiguous coordinate of the element
  const int64_t o0 = order == MFL_ROW_MAJOR ? row0 : col0, i0 = order == MFL_ROW_MAJOR ? col0 : row0;
  const int ro = order == MFL_ROW_MAJOR ? r : c, ri = order == MFL_ROW_MAJOR ? c : r;
  int64_t outer, inner, t, o;
  if (__builtin_add_overflow(i0, (int64_t)ri, &inner)) return MFL_EOVERFLOW;
  if (inner >= ld) return MFL_EOVERFLOW;  // would spill into the next row / column
  if (__builtin_add_overflow(o0, (int64_t)ro, &outer)) return MFL_EOVERFLOW;
  if (__builtin_mul_overflow(outer, ld, &t)) return MFL_EOVERFLOW;
  if (__builtin_add_overflow(t, inner, &o)) return MFL_EOVERFLOW;
  *out = o;
  return MFL_OK;
}

extern "C" int operand_load_strided(int shape, int operand, const void* m, int64_t row0, int64_t col0, int64_t ld,
                                    int order, void* frag, void* stream) {
  if (!valid_shape(shape) || !valid_operand(operand) || !m || !frag) return MFL_EINVAL;
  if (row0 < 0 || col0 < 0 || ld <= 0 || (order != MFL_ROW_MAJOR && order != MFL_COL_MAJOR)) return MFL_EINVAL;
  if (((uintptr_t)m & 1) || ((uintptr_t)frag & 1)) return MFL_EINVAL;
  int lanes, per_lane, rows, cols;
  mfl_operand_info(shape, operand, &lanes, &per_lane, &rows, &cols);
  // The tile's last element must fit: contiguous extent within ld, offset in int64.
  const int64_t o0 = order == MFL_ROW_MAJOR ? row0 : col0, i0 = order == MFL_ROW_MAJOR ? col0 : row0;
  const int no = order == MFL_ROW_MAJOR ? rows : cols, ni = order == MFL_ROW_MAJOR ? cols : rows;
  int64_t last, t;
  if (i0 > ld - ni) return MFL_EOVERFLOW;
  if (__builtin_add_overflow(o0, (int64_t)(no - 1), &last) || __builtin_mul_overflow(last, ld, &t) ||
      __builtin_add_overflow(t, i0 + ni - 1, &t))
    return MFL_EOVERFLOW;
  hipStream_t s = (hipStream_t)stream;
  if (shape == MFL_MFMA_16X16X32)
    hipLaunchKernelGGL(operand_load_kernel<0>, dim3(1), dim3(64), 0, s, (const uint16_t*)m, row0, col0, ld, order,
                       operand, (uint16_t*)frag);
  else
    hipLaunchKernelGGL(operand_load_kernel<1>, dim3(1), dim3(64), 0, s, (const uint16_t*)m, row0, col0, ld, order,
                       operand, (uint16_t*)frag);
  return launch_status();
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
