// C ABI of the split-precision fp32 GEMM (kernels in gemm_split.hpp).
#include "gemm_split.hpp"

namespace mfl {

// Validates one fp32 operand of `rows` x `cols` (logical) stored in `order`.
static int check32(const void* p, int64_t rows, int64_t cols, int64_t ld, int order) {
  if (order != MFL_ROW_MAJOR && order != MFL_COL_MAJOR) return MFL_EINVAL;
  if (rows == 0 || cols == 0) return MFL_OK;
  if (!p || !aligned16(p) || ld <= 0 || ld % 4 != 0) return MFL_EINVAL;
  const int64_t inner = order == MFL_ROW_MAJOR ? cols : rows;
  const int64_t outer = order == MFL_ROW_MAJOR ? rows : cols;
  if (ld < inner) return MFL_EINVAL;
  if (outer > INT64_MAX / ld) return MFL_EOVERFLOW;
  return MFL_OK;
}

template <int DT>
static int split_orders(bool ak, bool bk, bool sa, bool sb, int chains, bool lolo, const float* a, int64_t lda,
                        const float* b, int64_t ldb, float* c, int64_t ldc, int M, int N, int K, int accumulate,
                        hipStream_t s) {
  const int kps = K > 0 ? K : 1;
  if (ak && bk)
    return dispatch_split_modes<DT, true, true>(sa, sb, chains, lolo, a, lda, b, ldb, c, ldc, M, N, K, 1, kps, 0,
                                                accumulate, s);
  if (ak)
    return dispatch_split_modes<DT, true, false>(sa, sb, chains, lolo, a, lda, b, ldb, c, ldc, M, N, K, 1, kps, 0,
                                                 accumulate, s);
  if (bk)
    return dispatch_split_modes<DT, false, true>(sa, sb, chains, lolo, a, lda, b, ldb, c, ldc, M, N, K, 1, kps, 0,
                                                 accumulate, s);
  return dispatch_split_modes<DT, false, false>(sa, sb, chains, lolo, a, lda, b, ldb, c, ldc, M, N, K, 1, kps, 0,
                                                accumulate, s);
}

}  // namespace mfl

using namespace mfl;

extern "C" int gemm_split_fp32(int piece, int64_t m, int64_t n, int64_t k, const float* a, int64_t lda, int order_a,
                               int mode_a, const float* b, int64_t ldb, int order_b, int mode_b, int chains, int lolo,
                               float* c, int64_t ldc, int accumulate, void* stream) {
  if (piece != MFL_F16 && piece != MFL_BF16) return MFL_EINVAL;
  if ((mode_a != MFL_ROUND && mode_a != MFL_SPLIT) || (mode_b != MFL_ROUND && mode_b != MFL_SPLIT)) return MFL_EINVAL;
  if ((lolo != 0 && lolo != 1) || (accumulate != 0 && accumulate != 1)) return MFL_EINVAL;
  const bool sa = mode_a == MFL_SPLIT, sb = mode_b == MFL_SPLIT;
  const int nprod = 1 + (sa ? 1 : 0) + (sb ? 1 : 0) + (lolo && sa && sb ? 1 : 0);
  if (chains < 1 || chains > 3 || chains > nprod) return MFL_EINVAL;
  if (lolo && !(sa && sb)) return MFL_EINVAL;
  if (m < 0 || n < 0 || k < 0) return MFL_EINVAL;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return MFL_EUNSUPPORTED;
  int st;
  if ((st = check32(a, m, k, lda, order_a)) != MFL_OK) return st;
  if ((st = check32(b, k, n, ldb, order_b)) != MFL_OK) return st;
  if (m == 0 || n == 0) return MFL_OK;
  if (!c || ((uintptr_t)c & 3) || ldc < n) return MFL_EINVAL;
  if (m > INT64_MAX / ldc) return MFL_EOVERFLOW;
  const bool ak = order_a == MFL_ROW_MAJOR, bk = order_b == MFL_COL_MAJOR;
  hipStream_t s = (hipStream_t)stream;
  if (piece == MFL_BF16)
    return split_orders<MFL_BF16>(ak, bk, sa, sb, chains, lolo, a, lda, b, ldb, c, ldc, (int)m, (int)n, (int)k,
                                  accumulate, s);
  return split_orders<MFL_F16>(ak, bk, sa, sb, chains, lolo, a, lda, b, ldb, c, ldc, (int)m, (int)n, (int)k,
                               accumulate, s);
}
