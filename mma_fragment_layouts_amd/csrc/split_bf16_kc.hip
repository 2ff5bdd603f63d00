// Split-precision GEMM kernels with bf16 pieces, both operands K-contiguous.
#include "gemm_split.hpp"

namespace mfl {
MFL_INSTANTIATE_SPLIT(MFL_BF16, true, true);
}  // namespace mfl
