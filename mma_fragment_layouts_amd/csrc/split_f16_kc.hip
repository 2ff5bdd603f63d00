// Split-precision GEMM kernels with f16 pieces, both operands K-contiguous.
#include "gemm_split.hpp"

namespace mfl {
MFL_INSTANTIATE_SPLIT(MFL_F16, true, true);
}  // namespace mfl
