// Split-precision GEMM kernels with bf16 pieces, at least one operand K-strided.
#include "gemm_split.hpp"

namespace mfl {
MFL_INSTANTIATE_SPLIT(MFL_BF16, true, false);
MFL_INSTANTIATE_SPLIT(MFL_BF16, false, true);
MFL_INSTANTIATE_SPLIT(MFL_BF16, false, false);
}  // namespace mfl
