// Split-precision GEMM kernels with f16 pieces, at least one operand K-strided.
#include "gemm_split.hpp"

namespace mfl {
MFL_INSTANTIATE_SPLIT(MFL_F16, true, false);
MFL_INSTANTIATE_SPLIT(MFL_F16, false, true);
MFL_INSTANTIATE_SPLIT(MFL_F16, false, false);
}  // namespace mfl
