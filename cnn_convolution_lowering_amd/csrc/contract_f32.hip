// Contraction kernels for fp32 storage.
#include "contract.hpp"

namespace convlower {
template void launch_gemm<float>(const conv_desc&, const void*, const void*, const void*, void*, const void*,
                              hipStream_t);
}  // namespace convlower
