// Contraction kernels for fp16 storage.
#include "contract.hpp"

namespace convlower {
template void launch_gemm<_Float16>(const conv_desc&, const void*, const void*, const void*, void*, const void*, uint32_t,
                              hipStream_t);
}  // namespace convlower
