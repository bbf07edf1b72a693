// GEMM role kGemmProj: its kernels, compiled in a translation unit of their own.
#include "gemm_kernels.h"

namespace w2v2 {
template hipError_t launch_gemm_role<kGemmProj>(DType, const GemmArgs&, hipStream_t);
}  // namespace w2v2
