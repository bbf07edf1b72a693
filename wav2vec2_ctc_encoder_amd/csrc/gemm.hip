// GEMM entry point: dispatch to the role's kernels (instantiated per role in
// gemm_role_*.hip from gemm_kernels.h).
#include "common.h"

namespace w2v2 {

template <int ROLE>
hipError_t launch_gemm_role(DType t, const GemmArgs& a, hipStream_t s);

hipError_t launch_gemm(DType t, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0 || a.groups <= 0) return hipSuccess;
  switch (a.role) {
    case kGemmConv: return launch_gemm_role<kGemmConv>(t, a, s);
    case kGemmProj: return launch_gemm_role<kGemmProj>(t, a, s);
    case kGemmPos: return launch_gemm_role<kGemmPos>(t, a, s);
    case kGemmQKV: return launch_gemm_role<kGemmQKV>(t, a, s);
    case kGemmOut: return launch_gemm_role<kGemmOut>(t, a, s);
    case kGemmFFN1: return launch_gemm_role<kGemmFFN1>(t, a, s);
    case kGemmFFN2: return launch_gemm_role<kGemmFFN2>(t, a, s);
    case kGemmHead: return launch_gemm_role<kGemmHead>(t, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w2v2
