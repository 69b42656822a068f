// NVFP4 grouped GEMM instantiations: the gate/up GEMM with the SwiGLU epilogue, one tensor scale for A.
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m_swiglu(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_SWIGLU, true, false>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_SWIGLU, false, false>(g, stream);
}

}  // namespace nv4
