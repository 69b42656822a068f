// NVFP4 grouped GEMM instantiations: GROUP_M GEMMs without epilogue (down projection, data gradients), one tensor scale for A.
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, false>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, false>(g, stream);
}

}  // namespace nv4
