// NVFP4 grouped GEMM instantiations: GROUP_K GEMMs (weight gradients).
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_k(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_K, NV4_EPI_NONE, true, false, GemmTileK>(g, stream)
                    : launch_tile<NV4_GROUP_K, NV4_EPI_NONE, false, false, GemmTileK>(g, stream);
}

}  // namespace nv4
