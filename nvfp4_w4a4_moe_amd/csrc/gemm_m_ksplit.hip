// NVFP4 grouped GEMM instantiations: GROUP_M with a B decode scale per expert and K half
// (the per-expert transpose of the stacked gate/up weights in the data gradient).
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m_ksplit(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, false, GemmTile, true>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, false, GemmTile, true>(g, stream);
}

}  // namespace nv4
