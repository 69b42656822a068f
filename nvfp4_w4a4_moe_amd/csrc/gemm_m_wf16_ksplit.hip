// Grouped GEMM instantiations with NVFP4 A and exact FP16 B whose K halves carry their
// own decode scales (the data gradient through the gate/up weights, W13^T).
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m_wf16_ksplit(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, false, GemmTileWf16, true>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, false, GemmTileWf16, true>(g, stream);
}

}  // namespace nv4
