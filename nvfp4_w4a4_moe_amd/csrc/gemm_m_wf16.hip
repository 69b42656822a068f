// Grouped GEMM instantiations with NVFP4 A and exact FP16 B (the expert weights decoded
// once, e2m1 x e4m3 without the tensor scale): GROUP_M without epilogue and with the
// SwiGLU epilogue, one tensor scale for A.
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m_wf16(const GemmArgs &g, hipStream_t stream) {
  if (g.epilogue == NV4_EPI_SWIGLU)
    return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_SWIGLU, true, false, GemmTileWf16>(g, stream)
                      : launch_tile<NV4_GROUP_M, NV4_EPI_SWIGLU, false, false, GemmTileWf16>(g, stream);
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, false, GemmTileWf16>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, false, GemmTileWf16>(g, stream);
}

}  // namespace nv4
