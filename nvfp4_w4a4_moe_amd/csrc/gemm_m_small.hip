// NVFP4 grouped GEMM instantiations: GROUP_M without epilogue on 128 x 256 workgroup tiles, one
// tensor scale for A (problems too small to fill the device with 256 x 256 tiles).
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m_small(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, false, GemmTileSmall>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, false, GemmTileSmall>(g, stream);
}

}  // namespace nv4
