// NVFP4 grouped GEMM instantiations: GROUP_M GEMMs without epilogue, per-row (per-token) A scales.
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_m_rows(const GemmArgs &g, hipStream_t stream) {
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, true>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, true>(g, stream);
}

}  // namespace nv4
