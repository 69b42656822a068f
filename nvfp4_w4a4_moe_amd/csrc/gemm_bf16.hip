// BF16-operand grouped GEMM instantiations (the unquantised layer and the BF16 /
// dequantized backward): the same kernel with the decode removed.
#include "gemm_kernel.h"

namespace nv4 {

hipError_t launch_gemm_bf16(const GemmArgs &g, hipStream_t stream) {
  using C = GemmTileBf16;
  if (g.group_mode == NV4_GROUP_K)
    return g.c_is_f32 ? launch_tile<NV4_GROUP_K, NV4_EPI_NONE, true, false, C>(g, stream)
                      : launch_tile<NV4_GROUP_K, NV4_EPI_NONE, false, false, C>(g, stream);
  if (g.epilogue == NV4_EPI_SWIGLU)
    return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_SWIGLU, true, false, C>(g, stream)
                      : launch_tile<NV4_GROUP_M, NV4_EPI_SWIGLU, false, false, C>(g, stream);
  return g.c_is_f32 ? launch_tile<NV4_GROUP_M, NV4_EPI_NONE, true, false, C>(g, stream)
                    : launch_tile<NV4_GROUP_M, NV4_EPI_NONE, false, false, C>(g, stream);
}

}  // namespace nv4
