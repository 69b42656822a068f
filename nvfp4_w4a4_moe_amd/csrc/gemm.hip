// Grouped NVFP4 x NVFP4 GEMM for gfx950: dispatch to the kernel instantiation for
// the operand type, group mode, epilogue and A-scale mode.  The kernel is in
// gemm_kernel.h; its instantiations are compiled in gemm_m.hip, gemm_m_rows.hip,
// gemm_m_swiglu.hip, gemm_m_swiglu_rows.hip, gemm_m_ksplit.hip, gemm_k.hip and
// gemm_bf16.hip.
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {

hipError_t launch_gemm_m(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_m_rows(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_m_swiglu(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_m_swiglu_rows(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_k(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_m_ksplit(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_bf16(const GemmArgs &g, hipStream_t stream);

hipError_t launch_grouped_gemm(const GemmArgs &g, hipStream_t stream) {
  if (g.operands_bf16) return launch_gemm_bf16(g, stream);
  const bool rows = g.a_scale_mode == NV4_SCALE_ROW;
  if (g.group_mode == NV4_GROUP_K) return launch_gemm_k(g, stream);
  if (g.b_scale_mode == NV4_SCALE_SEGMENT_HALVES) return launch_gemm_m_ksplit(g, stream);
  if (g.epilogue == NV4_EPI_SWIGLU) return rows ? launch_gemm_m_swiglu_rows(g, stream) : launch_gemm_m_swiglu(g, stream);
  return rows ? launch_gemm_m_rows(g, stream) : launch_gemm_m(g, stream);
}

}  // namespace nv4
