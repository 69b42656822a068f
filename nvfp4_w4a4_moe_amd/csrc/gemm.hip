// Grouped NVFP4 x NVFP4 GEMM for gfx950: dispatch to the kernel instantiation for
// the operand type, group mode, epilogue and A-scale mode.  The kernel is in
// gemm_kernel.h; its instantiations are compiled in gemm_m.hip, gemm_m_rows.hip,
// gemm_m_swiglu.hip, gemm_m_swiglu_rows.hip, gemm_m_ksplit.hip, gemm_m_small.hip,
// gemm_m_wf16.hip, gemm_m_wf16_ksplit.hip, gemm_k.hip and gemm_bf16.hip.
#include <algorithm>

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
hipError_t launch_gemm_m_small(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_m_wf16(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_m_wf16_ksplit(const GemmArgs &g, hipStream_t stream);

namespace {

// one thread per 8-byte code chunk of a padded row (rows start 8-byte aligned: K/2 % 8 == 0)
__global__ void k_repack_codes(const uint2 *src, int64_t rows, int64_t sc, uint2 *dst, int64_t dc) {
  const int64_t n = rows * dc;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / dc, c = i - r * dc;
    dst[i] = c < sc ? src[r * sc + c] : make_uint2(0u, 0u);
  }
}

// one thread per scale byte of a padded row
__global__ void k_repack_scales(const uint8_t *src, int64_t rows, int64_t sb, uint8_t *dst, int64_t db) {
  const int64_t n = rows * db;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / db, c = i - r * db;
    dst[i] = c < sb ? src[r * sb + c] : (uint8_t)0;
  }
}

}  // namespace

hipError_t launch_repack_k(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, uint8_t *codes_p,
                           uint8_t *scales_p, int64_t Kp, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int cap = device_cu_count() * 8;
  const int64_t nc = rows * (Kp >> 4), ns = rows * (Kp >> 4);
  const int gc = (int)std::max<int64_t>(1, std::min<int64_t>((nc + 255) / 256, cap));
  const int gs = (int)std::max<int64_t>(1, std::min<int64_t>((ns + 255) / 256, cap));
  k_repack_codes<<<gc, 256, 0, stream>>>(reinterpret_cast<const uint2 *>(codes), rows, K >> 4,
                                         reinterpret_cast<uint2 *>(codes_p), Kp >> 4);
  k_repack_scales<<<gs, 256, 0, stream>>>(scales, rows, K >> 4, scales_p, Kp >> 4);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs &g, hipStream_t stream) {
  if (g.operands_bf16) return launch_gemm_bf16(g, stream);
  if (g.b_f16)  // exact FP16 B (GROUP_M, one tensor scale for A, K % 64 == 0: checked by the caller)
    return g.b_scale_mode == NV4_SCALE_SEGMENT_HALVES ? launch_gemm_m_wf16_ksplit(g, stream)
                                                      : launch_gemm_m_wf16(g, stream);
  const bool rows = g.a_scale_mode == NV4_SCALE_ROW;
  if (g.group_mode == NV4_GROUP_K) return launch_gemm_k(g, stream);
  if (g.b_scale_mode == NV4_SCALE_SEGMENT_HALVES) return launch_gemm_m_ksplit(g, stream);
  if (g.epilogue == NV4_EPI_SWIGLU) return rows ? launch_gemm_m_swiglu_rows(g, stream) : launch_gemm_m_swiglu(g, stream);
  if (rows) return launch_gemm_m_rows(g, stream);
  // Upper estimate of the 256 x 256 tiles (every expert adds at most one partial M
  // tile; the row counts stay on the device): with fewer than two per compute unit,
  // the 128 x 256 tiles spread the work over twice as many workgroups.
  const int64_t tiles = ((g.M_cap + 255) / 256 + g.E) * ((g.N + 255) / 256);
  if (tiles < 2 * (int64_t)device_cu_count()) return launch_gemm_m_small(g, stream);
  return launch_gemm_m(g, stream);
}

}  // namespace nv4
