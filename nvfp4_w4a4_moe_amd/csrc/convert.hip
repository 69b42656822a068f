// BF16 operands for the BF16 and dequantized backward of the expert layer.
//
// "The 4-bitter Lesson", section "Improving Gradient Stability": the dequantized
// backward runs the backward GEMMs on BF16 operands that hold DQ(Q(.)) of the
// exact NVFP4 tensors the forward used (weights and activations); section "Why
// is the NVFP4 pretraining recipe not sufficient for RL?": the conservative
// baseline keeps the backward in BF16 on the unquantised tensors.
//
// One BF16 element of an NVFP4 tensor: e2m1(q) * sf is exact in FP32 (at most 6
// significant bits), one FP32 multiply by the tensor decode scale G, then round
// to nearest even to BF16.
//
// Layouts (the operand layouts of the BF16 grouped GEMM, K contiguous):
//   rows          out [rows][K]: dequantised (or gathered) rows.
//   cols          out [K][cap]: logical row r of segment s lands in column
//                 padded_offsets[s] + (r - offsets[s]); each segment's padding up
//                 to the next multiple of 16 is written as zeros.  The operands of
//                 the weight-gradient GEMMs (contraction over each expert's rows).
//   cols_batched  nseg equal matrices of m rows, each transposed: out [nseg*K][m].
//                 The transposed expert weights of the data-gradient GEMMs.
// The transposes go through a 64 x 64 LDS tile: rows are read 32 bytes (16
// elements) per lane and written 16 bytes (8 elements) per lane, both coalesced.
#include <algorithm>

#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// BF16 bits of an NVFP4 element pair (packed byte `b` of a code dword) times the
// exact block scale `sf` and the tensor scale G
template <int SEL>
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, float sf, float G) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);  // exact
  const float a = (v[0] * sf) * G, b = (v[1] * sf) * G;                   // first product exact
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// decode scale of source row `sr` of an NVFP4 operand
__device__ __forceinline__ float row_tscale(const ConvertArgs &a, int64_t sr) {
  if (a.scale_mode == NV4_SCALE_ROW) return a.tscale[sr];
  if (a.scale_mode == NV4_SCALE_SEGMENT) return a.tscale[sr / (a.src_rows / a.src_nseg)];
  return a.tscale[0];
}

// a source row taken from the caller's row index, clamped into the source so that
// an index outside the contract cannot read outside the buffer
__device__ __forceinline__ int64_t src_of(const ConvertArgs &a, int32_t idx) {
  return idx < 0 ? 0 : (idx >= a.src_rows ? a.src_rows - 1 : idx);
}

// 16 BF16 values (8 dwords) of source row sr, columns [c, c + 16)
template <bool FP4>
__device__ __forceinline__ void load16(const ConvertArgs &a, int64_t sr, int64_t c, uint32_t (&o)[8]) {
  if (FP4) {
    const uint2 w = *reinterpret_cast<const uint2 *>(a.codes + sr * (a.K >> 1) + (c >> 1));
    const float sf = e4m3_to_f32(a.scales[sr * (a.K >> 4) + (c >> 4)] & 0x7Fu);
    const float G = row_tscale(a, sr);
    o[0] = dq_pair<0>(w.x, sf, G);
    o[1] = dq_pair<1>(w.x, sf, G);
    o[2] = dq_pair<2>(w.x, sf, G);
    o[3] = dq_pair<3>(w.x, sf, G);
    o[4] = dq_pair<0>(w.y, sf, G);
    o[5] = dq_pair<1>(w.y, sf, G);
    o[6] = dq_pair<2>(w.y, sf, G);
    o[7] = dq_pair<3>(w.y, sf, G);
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(a.x + sr * a.ldx + c);
    const uint4 u0 = p[0], u1 = p[1];
    o[0] = u0.x; o[1] = u0.y; o[2] = u0.z; o[3] = u0.w;
    o[4] = u1.x; o[5] = u1.y; o[6] = u1.z; o[7] = u1.w;
  }
}

template <bool FP4>
__global__ __launch_bounds__(256) void k_rows_bf16(ConvertArgs a) {
  const int64_t nb = a.K >> 4;
  const int64_t total = a.rows * nb;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / nb, c = (i - r * nb) * 16;
    const int64_t sr = a.row_index ? src_of(a, a.row_index[r]) : r;
    uint32_t o[8];
    load16<FP4>(a, sr, c, o);
    uint4 *dst = reinterpret_cast<uint4 *>(a.out + r * a.K + c);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// One 64 x 64 tile: output columns [p0, p0 + 64) (padded logical rows) of output
// rows for source columns [c0, c0 + 64).
template <bool FP4, bool BATCHED>
__global__ __launch_bounds__(256) void k_cols_bf16(ConvertArgs a) {
  __shared__ uint16_t tile[64][64 + 2];  // [output column][source column]
  __shared__ int64_t src_row[64];        // -1: padding
  const int tid = threadIdx.x;
  const int64_t p0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int batch = blockIdx.z;
  const int64_t m = BATCHED ? a.rows / a.nseg : 0;
  // output columns in use (never past the caller's capacity)
  const int64_t limit = BATCHED ? m : std::min<int64_t>(a.seg_padded_offsets[a.nseg], a.out_cols);
  if (p0 >= limit) return;  // the same for the whole block
  if (tid < 64) {
    const int64_t p = p0 + tid;
    int64_t sr = -1;
    if (p < limit) {
      if (BATCHED) {
        sr = (int64_t)batch * m + p;
      } else {
        int lo = 0, hi = a.nseg - 1;  // last segment with padded start <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (a.seg_padded_offsets[mid] <= p) lo = mid; else hi = mid - 1;
        }
        const int64_t r = a.seg_offsets[lo] + (p - a.seg_padded_offsets[lo]);
        if (r < a.seg_offsets[lo + 1] && r < a.rows) sr = a.row_index ? src_of(a, a.row_index[r]) : r;
      }
    }
    src_row[tid] = sr;
  }
  __syncthreads();
  {
    const int j = tid >> 2, grp = tid & 3;
    const int64_t c = c0 + grp * 16;
    uint32_t o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (src_row[j] >= 0 && c < a.K) load16<FP4>(a, src_row[j], c, o);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tile[j][grp * 16 + 2 * i] = (uint16_t)o[i];
      tile[j][grp * 16 + 2 * i + 1] = (uint16_t)(o[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = tid + it * 256;
    const int cc = idx >> 3, ch = idx & 7;
    const int64_t p = p0 + ch * 8;
    if (c0 + cc >= a.K || p >= limit) continue;  // limit and p are multiples of 8
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[t] = (uint32_t)tile[ch * 8 + 2 * t][cc] | ((uint32_t)tile[ch * 8 + 2 * t + 1][cc] << 16);
    const int64_t orow = (BATCHED ? (int64_t)batch * a.K : 0) + c0 + cc;
    *reinterpret_cast<uint4 *>(a.out + orow * a.out_cols + p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Exact FP16 values e2m1 * e4m3 of an NVFP4 tensor (the decode scale G not applied):
// one thread per 16-element block, 8 code bytes and 1 scale byte in, 32 bytes out.
__global__ __launch_bounds__(256) void k_decode_f16(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                                    int64_t K, uint16_t *out, int64_t ldo) {
  const int64_t nb = K >> 4, total = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / nb, b = i - r * nb;
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + r * (K >> 1) + b * 8);
    const f16x2 s2 = e4m3x2_to_f16<false>((uint32_t)scales[r * nb + b] * 0x0101u);
    const f16x8 lo = decode8_f16(c.x, s2), hi = decode8_f16(c.y, s2);
    uint4 *o = reinterpret_cast<uint4 *>(out + r * ldo + b * 16);
    o[0] = __builtin_bit_cast(uint4, lo);
    o[1] = __builtin_bit_cast(uint4, hi);
  }
}

}  // namespace

hipError_t launch_decode_f16(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, uint16_t *out,
                             int64_t ldo, hipStream_t stream) {
  const int64_t total = rows * (K >> 4);
  if (total == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, (int64_t)device_cu_count() * 16);
  k_decode_f16<<<grid, 256, 0, stream>>>(codes, scales, rows, K, out, ldo);
  return hipGetLastError();
}

hipError_t launch_convert(const ConvertArgs &a, hipStream_t stream) {
  const bool fp4 = a.codes != nullptr;
  if (a.layout == NV4_ROWS) {
    const int64_t total = a.rows * (a.K >> 4);
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    const int grid = (int)std::min<int64_t>(want, (int64_t)device_cu_count() * 16);
    if (fp4) k_rows_bf16<true><<<grid, 256, 0, stream>>>(a);
    else k_rows_bf16<false><<<grid, 256, 0, stream>>>(a);
    return hipGetLastError();
  }
  const bool batched = a.layout == NV4_COLS_BATCHED;
  const int64_t ncols = batched ? a.rows / a.nseg : a.out_cols;  // output columns (an upper bound for cols)
  if (ncols == 0 || a.K == 0) return hipSuccess;
  const dim3 grid((unsigned)((ncols + 63) / 64), (unsigned)((a.K + 63) / 64), batched ? (unsigned)a.nseg : 1u);
  if (batched) {
    if (fp4) k_cols_bf16<true, true><<<grid, 256, 0, stream>>>(a);
    else k_cols_bf16<false, true><<<grid, 256, 0, stream>>>(a);
  } else {
    if (fp4) k_cols_bf16<true, false><<<grid, 256, 0, stream>>>(a);
    else k_cols_bf16<false, false><<<grid, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace nv4
