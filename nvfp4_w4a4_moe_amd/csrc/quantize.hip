// NVFP4 quantisation kernels for gfx950.
//
// "The 4-bitter Lesson", section "Baseline: A starting recipe with stable training
// dynamics": 16-element blocks with E4M3 scales and one FP32 tensor scale.
// Section "Why is the NVFP4 pretraining recipe not sufficient for RL?": one global
// scale per weight tensor; the per-token variant computes each token row's FP32
// scale inside the quantisation kernel, then the E4M3 block scales, then packs
// the FP4 values, in one fused pass.  Section "Improving Gradient Stability",
// footnote 6: quantisation is clip(round(w/s), qmin, qmax).
//
// Arithmetic (each FP32 step a single correctly rounded operation, no contraction):
//   S = fp32(2688 / A) (1 if A == 0 or not finite), G = fp32(1 / S)
//   sf = E4M3(fp32(fp32(amax_block / 6) * S)),  inv = sf ? fp32(S / sf) : 0
//   q = E2M1(fp32(x * inv))  -- round to nearest even, saturating, sign kept.
//
// Memory: every kernel streams its input once with 16-byte loads (the amax pass
// is a second read when the group amax is not supplied).
#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const void *x, int x_is_f32, int64_t off, float v[8]) {
  if (x_is_f32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xFFFF0000u);
    v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float load1(const void *x, int x_is_f32, int64_t off) {
  if (x_is_f32) return static_cast<const float *>(x)[off];
  return bf16_bits_to_f32(static_cast<const uint16_t *>(x)[off]);
}

// group (tensor-scale index) of a source row
__device__ __forceinline__ int row_group(const QuantArgs &a, int64_t row) {
  if (a.scale_mode == NV4_SCALE_TENSOR) return 0;
  if (a.scale_mode == NV4_SCALE_ROW) return (int)row;
  if (a.seg_offsets == nullptr) return (int)(row / (a.rows / a.nseg));
  int lo = 0, hi = a.nseg - 1;  // last segment s with seg_offsets[s] <= row
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a.seg_offsets[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ const float *amax_src(const QuantArgs &a) {
  return a.amax_in ? a.amax_in : a.amax_acc;
}

__global__ void k_fill_zero(float *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Group amax.  Workgroup (p, g) scans rows p, p + P, ... of group g's row range
// (an equal split of the rows, or [seg_offsets[g], seg_offsets[g+1])); its
// waves reduce in registers and LDS, and one order-independent atomic max per
// workgroup goes to amax_acc[g], so a group sees at most P atomics.
__global__ __launch_bounds__(kThreads) void k_amax_rows(QuantArgs a, int P) {
  __shared__ float red[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x, g = blockIdx.y;
  int64_t r0, r1;
  if (a.scale_mode == NV4_SCALE_TENSOR) { r0 = 0; r1 = a.rows; }
  else if (a.seg_offsets) { r0 = a.seg_offsets[g]; r1 = a.seg_offsets[g + 1]; }
  else { const int64_t len = a.rows / a.nseg; r0 = (int64_t)g * len; r1 = r0 + len; }
  float m = 0.0f;
  bool bad = false;
  for (int64_t row = r0 + (int64_t)p * (kThreads / 64) + wave; row < r1; row += (int64_t)P * (kThreads / 64)) {
    const int64_t base = row * a.ldx;
    for (int64_t k = (int64_t)lane * 8; k < a.K; k += 512) {
      float v[8];
      load8(a.x, a.x_is_f32, base + k, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float av = fabsf(v[i]);
        bad |= !(av <= 3.402823466e38f);
        m = fmaxf(m, av);
      }
    }
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float w = red[0];
    for (int i = 1; i < kThreads / 64; ++i) w = fmaxf(w, red[i]);
    atomic_max_nonneg(&a.amax_acc[g], w);
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

// Quantise one 8-element half-block held by this lane; the partner lane (lane ^ 1)
// holds the other half of the same 16-element block.  Returns the packed codes
// and the block scale byte.
__device__ __forceinline__ uint32_t quant_half_block(const float v[8], float S, uint32_t &sf_out, bool &bad) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float av = fabsf(v[i]);
    bad |= !(av <= 3.402823466e38f);
    m = fmaxf(m, av);
  }
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  const uint32_t sf = e4m3_from_f32(__fmul_rn(__fdiv_rn(m, 6.0f), S));
  const float inv = sf ? __fdiv_rn(S, e4m3_to_f32(sf)) : 0.0f;
  uint32_t p = 0;
  p = pack_e2m1_pair<0>(p, __fmul_rn(v[0], inv), __fmul_rn(v[1], inv));
  p = pack_e2m1_pair<1>(p, __fmul_rn(v[2], inv), __fmul_rn(v[3], inv));
  p = pack_e2m1_pair<2>(p, __fmul_rn(v[4], inv), __fmul_rn(v[5], inv));
  p = pack_e2m1_pair<3>(p, __fmul_rn(v[6], inv), __fmul_rn(v[7], inv));
  sf_out = sf;
  return p;
}

// Same with fp32(S / sf) looked up in a table of the 127 E4M3 values.
__device__ __forceinline__ uint32_t quant_half_block_tab(const float v[8], float S, const float *inv_tab,
                                                         uint32_t &sf_out, bool &bad) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float av = fabsf(v[i]);
    bad |= !(av <= 3.402823466e38f);
    m = fmaxf(m, av);
  }
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  const uint32_t sf = e4m3_from_f32(__fmul_rn(__fdiv_rn(m, 6.0f), S));
  const float inv = inv_tab[sf];
  uint32_t p = 0;
  p = pack_e2m1_pair<0>(p, __fmul_rn(v[0], inv), __fmul_rn(v[1], inv));
  p = pack_e2m1_pair<1>(p, __fmul_rn(v[2], inv), __fmul_rn(v[3], inv));
  p = pack_e2m1_pair<2>(p, __fmul_rn(v[4], inv), __fmul_rn(v[5], inv));
  p = pack_e2m1_pair<3>(p, __fmul_rn(v[6], inv), __fmul_rn(v[7], inv));
  sf_out = sf;
  return p;
}

// Write the decode scales G (and, when the amax came from amax_in, amax_out).
__device__ void write_group_scales(const QuantArgs &a) {
  const float *A = amax_src(a);
  for (int g = threadIdx.x; g < a.ngroups; g += blockDim.x) {
    float S = tensor_encode_scale(A[g]);
    a.tscale[g] = __fdiv_rn(1.0f, S);
    if (a.amax_in && a.amax_acc) a.amax_acc[g] = a.amax_in[g];
  }
}

// Row layout, tensor or segment scales: every lane quantises 8 consecutive
// elements per chunk (16-byte load, 4-byte code store), two chunks in flight;
// waves stride over the flat (row, chunk) index so that loads and stores are
// fully coalesced.  With one tensor scale, fp32(S / sf) comes from an LDS table
// of the 127 E4M3 values (the same correctly rounded quotients).
__global__ __launch_bounds__(kThreads) void k_quant_rows(QuantArgs a) {
  __shared__ float inv_tab[128];
  if (blockIdx.x == 0) write_group_scales(a);
  const float *A = amax_src(a);
  const bool tensor = a.scale_mode == NV4_SCALE_TENSOR;
  const float S_tensor = tensor ? tensor_encode_scale(A[0]) : 1.0f;
  if (tensor) {
    if (threadIdx.x < 128) inv_tab[threadIdx.x] = threadIdx.x ? __fdiv_rn(S_tensor, e4m3_to_f32(threadIdx.x)) : 0.0f;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int64_t kc = a.K >> 3;  // 8-element chunks per row (even)
  const int64_t total = a.rows * kc;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int cur = -1;
  float S = 1.0f;
  bool bad = false;
  for (int64_t c0 = wave * 64; c0 < total; c0 += 2 * stride) {
    int64_t row[2], ch[2];
    bool act[2];
    float v[2][8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t base = c0 + u * stride;
      const int64_t c = base + lane;
      act[u] = c < total;
      const int64_t cc = act[u] ? c : (base < total ? base : c0);  // inactive lanes (and their partners) redo a valid chunk
      row[u] = cc / kc;
      ch[u] = cc - row[u] * kc;
      load8(a.x, a.x_is_f32, row[u] * a.ldx + ch[u] * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t sf, p;
      if (tensor) {
        p = quant_half_block_tab(v[u], S_tensor, inv_tab, sf, bad);
      } else {
        const int g = row_group(a, row[u]);
        if (g != cur) { cur = g; S = tensor_encode_scale(A[g]); }
        p = quant_half_block(v[u], S, sf, bad);
      }
      if (act[u]) {
        reinterpret_cast<uint32_t *>(a.codes)[row[u] * (a.out_K >> 3) + ch[u]] = p;
        if ((ch[u] & 1) == 0) a.scales[row[u] * (a.out_K >> 4) + (ch[u] >> 1)] = (uint8_t)sf;
      }
    }
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

// Row layout with one scale per row (the per-token variant): one wave per row,
// amax and quantisation fused (the row is read twice, the second time from cache).
__global__ __launch_bounds__(kThreads) void k_quant_rows_per_row(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  bool bad = false;
  for (int64_t row = wave; row < a.rows; row += nwaves) {
    const int64_t base = row * a.ldx;
    float A;
    if (a.amax_in) {
      A = a.amax_in[row];
    } else {
      float m = 0.0f;
      for (int64_t k = (int64_t)lane * 8; k < a.K; k += 512) {
        float v[8];
        load8(a.x, a.x_is_f32, base + k, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
      }
      A = wave_max(m);
    }
    const float S = tensor_encode_scale(A);
    if (lane == 0) {
      a.tscale[row] = __fdiv_rn(1.0f, S);
      if (a.amax_acc) a.amax_acc[row] = A;
    }
    for (int64_t k0 = 0; k0 < a.K; k0 += 512) {
      const int64_t k = k0 + (int64_t)lane * 8;
      const bool act = k < a.K;
      float v[8];
      load8(a.x, a.x_is_f32, base + (act ? k : k0), v);
      uint32_t sf;
      const uint32_t p = quant_half_block(v, S, sf, bad);
      if (act) {
        reinterpret_cast<uint32_t *>(a.codes)[row * (a.out_K >> 3) + (k >> 3)] = p;
        if (((k >> 3) & 1) == 0) a.scales[row * (a.out_K >> 4) + (k >> 4)] = (uint8_t)sf;
      }
    }
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

// Column layouts (transposed operands of the backward GEMMs).  One thread owns
// one column `col` of x and 4 consecutive output blocks (64 positions along the
// new K); each block is 16 consecutive rows of one segment (zero beyond the
// segment's end).  Reads are coalesced across the threads (consecutive columns);
// each thread writes 32 code bytes and 4 scale bytes of one output row.
constexpr int kColBlocks = 4;

__global__ __launch_bounds__(kThreads) void k_quant_cols(QuantArgs a) {
  if (blockIdx.x == 0 && blockIdx.y == 0) write_group_scales(a);
  const float *A = amax_src(a);
  const int64_t C = a.K;  // columns of x
  const int64_t col = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const bool batched = a.layout == NV4_COLS_BATCHED;
  const int64_t m = batched ? a.rows / a.nseg : 0;
  const int64_t nblk_total = batched ? (a.rows >> 4) : (int64_t)(a.seg_padded_offsets[a.nseg] >> 4);
  const int64_t b0 = (int64_t)blockIdx.y * kColBlocks;
  if (b0 >= nblk_total || col >= C) return;
  bool bad = false;
  for (int bi = 0; bi < kColBlocks; ++bi) {
    const int64_t b = b0 + bi;
    if (b >= nblk_total) break;
    int s;
    int64_t r0, rend, out_row, out_pos;
    if (batched) {
      s = (int)(b / (m >> 4));
      r0 = (int64_t)s * m + (b * 16 - (int64_t)s * m);
      rend = (int64_t)(s + 1) * m;
      out_row = (int64_t)s * C + col;
      out_pos = b * 16 - (int64_t)s * m;
    } else {
      int lo = 0, hi = a.nseg - 1;  // segment whose padded range holds position b*16
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (a.seg_padded_offsets[mid] <= b * 16) lo = mid; else hi = mid - 1;
      }
      s = lo;
      r0 = a.seg_offsets[s] + (b * 16 - a.seg_padded_offsets[s]);
      rend = a.seg_offsets[s + 1];
      out_row = col;
      out_pos = b * 16;
    }
    const int g = a.scale_mode == NV4_SCALE_TENSOR ? 0 : s;
    const float S = tensor_encode_scale(A[g]);
    float v[16];
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t r = r0 + i;
      v[i] = (r < rend) ? load1(a.x, a.x_is_f32, r * a.ldx + col) : 0.0f;
      const float av = fabsf(v[i]);
      bad |= !(av <= 3.402823466e38f);
      mx = fmaxf(mx, av);
    }
    const uint32_t sf = e4m3_from_f32(__fmul_rn(__fdiv_rn(mx, 6.0f), S));
    const float inv = sf ? __fdiv_rn(S, e4m3_to_f32(sf)) : 0.0f;
    uint32_t p0 = 0, p1 = 0;
    p0 = pack_e2m1_pair<0>(p0, __fmul_rn(v[0], inv), __fmul_rn(v[1], inv));
    p0 = pack_e2m1_pair<1>(p0, __fmul_rn(v[2], inv), __fmul_rn(v[3], inv));
    p0 = pack_e2m1_pair<2>(p0, __fmul_rn(v[4], inv), __fmul_rn(v[5], inv));
    p0 = pack_e2m1_pair<3>(p0, __fmul_rn(v[6], inv), __fmul_rn(v[7], inv));
    p1 = pack_e2m1_pair<0>(p1, __fmul_rn(v[8], inv), __fmul_rn(v[9], inv));
    p1 = pack_e2m1_pair<1>(p1, __fmul_rn(v[10], inv), __fmul_rn(v[11], inv));
    p1 = pack_e2m1_pair<2>(p1, __fmul_rn(v[12], inv), __fmul_rn(v[13], inv));
    p1 = pack_e2m1_pair<3>(p1, __fmul_rn(v[14], inv), __fmul_rn(v[15], inv));
    uint2 *dst = reinterpret_cast<uint2 *>(a.codes + out_row * (a.out_K >> 1) + (out_pos >> 1));
    *dst = make_uint2(p0, p1);
    a.scales[out_row * (a.out_K >> 4) + (out_pos >> 4)] = (uint8_t)sf;
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a, hipStream_t stream) {
  const int cus = device_cu_count();
  const int per_row = a.scale_mode == NV4_SCALE_ROW;
  // group amax pass (tensor / segment scales without a supplied amax)
  if (!a.amax_in && !per_row) {
    k_fill_zero<<<(a.ngroups + 255) / 256, 256, 0, stream>>>(a.amax_acc, a.ngroups);
    if (a.rows > 0) {
      // about two workgroups per CU in total, split over the groups
      const int groups = a.scale_mode == NV4_SCALE_TENSOR ? 1 : a.nseg;
      const int64_t rows_per_group = (a.rows + groups - 1) / groups;
      const int P = (int)std::max<int64_t>(1, std::min<int64_t>((2 * cus + groups - 1) / groups, (rows_per_group + 3) / 4));
      k_amax_rows<<<dim3(P, groups), kThreads, 0, stream>>>(a, P);
    }
  }
  if (a.layout == NV4_ROWS) {
    if (per_row) {
      const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((a.rows + 3) / 4, (int64_t)cus * 16));
      k_quant_rows_per_row<<<grid, kThreads, 0, stream>>>(a);
    } else {
      const int64_t chunks = a.rows * (a.K >> 3);
      const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((chunks + 2 * kThreads - 1) / (2 * kThreads), (int64_t)cus * 8));
      k_quant_rows<<<grid, kThreads, 0, stream>>>(a);
    }
  } else {
    // upper bound of output blocks: rows + 15 per segment, in 16-row blocks
    const int64_t nblk = a.layout == NV4_COLS_BATCHED ? (a.rows >> 4) : ((a.rows + 15 * (int64_t)a.nseg) >> 4) + 1;
    dim3 grid((unsigned)((a.K + kThreads - 1) / kThreads), (unsigned)std::max<int64_t>(1, (nblk + kColBlocks - 1) / kColBlocks));
    k_quant_cols<<<grid, kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace nv4
