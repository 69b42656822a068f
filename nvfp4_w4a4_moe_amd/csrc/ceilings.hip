// Measurement kernels: what a plain stream of HBM traffic and a plain loop of
// FP16 matrix instructions reach on this device.  The path's kernels are judged
// against these achievable rates as well as against the published peaks
// ("Low-Bit Precision Training ...", section "Throughput Gains and the Conditions
// That Produce Them": throughput gains depend on whether the kernels are bound by
// arithmetic or by memory movement).
//
//   k_stream_copy  16-byte non-temporal loads and stores, U vectors of every lane in
//                  flight, grid-stride over the buffer (read + write traffic).
//   k_stream_read  the same loads only; the XOR of the data goes to a sink word only
//                  when it equals a value the caller never passes, so nothing is
//                  written in practice and the loads cannot be removed.
//   k_stream_mix   4 reads of 16 bytes per 16-byte write, a quantiser's read:write mix.
//   k_stream_write 16-byte stores only (ordinary, write-back: a little faster here than
//                  non-temporal ones), the bound of an output-heavy kernel.
//   k_mfma_loop    eight independent v_mfma_f32_32x32x16_f16 chains per wave with no
//                  memory traffic: the matrix-core issue rate at a given occupancy.
//   k_lds_read     16-byte LDS reads of a 64 KB buffer, every wave reading 1 KB per
//                  instruction (no bank conflicts), two workgroups of four waves per CU:
//                  the LDS read bandwidth a compute unit delivers.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe_bench.h"

namespace nv4 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void k_stream_copy(const u32x4 *__restrict__ src,
                                                                u32x4 *__restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * stride < n; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const u32x4 *__restrict__ src, int64_t n,
                                                                uint32_t never, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (kStreamUnroll - 1) * stride < n; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == never) sink[0] = x;
}

__global__ __launch_bounds__(kStreamThreads) void k_stream_write(u32x4 *__restrict__ dst, int64_t n, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  const u32x4 w = {v, v ^ 1u, v ^ 2u, (uint32_t)threadIdx.x};
  for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride) dst[i] = w;
}

// Reads 4 x 16 bytes and writes 16 bytes per lane per round: the 4:1 read:write mix of
// a quantiser (2 bytes in, 0.5 bytes of codes and 1/16 byte of scales out per element).
// dst holds n / 4 vectors.
__global__ __launch_bounds__(kStreamThreads) void k_stream_mix(const u32x4 *__restrict__ src,
                                                               u32x4 *__restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  // n % 256 == 0, so every j + 192 below stays under n
  for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n / 4; i += stride) {
    const int64_t j = (i / 64) * 256 + (i % 64);   // a wave reads 4 consecutive 1 KB runs
    u32x4 v = __builtin_nontemporal_load(src + j);
    v ^= __builtin_nontemporal_load(src + j + 64);
    v ^= __builtin_nontemporal_load(src + j + 128);
    v ^= __builtin_nontemporal_load(src + j + 192);
    __builtin_nontemporal_store(v, dst + i);
  }
}

// Eight accumulator chains of 32x32x16 FP16 MFMAs per wave.  The operands depend on
// the lane so that the compiler cannot fold them; the sum of the accumulators is
// written once per lane.
template <int WAVES_PER_SIMD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD)))
void k_mfma_loop(float *out, int iters) {
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((lane + i) & 7) * (_Float16)0.125f;
    b[i] = (_Float16)((lane * 3 + i) & 7) * (_Float16)0.0625f;
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kLdsBytes = 65536;

__global__ __launch_bounds__(256) void k_lds_read(uint32_t *out, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[kLdsBytes];
  const int t = threadIdx.x;
  for (int i = t; i < kLdsBytes / 16; i += 256) reinterpret_cast<u32x4 *>(buf)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  u32x4 acc = {0, 0, 0, 0};
  const int base = t * 16;  // < 4096: a wave's 64 lanes read 1 KB of consecutive bytes
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int off = (base + ((it * 8 + u) & 15) * 4096) & (kLdsBytes - 1);  // 16-byte aligned, inside buf
      acc += *reinterpret_cast<const u32x4 *>(buf + off);
    }
    asm volatile("" : "+v"(acc));  // keeps every read: the sum is not folded across iterations
  }
  out[(int64_t)blockIdx.x * 256 + t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

int stream_grid(int64_t n) {
  const int64_t want = (n + (int64_t)kStreamThreads * kStreamUnroll - 1) / ((int64_t)kStreamThreads * kStreamUnroll);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)device_cu_count() * 16));
}

}  // namespace
}  // namespace nv4

extern "C" {

size_t nv4_bench_mfma_out_floats(int waves_per_simd) {
  return (size_t)nv4::device_cu_count() * 4 * (size_t)waves_per_simd * 64;
}

nv4_status nv4_bench_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes == 0 || bytes % 16) return NV4_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return NV4_EALIGN;
  const int64_t n = (int64_t)(bytes / 16);
  nv4::k_stream_copy<<<nv4::stream_grid(n), nv4::kStreamThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const nv4::u32x4 *>(src), static_cast<nv4::u32x4 *>(dst), n);
  return hipGetLastError() == hipSuccess ? NV4_OK : NV4_EHIP;
}

nv4_status nv4_bench_read(const void *src, size_t bytes, uint32_t never, uint32_t *sink, void *stream) {
  if (!src || !sink || bytes == 0 || bytes % 16) return NV4_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16) return NV4_EALIGN;
  const int64_t n = (int64_t)(bytes / 16);
  nv4::k_stream_read<<<nv4::stream_grid(n), nv4::kStreamThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const nv4::u32x4 *>(src), n, never, sink);
  return hipGetLastError() == hipSuccess ? NV4_OK : NV4_EHIP;
}

nv4_status nv4_bench_write(void *dst, size_t bytes, void *stream) {
  if (!dst || bytes == 0 || bytes % 16) return NV4_EINVAL;
  if (reinterpret_cast<uintptr_t>(dst) % 16) return NV4_EALIGN;
  const int64_t n = (int64_t)(bytes / 16);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + nv4::kStreamThreads - 1) / nv4::kStreamThreads,
                                                               (int64_t)nv4::device_cu_count() * 8));
  nv4::k_stream_write<<<grid, nv4::kStreamThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<nv4::u32x4 *>(dst), n, 0x3F800000u);
  return hipGetLastError() == hipSuccess ? NV4_OK : NV4_EHIP;
}

nv4_status nv4_bench_mix(const void *src, size_t bytes, void *dst, void *stream) {
  if (!src || !dst || bytes == 0 || bytes % 4096) return NV4_EINVAL;
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return NV4_EALIGN;
  const int64_t n = (int64_t)(bytes / 16);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n / 4 + nv4::kStreamThreads - 1) / nv4::kStreamThreads,
                                                               (int64_t)nv4::device_cu_count() * 16));
  nv4::k_stream_mix<<<grid, nv4::kStreamThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const nv4::u32x4 *>(src), static_cast<nv4::u32x4 *>(dst), n);
  return hipGetLastError() == hipSuccess ? NV4_OK : NV4_EHIP;
}

size_t nv4_bench_lds_out_words(void) { return (size_t)nv4::device_cu_count() * 2 * 256; }

nv4_status nv4_bench_lds(uint32_t *out, int iters, void *stream) {
  if (!out || iters <= 0) return NV4_EINVAL;
  nv4::k_lds_read<<<nv4::device_cu_count() * 2, 256, 0, static_cast<hipStream_t>(stream)>>>(out, iters);
  return hipGetLastError() == hipSuccess ? NV4_OK : NV4_EHIP;
}

nv4_status nv4_bench_mfma(float *out, int iters, int waves_per_simd, void *stream) {
  if (!out || iters <= 0 || (waves_per_simd != 1 && waves_per_simd != 2)) return NV4_EINVAL;
  const int grid = nv4::device_cu_count() * waves_per_simd;  // four waves (one per SIMD) per workgroup
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (waves_per_simd == 1) nv4::k_mfma_loop<1><<<grid, 256, 0, s>>>(out, iters);
  else nv4::k_mfma_loop<2><<<grid, 256, 0, s>>>(out, iters);
  return hipGetLastError() == hipSuccess ? NV4_OK : NV4_EHIP;
}

}  // extern "C"
