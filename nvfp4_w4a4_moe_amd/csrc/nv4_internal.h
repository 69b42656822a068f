// Internal launch interface between the C ABI (api.cpp) and the kernel files.
// Every launcher only enqueues work on `stream`; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nv4 {

// ---------------------------------------------------------------- quantisation
struct QuantArgs {
  const void *x;
  int x_is_f32;
  int64_t rows, K, ldx;
  const int32_t *row_index;  // may be null: logical row r reads x row row_index[r]
  int layout;        // NV4_ROWS / NV4_COLS / NV4_COLS_BATCHED
  int scale_mode;    // NV4_SCALE_*
  int nseg;
  const int32_t *seg_offsets;         // may be null
  const int32_t *seg_padded_offsets;  // NV4_COLS
  const float *amax_in;               // may be null
  float *amax_acc;                    // ngroups floats: amax_out or workspace
  uint8_t *codes;
  uint8_t *scales;
  float *tscale;
  int64_t out_rows, out_K;            // output tensor shape (codes row stride out_K/2)
  uint8_t *codes2, *scales2;          // NV4_ROWS_AND_COLS: the row-direction output [rows][K]
  float *tscale2;
  int32_t *dev_status;
  int ngroups;
  int sr;                             // 1: stochastic rounding of the elements
  uint64_t sr_seed;
};
hipError_t launch_quantize(const QuantArgs &a, hipStream_t stream);
hipError_t launch_amax_vec(const float *x, int64_t n, float *amax, int32_t *dev_status, hipStream_t stream);

// ---------------------------------------------------------------- routing / permutation
constexpr int kPermuteChunk = 1024;  // assignments ranked per wave
struct PermuteArgs {
  const float *logits;
  int64_t T;
  int E, k, flags;
  int32_t *topk_ids;
  float *topk_w;
  int32_t *expert_offsets, *padded_offsets, *row_token, *token_row;
  const uint8_t *src_codes, *src_scales;
  uint8_t *dst_codes, *dst_scales;
  int64_t gather_K;  // 0 = no gather
  int32_t *chunk_counts;  // workspace [nchunks][E]
  int32_t *local_rank;    // workspace [T*k]
  int32_t *dev_status;
};
size_t permute_workspace_bytes(int64_t T, int E, int k);
hipError_t launch_permute(const PermuteArgs &a, hipStream_t stream);
// moe_permute_noalloc: the device address of this device's static workspace of
// kPermuteStaticBytes (looked up once per device, then cached)
constexpr size_t kPermuteStaticBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t permute_static_workspace(void **ptr);

// ---------------------------------------------------------------- grouped GEMM
struct GemmArgs {
  const uint8_t *a_codes, *a_scales;
  const float *a_tscale;
  int a_scale_mode;
  int64_t a_rows, K;
  const int32_t *a_rows_index;   // may be null
  const uint8_t *b_codes, *b_scales;
  const float *b_tscale;
  int b_scale_mode;
  int b_nseg;                    // scale segments of B (SCALE_SEGMENT: E, or 2E gate/up; HALVES: E)
  int64_t b_rows;
  const int32_t *offsets;
  int E;
  int64_t M_cap, N;              // N = output columns
  int group_mode, epilogue;
  void *C;
  int c_is_f32;
  int64_t ldc;
  float *amax_out;
  int operands_bf16;             // 1: a_codes / b_codes hold BF16 elements (no scales)
  const uint16_t *b_f16;         // GROUP_M: B as exact FP16 values [b_rows][K] (no decode), or null
  int32_t *tile_counter;         // GROUP_K: workspace word for the dynamic tile schedule, or null
};
hipError_t launch_grouped_gemm(const GemmArgs &a, hipStream_t stream);
// copy an NVFP4 operand [rows][K] (K % 16 == 0) into [rows][Kp] (Kp % 64 == 0, Kp >= K):
// the extra codes and scale bytes are zero, so the padded blocks add exact zeros
hipError_t launch_repack_k(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                           uint8_t *codes_p, uint8_t *scales_p, int64_t Kp, hipStream_t stream);

// ---------------------------------------------------------------- BF16 operands
struct ConvertArgs {
  const uint16_t *x;                  // BF16 source [.][ldx], or null
  int64_t ldx;
  const uint8_t *codes, *scales;      // NVFP4 source, or null
  const float *tscale;
  int scale_mode;                     // of the NVFP4 source
  int64_t src_rows;                   // rows of the source (x or the NVFP4 tensor)
  int src_nseg;
  int64_t rows, K;                    // logical rows (after the gather) and columns
  const int32_t *row_index;           // may be null
  int layout;                         // NV4_ROWS / NV4_COLS / NV4_COLS_BATCHED
  int nseg;
  const int32_t *seg_offsets, *seg_padded_offsets;
  uint16_t *out;
  int64_t out_rows, out_cols;
};
hipError_t launch_convert(const ConvertArgs &a, hipStream_t stream);
// exact FP16 values e2m1 * e4m3 of an NVFP4 tensor [rows][K] into out [rows][ldo]
hipError_t launch_decode_f16(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, uint16_t *out,
                             int64_t ldo, hipStream_t stream);

// ---------------------------------------------------------------- combine
struct CombineArgs {
  const void *Y;
  int y_is_f32;
  int64_t ldy;
  const int32_t *token_row;
  const float *topk_w;
  int64_t T;
  int k;
  int64_t H;
  void *out;
  int out_is_f32;
};
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream);

// number of compute units of the current device (cached per device)
int device_cu_count();

}  // namespace nv4
