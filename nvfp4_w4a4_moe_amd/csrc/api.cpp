// C ABI of the NVFP4 W4A4 expert path (declarations and contracts: include/nv4moe.h).
// Host side only: argument validation, workspace carving, dispatch to the kernel
// launchers, and mapping of HIP errors.  No call allocates memory or waits on the
// device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "../../include/nv4moe.h"
#include "nv4_internal.h"

namespace {

thread_local char g_err[512] = "no error";

nv4_status fail(nv4_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

nv4_status ok() {
  snprintf(g_err, sizeof(g_err), "no error");
  return NV4_OK;
}

nv4_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(NV4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

int ngroups_of(int64_t rows, int scale_mode, int nseg) {
  if (scale_mode == NV4_SCALE_TENSOR) return 1;
  if (scale_mode == NV4_SCALE_SEGMENT) return nseg;
  if (scale_mode == NV4_SCALE_SEGMENT_HALVES) return 2 * nseg;
  return (int)rows;
}

}  // namespace

namespace nv4 {

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace nv4

extern "C" {

int nv4_version(void) { return 100; }

const char *nv4_status_string(nv4_status s) {
  switch (s) {
    case NV4_OK: return "ok";
    case NV4_EINVAL: return "invalid argument";
    case NV4_EALIGN: return "misaligned size or pointer";
    case NV4_EUNSUPPORTED: return "unsupported mode combination";
    case NV4_EWORKSPACE: return "workspace too small";
    case NV4_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char *nv4_last_error(void) { return g_err; }

// ---------------------------------------------------------------- quantisation

size_t nvfp4_quantize_workspace(int64_t rows, int64_t K, int layout, int scale_mode, int nseg) {
  (void)K;
  (void)layout;
  const int ng = ngroups_of(rows, scale_mode, nseg);
  return round256((size_t)std::max(ng, 1) * sizeof(float));
}

// nvfp4_quantize and nvfp4_quantize_sr: the same validation and launch, the latter
// with stochastic rounding of the elements
static nv4_status quantize_impl(const void *x, nv4_dtype xtype, int64_t rows, int64_t K, int64_t ldx,
                                const int32_t *row_index, int layout, int scale_mode, int nseg,
                                const int32_t *seg_offsets, const int32_t *seg_padded_offsets,
                                const float *amax_in, float *amax_out, nv4_tensor *out, nv4_tensor *out_rows,
                                void *ws, size_t ws_bytes, int32_t *dev_status, void *stream, int sr,
                                uint64_t sr_seed) {
  if (!out) return fail(NV4_EINVAL, "nvfp4_quantize: out descriptor is NULL");
  if (rows < 0 || K < 0) return fail(NV4_EINVAL, "nvfp4_quantize: negative shape");
  if (xtype != NV4_BF16 && xtype != NV4_F32) return fail(NV4_EINVAL, "nvfp4_quantize: bad input dtype");
  if (layout != NV4_ROWS && layout != NV4_COLS && layout != NV4_COLS_BATCHED && layout != NV4_ROWS_AND_COLS)
    return fail(NV4_EINVAL, "nvfp4_quantize: bad layout %d", layout);
  const bool both = layout == NV4_ROWS_AND_COLS;
  if (both) {
    if (scale_mode != NV4_SCALE_TENSOR)
      return fail(NV4_EUNSUPPORTED, "nvfp4_quantize: NV4_ROWS_AND_COLS needs one tensor scale");
    if (!out_rows || !out_rows->codes || !out_rows->scales || !out_rows->tscale)
      return fail(NV4_EINVAL, "nvfp4_quantize: NV4_ROWS_AND_COLS needs out_rows");
    if (K % 64) return fail(NV4_EALIGN, "nvfp4_quantize: NV4_ROWS_AND_COLS needs K %% 64 == 0");
    if (out_rows->rows != rows || out_rows->K != K)
      return fail(NV4_EINVAL, "nvfp4_quantize: out_rows must be [rows][K]");
    if (!aligned(out_rows->codes, 16) || !aligned(out_rows->scales, 4))
      return fail(NV4_EALIGN, "nvfp4_quantize: out_rows codes must be 16-byte and scales 4-byte aligned");
  }
  if (scale_mode != NV4_SCALE_TENSOR && scale_mode != NV4_SCALE_SEGMENT && scale_mode != NV4_SCALE_ROW &&
      scale_mode != NV4_SCALE_SEGMENT_HALVES)
    return fail(NV4_EINVAL, "nvfp4_quantize: bad scale_mode %d", scale_mode);
  if (scale_mode == NV4_SCALE_SEGMENT_HALVES) {
    if (layout != NV4_COLS_BATCHED)
      return fail(NV4_EUNSUPPORTED, "nvfp4_quantize: NV4_SCALE_SEGMENT_HALVES needs the NV4_COLS_BATCHED layout");
    if (seg_offsets) return fail(NV4_EINVAL, "nvfp4_quantize: NV4_SCALE_SEGMENT_HALVES takes no seg_offsets");
    if (nseg <= 0 || rows % nseg || (rows / nseg) % 32)
      return fail(NV4_EALIGN, "nvfp4_quantize: NV4_SCALE_SEGMENT_HALVES needs rows/nseg to be a multiple of 32");
  }
  if (scale_mode == NV4_SCALE_ROW && layout != NV4_ROWS)
    return fail(NV4_EUNSUPPORTED, "nvfp4_quantize: per-row scales need the NV4_ROWS layout");
  if (row_index && layout == NV4_COLS_BATCHED)
    return fail(NV4_EUNSUPPORTED, "nvfp4_quantize: row_index is not supported with NV4_COLS_BATCHED");
  if (K % 16) return fail(NV4_EALIGN, "nvfp4_quantize: K = %lld is not a multiple of 16", (long long)K);
  if (ldx < K) return fail(NV4_EINVAL, "nvfp4_quantize: ldx < K");
  const int64_t esz = xtype == NV4_F32 ? 4 : 2;
  if ((ldx * esz) % 16 || !aligned(x, 16))
    return fail(NV4_EALIGN, "nvfp4_quantize: x and its row stride must be 16-byte aligned");
  const bool seg_layout = layout != NV4_ROWS;
  if ((scale_mode == NV4_SCALE_SEGMENT || seg_layout) && nseg <= 0)
    return fail(NV4_EINVAL, "nvfp4_quantize: nseg must be positive");
  if ((layout == NV4_COLS || both) && (!seg_offsets || !seg_padded_offsets))
    return fail(NV4_EINVAL, "nvfp4_quantize: NV4_COLS needs seg_offsets and seg_padded_offsets");
  if (layout == NV4_COLS_BATCHED && (rows % nseg || (rows / nseg) % 16))
    return fail(NV4_EALIGN, "nvfp4_quantize: NV4_COLS_BATCHED needs rows/nseg to be a multiple of 16");
  if ((layout == NV4_ROWS || layout == NV4_COLS_BATCHED) && scale_mode == NV4_SCALE_SEGMENT && !seg_offsets &&
      rows % nseg)
    return fail(NV4_EINVAL, "nvfp4_quantize: equal segments need rows %% nseg == 0");
  if (layout == NV4_COLS && scale_mode == NV4_SCALE_SEGMENT && !seg_offsets)
    return fail(NV4_EINVAL, "nvfp4_quantize: segment scales need seg_offsets");
  if (rows >= (1ll << 31) || K >= (1ll << 31)) return fail(NV4_EINVAL, "nvfp4_quantize: shape too large");
  int64_t o_rows, o_K;
  if (layout == NV4_ROWS) { o_rows = rows; o_K = K; }
  else if (layout == NV4_COLS_BATCHED) { o_rows = (int64_t)nseg * K; o_K = rows / nseg; }
  else { o_rows = K; o_K = out->K; }
  if (out->rows != o_rows) return fail(NV4_EINVAL, "nvfp4_quantize: out->rows = %lld, expected %lld",
                                         (long long)out->rows, (long long)o_rows);
  if (layout == NV4_COLS || both) {
    if (out->K % 64) return fail(NV4_EALIGN, "nvfp4_quantize: NV4_COLS needs out->K %% 64 == 0");
    if (out->K < rows + 15 * (int64_t)nseg)
      return fail(NV4_EINVAL, "nvfp4_quantize: out->K must be >= rows + 15 * nseg (padded capacity)");
  } else if (out->K != o_K) {
    return fail(NV4_EINVAL, "nvfp4_quantize: out->K = %lld, expected %lld", (long long)out->K, (long long)o_K);
  }
  if (o_rows * o_K >= (1ll << 32)) return fail(NV4_EINVAL, "nvfp4_quantize: output too large");
  if ((rows > 0 && K > 0) && (!x || !out->codes || !out->scales))
    return fail(NV4_EINVAL, "nvfp4_quantize: NULL data pointer");
  if (!out->tscale) return fail(NV4_EINVAL, "nvfp4_quantize: out->tscale is NULL");
  if (!aligned(out->codes, 16) || !aligned(out->scales, 4))
    return fail(NV4_EALIGN, "nvfp4_quantize: codes must be 16-byte and scales 4-byte aligned");
  const int ng = ngroups_of(rows, scale_mode, nseg);
  const size_t need = nvfp4_quantize_workspace(rows, K, layout, scale_mode, nseg);
  if (!amax_out && !amax_in && (!ws || ws_bytes < need))
    return fail(NV4_EWORKSPACE, "nvfp4_quantize: workspace of %zu bytes required", need);

  out->scale_mode = scale_mode;
  out->nseg = (scale_mode == NV4_SCALE_SEGMENT || scale_mode == NV4_SCALE_SEGMENT_HALVES)
                  ? nseg
                  : (scale_mode == NV4_SCALE_ROW ? (int32_t)rows : 1);
  if (rows == 0 || K == 0) {
    if (ng == 0) return ok();
  }
  nv4::QuantArgs a{};
  a.x = x;
  a.x_is_f32 = xtype == NV4_F32;
  a.rows = rows;
  a.K = K;
  a.ldx = ldx;
  a.row_index = row_index;
  a.layout = layout;
  a.scale_mode = scale_mode;
  a.nseg = nseg > 0 ? nseg : 1;
  a.seg_offsets = seg_offsets;
  a.seg_padded_offsets = seg_padded_offsets;
  a.amax_in = amax_in;
  a.amax_acc = amax_out ? amax_out : static_cast<float *>(ws);
  a.codes = out->codes;
  a.scales = out->scales;
  a.tscale = out->tscale;
  if (both) {
    a.codes2 = out_rows->codes;
    a.scales2 = out_rows->scales;
    a.tscale2 = out_rows->tscale;
    out_rows->scale_mode = NV4_SCALE_TENSOR;
    out_rows->nseg = 1;
  }
  a.out_rows = o_rows;
  a.out_K = (layout == NV4_COLS || both) ? out->K : o_K;
  a.dev_status = dev_status;
  a.ngroups = ng;
  a.sr = sr;
  a.sr_seed = sr_seed;
  return from_hip(nv4::launch_quantize(a, static_cast<hipStream_t>(stream)), "nvfp4_quantize");
}

nv4_status nvfp4_quantize(const void *x, nv4_dtype xtype, int64_t rows, int64_t K, int64_t ldx,
                          const int32_t *row_index, int layout, int scale_mode, int nseg,
                          const int32_t *seg_offsets, const int32_t *seg_padded_offsets,
                          const float *amax_in, float *amax_out, nv4_tensor *out, nv4_tensor *out_rows,
                          void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  return quantize_impl(x, xtype, rows, K, ldx, row_index, layout, scale_mode, nseg, seg_offsets,
                       seg_padded_offsets, amax_in, amax_out, out, out_rows, ws, ws_bytes, dev_status, stream, 0, 0);
}

nv4_status nvfp4_quantize_sr(const void *x, nv4_dtype xtype, int64_t rows, int64_t K, int64_t ldx,
                             const int32_t *row_index, int layout, int scale_mode, int nseg,
                             const int32_t *seg_offsets, const int32_t *seg_padded_offsets,
                             const float *amax_in, float *amax_out, nv4_tensor *out, nv4_tensor *out_rows,
                             void *ws, size_t ws_bytes, int32_t *dev_status, uint64_t seed, void *stream) {
  return quantize_impl(x, xtype, rows, K, ldx, row_index, layout, scale_mode, nseg, seg_offsets,
                       seg_padded_offsets, amax_in, amax_out, out, out_rows, ws, ws_bytes, dev_status, stream, 1,
                       seed);
}

nv4_status nv4_amax(const float *x, int64_t n, float *amax, int32_t *dev_status, void *stream) {
  if (n < 0 || !amax || (n > 0 && !x)) return fail(NV4_EINVAL, "nv4_amax: bad arguments");
  return from_hip(nv4::launch_amax_vec(x, n, amax, dev_status, static_cast<hipStream_t>(stream)), "nv4_amax");
}

// ---------------------------------------------------------------- routing / permutation

size_t moe_permute_workspace(int64_t T, int E, int k) {
  if (T < 0 || E <= 0 || k <= 0) return 0;
  return nv4::permute_workspace_bytes(T, E, k);
}

nv4_status moe_permute(const float *logits, int64_t T, int E, int k, int flags,
                       int32_t *topk_ids, float *topk_w,
                       int32_t *expert_offsets, int32_t *padded_offsets,
                       int32_t *row_token, int32_t *token_row,
                       const nv4_tensor *gather_src, nv4_tensor *gather_dst,
                       void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  if (T < 0) return fail(NV4_EINVAL, "moe_permute: T < 0");
  if (E <= 0 || k <= 0) return fail(NV4_EINVAL, "moe_permute: E and k must be positive");
  if (E > 1024) return fail(NV4_EUNSUPPORTED, "moe_permute: E = %d exceeds 1024", E);
  if (k > 32 || k > E) return fail(NV4_EUNSUPPORTED, "moe_permute: k = %d must be <= min(E, 32)", k);
  if (T * (int64_t)k >= (1ll << 31)) return fail(NV4_EINVAL, "moe_permute: T * k must stay below 2^31");
  if (flags & ~NV4_RENORM) return fail(NV4_EINVAL, "moe_permute: unknown flags");
  if (!topk_ids || !expert_offsets || !row_token || !token_row)
    return fail(NV4_EINVAL, "moe_permute: NULL output pointer");
  if (logits && !topk_w) return fail(NV4_EINVAL, "moe_permute: topk_w is required with logits");
  if ((gather_src == nullptr) != (gather_dst == nullptr))
    return fail(NV4_EINVAL, "moe_permute: gather needs both src and dst");
  int64_t gK = 0;
  if (gather_src) {
    if (gather_src->K != gather_dst->K || gather_src->K % 16 || gather_src->K <= 0)
      return fail(NV4_EALIGN, "moe_permute: gather tensors need equal K, multiple of 16");
    if (gather_src->rows != T || gather_dst->rows != T * (int64_t)k)
      return fail(NV4_EINVAL, "moe_permute: gather shapes must be [T][K] -> [T*k][K]");
    if (!gather_src->codes || !gather_src->scales || !gather_dst->codes || !gather_dst->scales)
      return fail(NV4_EINVAL, "moe_permute: NULL gather buffer");
    if (!aligned(gather_src->codes, 16) || !aligned(gather_dst->codes, 16) || !aligned(gather_src->scales, 4) ||
        !aligned(gather_dst->scales, 4))
      return fail(NV4_EALIGN, "moe_permute: gather buffers misaligned");
    gK = gather_src->K;
  }
  const size_t need = nv4::permute_workspace_bytes(T, E, k);
  if (!ws || ws_bytes < need) return fail(NV4_EWORKSPACE, "moe_permute: workspace of %zu bytes required", need);
  nv4::PermuteArgs a{};
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.k = k;
  a.flags = flags;
  a.topk_ids = topk_ids;
  a.topk_w = topk_w;
  a.expert_offsets = expert_offsets;
  a.padded_offsets = padded_offsets;
  a.row_token = row_token;
  a.token_row = token_row;
  if (gather_src) {
    a.src_codes = gather_src->codes;
    a.src_scales = gather_src->scales;
    a.dst_codes = gather_dst->codes;
    a.dst_scales = gather_dst->scales;
  }
  a.gather_K = gK;
  const int64_t R = T * k;
  const int64_t nchunks = std::max<int64_t>(1, (R + nv4::kPermuteChunk - 1) / nv4::kPermuteChunk);
  a.chunk_counts = static_cast<int32_t *>(ws);
  a.local_rank = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + round256((size_t)nchunks * E * 4));
  a.dev_status = dev_status;
  return from_hip(nv4::launch_permute(a, static_cast<hipStream_t>(stream)), "moe_permute");
}

nv4_status moe_permute_noalloc(const float *logits, int64_t T, int E, int k, int flags,
                               int32_t *topk_ids, float *topk_w,
                               int32_t *expert_offsets, int32_t *padded_offsets,
                               int32_t *row_token, int32_t *token_row,
                               const nv4_tensor *gather_src, nv4_tensor *gather_dst,
                               int32_t *dev_status, void *stream) {
  // the size check comes first: a call that does not fit touches no device
  if (T < 0 || E <= 0 || k <= 0 || E > 1024 || k > 32 || T * (int64_t)k >= (1ll << 31))
    return moe_permute(logits, T, E, k, flags, topk_ids, topk_w, expert_offsets, padded_offsets, row_token,
                       token_row, gather_src, gather_dst, nullptr, 0, dev_status, stream);  // reports the error
  const size_t need = nv4::permute_workspace_bytes(T, E, k);
  if (need > nv4::kPermuteStaticBytes)
    return fail(NV4_EWORKSPACE,
                "moe_permute_noalloc: T = %lld, E = %d, k = %d needs %zu bytes of workspace, above the static %zu; "
                "use moe_permute with a caller workspace",
                (long long)T, E, k, need, nv4::kPermuteStaticBytes);
  void *ws = nullptr;
  const hipError_t e = nv4::permute_static_workspace(&ws);
  if (e != hipSuccess) return from_hip(e, "moe_permute_noalloc: static workspace");
  return moe_permute(logits, T, E, k, flags, topk_ids, topk_w, expert_offsets, padded_offsets, row_token,
                     token_row, gather_src, gather_dst, ws, nv4::kPermuteStaticBytes, dev_status, stream);
}

size_t moe_permute_noalloc_max_workspace(void) { return nv4::kPermuteStaticBytes; }

// ---------------------------------------------------------------- grouped GEMM

// Workspace layout of nvfp4_grouped_gemm: [0, 256) the dynamic tile schedule's counter
// (GROUP_K); then, when K % 64 != 0, A and B repacked to Kp = K rounded up to 64
// (codes, then scale bytes, each region 256-aligned).
static int64_t padded_k(int64_t K) { return (K + 63) / 64 * 64; }
static size_t gemm_ws_bytes(int64_t a_rows, int64_t b_rows, int64_t K, int group_mode) {
  size_t n = group_mode == NV4_GROUP_K ? 256 : 0;
  if (K % 64) {
    const int64_t Kp = padded_k(K);
    n += round256((size_t)a_rows * (Kp / 2)) + round256((size_t)a_rows * (Kp / 16));
    n += round256((size_t)b_rows * (Kp / 2)) + round256((size_t)b_rows * (Kp / 16));
  }
  return n;
}

size_t nvfp4_grouped_gemm_workspace(const nv4_tensor *A, const nv4_tensor *B, int group_mode) {
  if (!A || !B || A->rows < 0 || B->rows < 0 || A->K <= 0) return 0;
  return gemm_ws_bytes(A->rows, B->rows, A->K, group_mode);
}

nv4_status nvfp4_grouped_gemm(const nv4_tensor *A, const nv4_tensor *B, const int32_t *offsets, int E,
                              int64_t M_cap, int64_t N, const int32_t *a_rows,
                              int group_mode, int epilogue,
                              void *C, nv4_dtype ctype, int64_t ldc, float *amax_out,
                              void *ws, size_t ws_bytes, void *stream) {
  if (!A || !B || !offsets || !C) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: NULL argument");
  if (E <= 0 || E > 1024) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: E must be in [1, 1024]");
  if (group_mode != NV4_GROUP_M && group_mode != NV4_GROUP_K)
    return fail(NV4_EINVAL, "nvfp4_grouped_gemm: bad group_mode");
  if (epilogue != NV4_EPI_NONE && epilogue != NV4_EPI_SWIGLU)
    return fail(NV4_EINVAL, "nvfp4_grouped_gemm: bad epilogue");
  if (ctype != NV4_BF16 && ctype != NV4_F32) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: bad C dtype");
  if (A->K != B->K) return fail(NV4_EALIGN, "nvfp4_grouped_gemm: A->K != B->K");
  if (A->K <= 0 || A->K % 16)
    return fail(NV4_EALIGN, "nvfp4_grouped_gemm: K = %lld must be a positive multiple of 16", (long long)A->K);
  if (!A->codes || !A->scales || !A->tscale || !B->codes || !B->scales || !B->tscale)
    return fail(NV4_EINVAL, "nvfp4_grouped_gemm: NULL tensor buffer");
  // (K % 64 != 0: both operands are first repacked, zero-padded to a multiple of 64, into the workspace)
  const bool repack = A->K % 64 != 0;
  if (!aligned(A->codes, 16) || !aligned(B->codes, 16) || (!repack && (!aligned(A->scales, 4) ||
                                                                       !aligned(B->scales, 4))))
    return fail(NV4_EALIGN, "nvfp4_grouped_gemm: codes must be 16-byte and scales 4-byte aligned");
  // the kernel addresses operands with 32-bit byte offsets and C with 32-bit element offsets
  const int64_t Kk = padded_k(A->K);
  if (A->rows < 0 || B->rows < 0 || A->rows * (Kk / 2) >= (1ll << 32) || B->rows * (Kk / 2) >= (1ll << 32))
    return fail(NV4_EINVAL, "nvfp4_grouped_gemm: each operand must stay below 4 GiB of codes");
  const size_t need = gemm_ws_bytes(A->rows, B->rows, A->K, group_mode);
  if (repack && (!ws || ws_bytes < need))
    return fail(NV4_EWORKSPACE, "nvfp4_grouped_gemm: K = %lld needs a workspace of %zu bytes (repacked operands)",
                (long long)A->K, need);
  if (ws && !aligned(ws, 256) && repack)
    return fail(NV4_EALIGN, "nvfp4_grouped_gemm: workspace must be 256-byte aligned");
  nv4::GemmArgs g{};
  g.a_codes = A->codes;
  g.a_scales = A->scales;
  g.a_tscale = A->tscale;
  g.a_scale_mode = A->scale_mode;
  g.a_rows = A->rows;
  g.K = A->K;
  g.a_rows_index = a_rows;
  g.b_codes = B->codes;
  g.b_scales = B->scales;
  g.b_tscale = B->tscale;
  g.b_scale_mode = B->scale_mode;
  g.b_nseg = B->nseg;
  g.b_rows = B->rows;
  g.offsets = offsets;
  g.E = E;
  g.M_cap = M_cap;
  g.N = N;
  g.group_mode = group_mode;
  g.epilogue = epilogue;
  g.C = C;
  g.c_is_f32 = ctype == NV4_F32;
  g.ldc = ldc;
  g.amax_out = amax_out;
  if (group_mode == NV4_GROUP_K && ws && ws_bytes >= 4) {
    if (!aligned(ws, 4)) return fail(NV4_EALIGN, "nvfp4_grouped_gemm: workspace must be 4-byte aligned");
    g.tile_counter = static_cast<int32_t *>(ws);
  }
  if (group_mode == NV4_GROUP_M) {
    const int64_t Nb = epilogue == NV4_EPI_SWIGLU ? 2 * N : N;
    if (N <= 0) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: N must be positive");
    if (B->rows != (int64_t)E * Nb)
      return fail(NV4_EINVAL, "nvfp4_grouped_gemm: B->rows = %lld, expected E * %lld", (long long)B->rows,
                  (long long)Nb);
    if (A->scale_mode != NV4_SCALE_TENSOR && A->scale_mode != NV4_SCALE_ROW)
      return fail(NV4_EUNSUPPORTED, "nvfp4_grouped_gemm: A scales must be per tensor or per row");
    if (B->scale_mode == NV4_SCALE_SEGMENT) {
      const bool swiglu2 = epilogue == NV4_EPI_SWIGLU && B->nseg == 2 * E;
      if (B->nseg != E && !swiglu2)
        return fail(NV4_EINVAL,
                    "nvfp4_grouped_gemm: B has %d scale segments, expected E = %d (or 2E with the SwiGLU epilogue)",
                    B->nseg, E);
    } else if (B->scale_mode == NV4_SCALE_SEGMENT_HALVES) {
      if (epilogue != NV4_EPI_NONE || A->scale_mode != NV4_SCALE_TENSOR)
        return fail(NV4_EUNSUPPORTED,
                    "nvfp4_grouped_gemm: per-K-half B scales need EPI_NONE and a per-tensor A scale");
      if (B->nseg != E)
        return fail(NV4_EINVAL, "nvfp4_grouped_gemm: B has %d scale segments, expected E = %d", B->nseg, E);
      if ((A->K / 2) % 128)
        return fail(NV4_EUNSUPPORTED, "nvfp4_grouped_gemm: per-K-half B scales need (K/2) %% 128 == 0");
    } else if (B->scale_mode != NV4_SCALE_TENSOR) {
      return fail(NV4_EUNSUPPORTED, "nvfp4_grouped_gemm: B scales must be per tensor, expert or projection");
    }
    if (M_cap < 0 || (a_rows == nullptr && M_cap > A->rows))
      return fail(NV4_EINVAL, "nvfp4_grouped_gemm: M_cap exceeds the rows of A");
    if (ldc < N) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: ldc < N");
    if (M_cap * ldc >= (1ll << 31)) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: C must stay below 2^31 elements");
  } else {
    if (epilogue != NV4_EPI_NONE) return fail(NV4_EUNSUPPORTED, "nvfp4_grouped_gemm: GROUP_K has no SwiGLU epilogue");
    if (a_rows) return fail(NV4_EUNSUPPORTED, "nvfp4_grouped_gemm: GROUP_K takes no row index");
    if (A->scale_mode != NV4_SCALE_TENSOR || B->scale_mode != NV4_SCALE_TENSOR)
      return fail(NV4_EUNSUPPORTED, "nvfp4_grouped_gemm: GROUP_K needs per-tensor scales");
    if (ldc < B->rows) return fail(NV4_EINVAL, "nvfp4_grouped_gemm: ldc < rows of B");
    if ((int64_t)E * A->rows * ldc >= (1ll << 31))
      return fail(NV4_EINVAL, "nvfp4_grouped_gemm: C must stay below 2^31 elements");
    g.N = B->rows;
  }
  // exact FP16 B (decoded weights): GROUP_M, one tensor scale for A, whole 64-wide stages
  if (B->f16 && group_mode == NV4_GROUP_M && A->scale_mode == NV4_SCALE_TENSOR && A->K % 64 == 0) {
    if (!aligned(B->f16, 16)) return fail(NV4_EALIGN, "nvfp4_grouped_gemm: B->f16 must be 16-byte aligned");
    if (B->rows * A->K * 2 >= (1ll << 32))
      return fail(NV4_EINVAL, "nvfp4_grouped_gemm: B->f16 must stay below 4 GiB");
    g.b_f16 = B->f16;
  }
  if (repack) {
    // zero-padded copies of both operands, then the GEMM on K = Kp (padded blocks carry
    // scale 0 and add exact zeros)
    char *p = static_cast<char *>(ws) + (group_mode == NV4_GROUP_K ? 256 : 0);
    uint8_t *ac = reinterpret_cast<uint8_t *>(p);
    p += round256((size_t)A->rows * (Kk / 2));
    uint8_t *as = reinterpret_cast<uint8_t *>(p);
    p += round256((size_t)A->rows * (Kk / 16));
    uint8_t *bc = reinterpret_cast<uint8_t *>(p);
    p += round256((size_t)B->rows * (Kk / 2));
    uint8_t *bs = reinterpret_cast<uint8_t *>(p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = nv4::launch_repack_k(A->codes, A->scales, A->rows, A->K, ac, as, Kk, st);
    if (e == hipSuccess) e = nv4::launch_repack_k(B->codes, B->scales, B->rows, B->K, bc, bs, Kk, st);
    if (e != hipSuccess) return from_hip(e, "nvfp4_grouped_gemm: repack");
    g.a_codes = ac;
    g.a_scales = as;
    g.b_codes = bc;
    g.b_scales = bs;
    g.K = Kk;
  }
  return from_hip(nv4::launch_grouped_gemm(g, static_cast<hipStream_t>(stream)), "nvfp4_grouped_gemm");
}

nv4_status bf16_grouped_gemm(const void *A, int64_t a_rows_n, const void *B, int64_t b_rows_n, int64_t K,
                             const int32_t *offsets, int E, int64_t M_cap, int64_t N, const int32_t *a_rows,
                             int group_mode, int epilogue, void *C, nv4_dtype ctype, int64_t ldc,
                             float *amax_out, void *ws, size_t ws_bytes, void *stream) {
  if (!A || !B || !offsets || !C) return fail(NV4_EINVAL, "bf16_grouped_gemm: NULL argument");
  if (E <= 0 || E > 1024) return fail(NV4_EINVAL, "bf16_grouped_gemm: E must be in [1, 1024]");
  if (group_mode != NV4_GROUP_M && group_mode != NV4_GROUP_K)
    return fail(NV4_EINVAL, "bf16_grouped_gemm: bad group_mode");
  if (epilogue != NV4_EPI_NONE && epilogue != NV4_EPI_SWIGLU)
    return fail(NV4_EINVAL, "bf16_grouped_gemm: bad epilogue");
  if (ctype != NV4_BF16 && ctype != NV4_F32) return fail(NV4_EINVAL, "bf16_grouped_gemm: bad C dtype");
  if (K <= 0 || K % 32)
    return fail(NV4_EALIGN, "bf16_grouped_gemm: K = %lld must be a positive multiple of 32", (long long)K);
  if (!aligned(A, 16) || !aligned(B, 16)) return fail(NV4_EALIGN, "bf16_grouped_gemm: A and B must be 16-byte aligned");
  // the kernel addresses operands with 32-bit byte offsets and C with 32-bit element offsets
  if (a_rows_n < 0 || b_rows_n < 0 || a_rows_n * K * 2 >= (1ll << 32) || b_rows_n * K * 2 >= (1ll << 32))
    return fail(NV4_EINVAL, "bf16_grouped_gemm: each operand must stay below 4 GiB");
  nv4::GemmArgs g{};
  g.operands_bf16 = 1;
  if (group_mode == NV4_GROUP_K && ws && ws_bytes >= 4) {
    if (!aligned(ws, 4)) return fail(NV4_EALIGN, "bf16_grouped_gemm: workspace must be 4-byte aligned");
    g.tile_counter = static_cast<int32_t *>(ws);
  }
  g.a_codes = static_cast<const uint8_t *>(A);
  g.a_scale_mode = NV4_SCALE_TENSOR;
  g.a_rows = a_rows_n;
  g.K = K;
  g.a_rows_index = a_rows;
  g.b_codes = static_cast<const uint8_t *>(B);
  g.b_scale_mode = NV4_SCALE_TENSOR;
  g.b_rows = b_rows_n;
  g.offsets = offsets;
  g.E = E;
  g.M_cap = M_cap;
  g.N = N;
  g.group_mode = group_mode;
  g.epilogue = epilogue;
  g.C = C;
  g.c_is_f32 = ctype == NV4_F32;
  g.ldc = ldc;
  g.amax_out = amax_out;
  if (group_mode == NV4_GROUP_M) {
    const int64_t Nb = epilogue == NV4_EPI_SWIGLU ? 2 * N : N;
    if (N <= 0) return fail(NV4_EINVAL, "bf16_grouped_gemm: N must be positive");
    if (b_rows_n != (int64_t)E * Nb)
      return fail(NV4_EINVAL, "bf16_grouped_gemm: B has %lld rows, expected E * %lld", (long long)b_rows_n,
                  (long long)Nb);
    if (M_cap < 0 || (a_rows == nullptr && M_cap > a_rows_n))
      return fail(NV4_EINVAL, "bf16_grouped_gemm: M_cap exceeds the rows of A");
    if (ldc < N) return fail(NV4_EINVAL, "bf16_grouped_gemm: ldc < N");
    if (M_cap * ldc >= (1ll << 31)) return fail(NV4_EINVAL, "bf16_grouped_gemm: C must stay below 2^31 elements");
  } else {
    if (epilogue != NV4_EPI_NONE) return fail(NV4_EUNSUPPORTED, "bf16_grouped_gemm: GROUP_K has no SwiGLU epilogue");
    if (a_rows) return fail(NV4_EUNSUPPORTED, "bf16_grouped_gemm: GROUP_K takes no row index");
    if (ldc < b_rows_n) return fail(NV4_EINVAL, "bf16_grouped_gemm: ldc < rows of B");
    if ((int64_t)E * a_rows_n * ldc >= (1ll << 31))
      return fail(NV4_EINVAL, "bf16_grouped_gemm: C must stay below 2^31 elements");
    g.N = b_rows_n;
  }
  return from_hip(nv4::launch_grouped_gemm(g, static_cast<hipStream_t>(stream)), "bf16_grouped_gemm");
}

// ---------------------------------------------------------------- BF16 operands

nv4_status nvfp4_decode_f16(const nv4_tensor *q, void *out, int64_t ldo, void *stream) {
  if (!q) return fail(NV4_EINVAL, "nvfp4_decode_f16: q is NULL");
  if (q->rows < 0 || q->K < 0) return fail(NV4_EINVAL, "nvfp4_decode_f16: negative shape");
  if (q->K % 16) return fail(NV4_EALIGN, "nvfp4_decode_f16: K = %lld is not a multiple of 16", (long long)q->K);
  if (ldo < q->K || ldo % 8) return fail(NV4_EALIGN, "nvfp4_decode_f16: ldo must be >= K and a multiple of 8");
  if (q->rows == 0 || q->K == 0) return NV4_OK;
  if (!q->codes || !q->scales || !out) return fail(NV4_EINVAL, "nvfp4_decode_f16: NULL buffer");
  if (!aligned(q->codes, 8) || !aligned(out, 16))
    return fail(NV4_EALIGN, "nvfp4_decode_f16: codes must be 8-byte and out 16-byte aligned");
  return from_hip(nv4::launch_decode_f16(q->codes, q->scales, q->rows, q->K, static_cast<uint16_t *>(out), ldo,
                                         static_cast<hipStream_t>(stream)),
                  "nvfp4_decode_f16");
}

nv4_status nv4_to_bf16(const void *x, int64_t x_rows, int64_t ldx, const nv4_tensor *q, int64_t rows, int64_t K,
                       const int32_t *row_index, int layout, int nseg, const int32_t *seg_offsets,
                       const int32_t *seg_padded_offsets, void *out, int64_t out_rows, int64_t out_cols,
                       void *stream) {
  // an empty source (rows == 0) may come with NULL pointers: nothing is read
  if (x && q) return fail(NV4_EINVAL, "nv4_to_bf16: give exactly one of x and q");
  if (!x && !q && rows != 0) return fail(NV4_EINVAL, "nv4_to_bf16: give exactly one of x and q");
  if (!out && out_rows * out_cols != 0) return fail(NV4_EINVAL, "nv4_to_bf16: NULL out");
  if (rows < 0 || K <= 0) return fail(NV4_EINVAL, "nv4_to_bf16: bad shape");
  if (K % 16) return fail(NV4_EALIGN, "nv4_to_bf16: K must be a multiple of 16");
  if (!aligned(out, 16)) return fail(NV4_EALIGN, "nv4_to_bf16: out must be 16-byte aligned");
  nv4::ConvertArgs a{};
  if (x) {
    if (ldx < K || ldx % 8) return fail(NV4_EALIGN, "nv4_to_bf16: ldx must be >= K and a multiple of 8");
    if (!aligned(x, 16)) return fail(NV4_EALIGN, "nv4_to_bf16: x must be 16-byte aligned");
    if (x_rows < 0 || (!row_index && x_rows != rows)) return fail(NV4_EINVAL, "nv4_to_bf16: x_rows != rows");
    if (row_index && rows > 0 && x_rows == 0) return fail(NV4_EINVAL, "nv4_to_bf16: row index into an empty x");
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.src_rows = x_rows;
  } else if (q) {
    if (!q->codes || !q->scales || !q->tscale) return fail(NV4_EINVAL, "nv4_to_bf16: NULL tensor buffer");
    if (q->K != K) return fail(NV4_EINVAL, "nv4_to_bf16: q->K != K");
    if (!aligned(q->codes, 8)) return fail(NV4_EALIGN, "nv4_to_bf16: codes must be 8-byte aligned");
    if (!row_index && q->rows != rows) return fail(NV4_EINVAL, "nv4_to_bf16: q->rows != rows");
    if (row_index && rows > 0 && q->rows <= 0) return fail(NV4_EINVAL, "nv4_to_bf16: row index into an empty q");
    if (q->scale_mode == NV4_SCALE_SEGMENT && (q->nseg <= 0 || q->rows % q->nseg))
      return fail(NV4_EINVAL, "nv4_to_bf16: segment scales need q->rows % q->nseg == 0");
    if (q->scale_mode == NV4_SCALE_SEGMENT_HALVES)
      return fail(NV4_EUNSUPPORTED, "nv4_to_bf16: per-K-half scales are not supported as a source");
    if (q->scale_mode != NV4_SCALE_TENSOR && q->scale_mode != NV4_SCALE_SEGMENT && q->scale_mode != NV4_SCALE_ROW)
      return fail(NV4_EINVAL, "nv4_to_bf16: bad q->scale_mode");
    a.codes = q->codes;
    a.scales = q->scales;
    a.tscale = q->tscale;
    a.scale_mode = q->scale_mode;
    a.src_rows = q->rows;
    a.src_nseg = q->nseg;
  }
  a.rows = rows;
  a.K = K;
  a.row_index = row_index;
  a.layout = layout;
  a.nseg = nseg;
  a.seg_offsets = seg_offsets;
  a.seg_padded_offsets = seg_padded_offsets;
  a.out = static_cast<uint16_t *>(out);
  a.out_rows = out_rows;
  a.out_cols = out_cols;
  if (layout == NV4_ROWS) {
    if (out_rows != rows || out_cols != K) return fail(NV4_EINVAL, "nv4_to_bf16: ROWS output must be [rows][K]");
  } else if (layout == NV4_COLS) {
    if (nseg < 1 || nseg > (1 << 20) || !seg_offsets || !seg_padded_offsets)
      return fail(NV4_EINVAL, "nv4_to_bf16: COLS needs nseg >= 1 and both offset arrays");
    if (out_rows != K) return fail(NV4_EINVAL, "nv4_to_bf16: COLS output must have K rows");
    if (out_cols < rows + 15 * (int64_t)nseg || out_cols % 8)
      return fail(NV4_EINVAL, "nv4_to_bf16: COLS output needs >= rows + 15 * nseg columns, a multiple of 8");
  } else if (layout == NV4_COLS_BATCHED) {
    if (row_index) return fail(NV4_EUNSUPPORTED, "nv4_to_bf16: COLS_BATCHED takes no row index");
    if (nseg < 1 || nseg > 65535 || rows % nseg || (rows / nseg) % 16)
      return fail(NV4_EINVAL, "nv4_to_bf16: COLS_BATCHED needs rows / nseg a multiple of 16");
    if (out_rows != (int64_t)nseg * K || out_cols != rows / nseg)
      return fail(NV4_EINVAL, "nv4_to_bf16: COLS_BATCHED output must be [nseg * K][rows / nseg]");
  } else {
    return fail(NV4_EINVAL, "nv4_to_bf16: bad layout");
  }
  return from_hip(nv4::launch_convert(a, static_cast<hipStream_t>(stream)), "nv4_to_bf16");
}

// ---------------------------------------------------------------- combine

nv4_status moe_combine(const void *Y, nv4_dtype ytype, int64_t ldy, const int32_t *token_row,
                       const float *topk_w, int64_t T, int k, int64_t H,
                       void *out, nv4_dtype otype, void *stream) {
  if (T < 0 || k <= 0 || H <= 0) return fail(NV4_EINVAL, "moe_combine: bad shape");
  if (ytype != NV4_BF16 && ytype != NV4_F32) return fail(NV4_EINVAL, "moe_combine: bad Y dtype");
  if (otype != NV4_BF16 && otype != NV4_F32) return fail(NV4_EINVAL, "moe_combine: bad out dtype");
  if (T > 0 && (!Y || !token_row || !topk_w || !out)) return fail(NV4_EINVAL, "moe_combine: NULL pointer");
  if (H % 4 || ldy % 4 || ldy < H) return fail(NV4_EALIGN, "moe_combine: H and ldy must be multiples of 4, ldy >= H");
  if (!aligned(Y, 16) || !aligned(out, 16)) return fail(NV4_EALIGN, "moe_combine: Y and out must be 16-byte aligned");
  nv4::CombineArgs a{};
  a.Y = Y;
  a.y_is_f32 = ytype == NV4_F32;
  a.ldy = ldy;
  a.token_row = token_row;
  a.topk_w = topk_w;
  a.T = T;
  a.k = k;
  a.H = H;
  a.out = out;
  a.out_is_f32 = otype == NV4_F32;
  return from_hip(nv4::launch_combine(a, static_cast<hipStream_t>(stream)), "moe_combine");
}

}  // extern "C"
