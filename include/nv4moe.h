/*
 * nv4moe.h -- C ABI of the NVFP4 W4A4 mixture-of-experts expert path for AMD
 * Instinct MI355X (gfx950, CDNA4).
 *
 * The path is the expert computation of a mixture-of-experts layer with both
 * operands of every expert GEMM in NVFP4 ("W4A4"): quantise activations and
 * weights, permute tokens by expert, run the grouped expert GEMMs (gate/up with
 * a fused SwiGLU, then down), and combine the top-k expert outputs back into
 * token order with the routing weights.  Sources:
 *
 *   [LBP]  "Low-Bit Precision Training Is Ready for Production: What Engineering
 *          Leaders Need to Know Before Adopting NVFP4" (vector-labs.ai)
 *   [4BL]  "The 4-bitter Lesson: Balancing Stability and Performance in NVFP4 RL"
 *   [MTE]  "miniTE identifies and closes the execution gap in native NVFP4
 *          reinforcement learning" (n884.com)
 *
 * NVFP4 ([4BL], section "Baseline: A starting recipe with stable training
 * dynamics"): blocks of 16 FP4 E2M1 values, each block with an FP8 E4M3 scale,
 * plus one FP32 scale for the tensor.  The element and scale formats are those
 * of the OCP MX v1.0 (E2M1) and OCP OFP8 (E4M3, max 448) specifications.
 *
 * Numerics fixed by this library (the pages leave them open; [LBP], section
 * "The Cross-Engine Alignment Problem", names scale domains, rounding modes,
 * accumulation precision and operator composition as the choices two engines
 * must agree on):
 *   A  = max|x| over the scale group;  S = fp32(2688 / A), or 1 if A == 0 or the
 *        quotient is not finite;  the stored FP32 tensor scale is G = fp32(1 / S).
 *   per 16-block:  sf = E4M3_rne_sat(fp32(fp32(max|x_b| / 6) * S));
 *                  inv = sf ? fp32(S / sf) : 0;   q = E2M1_rne_sat(fp32(x * inv)).
 *   value(q, sf, G) = e2m1(q) * sf * G.  Element 2i sits in the low nibble of
 *   byte i; an FP4 code is sign << 3 | magnitude index (0, .5, 1, 1.5, 2, 3, 4, 6).
 *   Every FP32 step is one correctly rounded operation, so codes and scale bytes
 *   are exactly defined.  GEMMs multiply the exactly decoded operands
 *   (e2m1 * sf fits BF16 exactly) with FP32 accumulation and apply G_a * G_b in
 *   the epilogue.  Every call is deterministic: repeated calls on the same input
 *   give bitwise identical output.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers unless marked (host).  The caller
 *     owns every buffer (inputs, outputs, workspace); the library never allocates
 *     or frees memory and keeps no state besides a thread-local error message.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *     work; nothing waits on the host and no device value is read back.
 *   - Shapes are validated on the host before any launch; a failed check returns
 *     an error status and enqueues nothing.  nv4_last_error() explains it.
 *   - Faults in the data itself (non-finite values, expert ids out of range, NaN
 *     logits) are never checked on the host: kernels OR bits into the optional
 *     device word `dev_status` (NV4_DS_*), which the caller reads after
 *     synchronising.  Results computed from such data are unspecified.
 *   - Index arithmetic is 32-bit on the device: rows * K and T * k must stay
 *     below 2^31.
 */
#ifndef NV4MOE_H
#define NV4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nv4_status {
  NV4_OK = 0,
  NV4_EINVAL = -1,        /* NULL where a pointer is required, negative or inconsistent size */
  NV4_EALIGN = -2,        /* K or a stride not a multiple of 16, or a misaligned pointer */
  NV4_EUNSUPPORTED = -3,  /* a combination of modes this library does not implement */
  NV4_EWORKSPACE = -4,    /* workspace smaller than the matching *_workspace() query */
  NV4_EHIP = -5           /* a HIP launch failed (hipGetLastError) */
} nv4_status;

typedef enum nv4_dtype { NV4_BF16 = 0, NV4_F32 = 1 } nv4_dtype;

/* quantisation direction (nvfp4_quantize `layout`) */
#define NV4_ROWS 1          /* blocks of 16 along the contiguous dimension K */
#define NV4_COLS 2          /* transpose: blocks of 16 down the rows of each segment */
#define NV4_COLS_BATCHED 3  /* transpose each of nseg equal row-slices separately */
#define NV4_ROWS_AND_COLS 4 /* NV4_COLS into out and NV4_ROWS into out_rows, one read of x */

/* tensor-scale grouping (nvfp4_quantize `scale_mode`, nv4_tensor.scale_mode) */
#define NV4_SCALE_TENSOR 0  /* one G for the whole tensor */
#define NV4_SCALE_SEGMENT 1 /* one G per segment (expert) */
#define NV4_SCALE_ROW 2     /* one G per row: the per-token variant */
#define NV4_SCALE_SEGMENT_HALVES 3 /* one G per half of each segment's rows (NV4_COLS_BATCHED): two
                                    * projections stacked in one matrix, e.g. an expert's gate and up
                                    * weights; in the transposed output they are the two halves of K */

/* grouped GEMM */
#define NV4_GROUP_M 0       /* expert e owns rows [offsets[e], offsets[e+1]) of A and C */
#define NV4_GROUP_K 1       /* expert e owns columns [offsets[e], offsets[e+1]) of the K dimension */
#define NV4_EPI_NONE 0
#define NV4_EPI_SWIGLU 1

/* routing flags */
#define NV4_RENORM 1        /* divide the k routing weights of a token by their sum */

/* dev_status bits */
#define NV4_DS_NONFINITE 1  /* a quantiser met a NaN or infinity */
#define NV4_DS_BAD_EXPERT 2 /* an expert id outside [0, E) */
#define NV4_DS_NAN_LOGIT 4  /* a NaN router logit */

/*
 * One NVFP4 tensor of logical shape [rows][K] (K % 16 == 0), memory owned by the
 * caller:
 *   codes  [rows][K/2]   packed E2M1 codes, row-major, rows K/2 bytes apart
 *   scales [rows][K/16]  E4M3 block scales, row-major
 *   tscale               FP32 decode scales G: 1 (SCALE_TENSOR), nseg
 *                        (SCALE_SEGMENT: segment s = rows [s*rows/nseg, (s+1)*rows/nseg)
 *                        when used as a grouped-GEMM B operand), rows (SCALE_ROW), or
 *                        2*nseg (SCALE_SEGMENT_HALVES: segment s = rows [s*rows/nseg,
 *                        (s+1)*rows/nseg), tscale[2s] for columns [0, K/2) and
 *                        tscale[2s+1] for [K/2, K))
 *
 * Weight scale groups ([4BL] "Why is the NVFP4 pretraining recipe not sufficient for
 * RL?": one FP32 scale per weight tensor; its footnote 5 counts three projection
 * matrices per expert): every projection of every expert has its own G.  The
 * stacked gate/up weights W13 [E*2I][K] are SCALE_SEGMENT with nseg = 2E (segment 2e
 * is gate_e, 2e+1 is up_e); the down weights W2 [E*H][I] SCALE_SEGMENT with nseg = E;
 * the per-expert transposes of the data gradients are NV4_COLS_BATCHED outputs: W2^T
 * SCALE_SEGMENT (nseg = E) and W13^T [E*H][2I] SCALE_SEGMENT_HALVES (nseg = E).
 */
typedef struct nv4_tensor {
  uint8_t *codes;
  uint8_t *scales;
  float *tscale;
  int64_t rows;
  int64_t K;
  int32_t scale_mode;
  int32_t nseg;
  /* Optional (NULL when absent): the tensor's exact FP16 values without the decode
   * scale, e2m1(code) * e4m3(block scale) for every element, [rows][K] row-major,
   * 16-byte aligned (nvfp4_decode_f16 makes them).  Only B of a GROUP_M
   * nvfp4_grouped_gemm reads them (see there); codes, scales and tscale stay
   * required. */
  const uint16_t *f16;
} nv4_tensor;

/* Library version (major * 10000 + minor * 100 + patch). */
int nv4_version(void);

/* Text for a status code, and the detail of the last failed call on this thread
 * (host strings owned by the library; never NULL). */
const char *nv4_status_string(nv4_status s);
const char *nv4_last_error(void);

/*
 * nvfp4_quantize -- NVFP4 quantisation of a BF16 or FP32 matrix.
 * [4BL] "Baseline: A starting recipe with stable training dynamics" (format);
 * [4BL] "Why is the NVFP4 pretraining recipe not sufficient for RL?" (one FP32
 * scale per weight tensor; per-token activation scale, fused into the quantiser);
 * [4BL] "Improving Gradient Stability", footnote 6 (clip(round(w/s)));
 * [LBP] "What W4A4 GEMM Actually Changes" (per-tensor or per-token scaling).
 *
 *   x, xtype, ldx    input [rows][ldx] (element stride ldx >= K), BF16 or FP32.
 *   row_index        device int32 [rows] or NULL (ROWS and COLS layouts): logical
 *                    row r is read from row row_index[r] of x (a gather fused into
 *                    the load, e.g. tokens in expert order through moe_permute's
 *                    row_token); every index must address a row of x.
 *   layout           NV4_ROWS: out is [rows][K], blocks along K.
 *                    NV4_COLS: out is the transpose [K][Kout] of x, where row
 *                      segment s of x (rows [seg_offsets[s], seg_offsets[s+1]))
 *                      lands in out columns [seg_padded_offsets[s], ...); every
 *                      segment starts a new block and is zero-padded to a
 *                      multiple of 16 (padding is written as code 0 / scale 0).
 *                      out->K is the column capacity: >= rows + 15 * nseg, % 16.
 *                      Used for the re-quantised operands of the weight gradients.
 *                    NV4_ROWS_AND_COLS: both NV4_COLS (into out) and NV4_ROWS
 *                      (into out_rows) from one read of x, with one tensor scale
 *                      (SCALE_TENSOR only, K % 64 == 0).  Used for an upstream
 *                      gradient, which feeds a data gradient (along its rows) and
 *                      a weight gradient (along its tokens).
 *                    NV4_COLS_BATCHED: x is nseg equal matrices of rows/nseg rows
 *                      (rows/nseg % 16 == 0); out is [nseg*K][rows/nseg], matrix s
 *                      transposed into out rows [s*K, (s+1)*K).  Used for the
 *                      transposed expert weights of the data gradients.
 *   scale_mode, nseg NV4_SCALE_TENSOR (nseg ignored unless a segmented layout),
 *                    NV4_SCALE_SEGMENT (one G per segment; ROWS/COLS_BATCHED use
 *                    equal segments of rows/nseg rows when seg_offsets is NULL),
 *                    NV4_SCALE_ROW (ROWS layout only: one G per row, computed in
 *                    the same single pass), NV4_SCALE_SEGMENT_HALVES
 *                    (NV4_COLS_BATCHED only, rows/nseg % 32 == 0: group 2s is the
 *                    first half of matrix s's rows, 2s+1 the second half; the output
 *                    row of the transpose then has K/2-column halves with a G each).
 *                    ngroups = 1, nseg, rows or 2*nseg.
 *   seg_offsets      device int32 [nseg+1], non-decreasing, seg_offsets[nseg] == rows;
 *                    required for NV4_COLS, optional for SCALE_SEGMENT with ROWS.
 *   seg_padded_offsets device int32 [nseg+1], required for NV4_COLS: the 16-padded
 *                    prefix sums (as produced by moe_permute's padded_offsets).
 *   amax_in          device FP32 [ngroups] or NULL.  When given, the amax pass is
 *                    skipped and these values are used as A (one pass over x).
 *   amax_out         device FP32 [ngroups] or NULL: receives the A that was used.
 *   out              host pointer to a descriptor whose device buffers the caller
 *                    allocated: codes, scales, tscale (ngroups floats) and the
 *                    expected output shape in rows/K.  The library sets
 *                    out->scale_mode and out->nseg.
 *   out_rows         NV4_ROWS_AND_COLS only (NULL otherwise): descriptor of the
 *                    row-direction output [rows][K], as `out` for NV4_ROWS.
 *   ws, ws_bytes     device workspace of at least nvfp4_quantize_workspace().
 * Errors: EINVAL (NULL pointer, bad sizes, out shape mismatch), EALIGN (K % 16,
 * ldx % 8 for BF16 / % 4 for FP32, x not 16-byte aligned), EUNSUPPORTED
 * (SCALE_ROW with a COLS layout, row_index with NV4_COLS_BATCHED, ROWS_AND_COLS
 * without SCALE_TENSOR), EWORKSPACE, EHIP.
 */
size_t nvfp4_quantize_workspace(int64_t rows, int64_t K, int layout, int scale_mode, int nseg);
nv4_status nvfp4_quantize(const void *x, nv4_dtype xtype, int64_t rows, int64_t K, int64_t ldx,
                          const int32_t *row_index, int layout, int scale_mode, int nseg,
                          const int32_t *seg_offsets, const int32_t *seg_padded_offsets,
                          const float *amax_in, float *amax_out, nv4_tensor *out, nv4_tensor *out_rows,
                          void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * nvfp4_quantize_sr -- nvfp4_quantize with stochastic rounding of the elements
 * (every argument as there, plus the seed).  [4BL] "Why is the NVFP4 pretraining
 * recipe not sufficient for RL?": the pretraining recipe rounds gradients
 * stochastically so that their quantisation is unbiased.
 *
 * The block scales are the round-to-nearest ones.  Each element v = fp32(x * inv)
 * rounds |v| up to its upper E2M1 neighbour exactly when u < (|v| - lo) / (hi - lo)
 * (|v| >= 6 saturates to 6), with u = (bits >> 8) * 2^-24 and bits a 32-bit word of
 * Philox4x64-10 (Salmon et al., SC 2011): counter (pos >> 3, out_row, stream, 0),
 * key (seed, 0), word (pos >> 1) & 3, its high half for odd pos.  pos and out_row
 * are the element's position and row in its output tensor (for NV4_COLS the padded
 * position, for NV4_COLS_BATCHED the stacked output row); stream is 0 for the
 * NV4_ROWS output (and out_rows of NV4_ROWS_AND_COLS) and 1 for column outputs.
 * Results depend only on the data, the seed and these positions: deterministic
 * and independent of launch geometry.
 */
nv4_status nvfp4_quantize_sr(const void *x, nv4_dtype xtype, int64_t rows, int64_t K, int64_t ldx,
                             const int32_t *row_index, int layout, int scale_mode, int nseg,
                             const int32_t *seg_offsets, const int32_t *seg_padded_offsets,
                             const float *amax_in, float *amax_out, nv4_tensor *out, nv4_tensor *out_rows,
                             void *ws, size_t ws_bytes, int32_t *dev_status, uint64_t seed, void *stream);

/*
 * nv4_amax -- *amax = max_i |x[i]| over n FP32 values (0 when n == 0).  [4BL] "Why is
 * the NVFP4 pretraining recipe not sufficient for RL?": with per-token scales the
 * quantiser records each row's amax (amax_out of nvfp4_quantize with NV4_SCALE_ROW);
 * their maximum is the tensor amax, so a per-tensor quantisation of the same tensor
 * (the token-direction operand of a weight gradient) takes it through amax_in without
 * another pass over the tensor.
 *   x      device FP32 [n];  amax  device FP32 [1], overwritten;
 *   dev_status  optional device word: NV4_DS_NONFINITE for a NaN or infinity.
 * Errors: EINVAL (n < 0, NULL pointers), EHIP.
 */
nv4_status nv4_amax(const float *x, int64_t n, float *amax, int32_t *dev_status, void *stream);

/*
 * moe_permute -- route tokens to experts and permute them by expert.
 * [LBP] "What W4A4 GEMM Actually Changes" (expert routing concentrates
 * activations); [MTE] "Background: Same Weights Did Not Guarantee Same Policy"
 * (grouped GEMMs over experts).  Router: top-k of the logits (larger first, ties
 * to the lower expert id); weight = softmax over all E logits at the chosen id
 * (divided by the k weights' sum with NV4_RENORM).  Permutation: stable counting
 * sort of the T*k assignments by expert (rows of one expert in increasing token
 * order), computed without atomics-order dependence.
 *
 *   logits           FP32 [T][E] or NULL; NULL means topk_ids (and topk_w) are
 *                    inputs and only the permutation is computed.
 *   T, E, k, flags   tokens, experts (1..1024), experts per token (1..min(E, 32)).
 *   topk_ids, topk_w int32 / FP32 [T][k]: outputs (or inputs when logits NULL;
 *                    topk_w may then be NULL).
 *   expert_offsets   int32 [E+1]: exclusive prefix sum of per-expert counts.
 *   padded_offsets   int32 [E+1] or NULL: same with each count rounded up to 16.
 *   row_token        int32 [T*k]: token of permuted row r.
 *   token_row        int32 [T][k]: permuted row of assignment (t, j).
 *   gather_src, gather_dst  optional (both or neither): NVFP4 tensors [T][K] and
 *                    [T*k][K]; dst row r = src row row_token[r] (codes and scales;
 *                    the tensor scale is per tensor and is not copied).
 *   ws, ws_bytes     device workspace of at least moe_permute_workspace().
 * Errors: EINVAL, EUNSUPPORTED (E > 1024, k > 32), EWORKSPACE, EHIP.
 */
size_t moe_permute_workspace(int64_t T, int E, int k);
nv4_status moe_permute(const float *logits, int64_t T, int E, int k, int flags,
                       int32_t *topk_ids, float *topk_w,
                       int32_t *expert_offsets, int32_t *padded_offsets,
                       int32_t *row_token, int32_t *token_row,
                       const nv4_tensor *gather_src, nv4_tensor *gather_dst,
                       void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace, the same results bit for
 * bit.  Its workspace is a static device array of moe_permute_noalloc_max_workspace()
 * bytes (16 MiB) per GPU, held from the library's first use on that GPU until the
 * process ends; the call allocates nothing.  Every call on one GPU shares that
 * array, so calls that may overlap on one GPU (different streams without ordering)
 * race and give unspecified results; calls on one stream are safe.  Nothing in the
 * array needs clearing: every call writes each word it later reads.
 * Errors: as moe_permute; NV4_EWORKSPACE (before anything is enqueued) when
 * moe_permute_workspace(T, E, k) exceeds the static size -- T * k up to about
 * 3.7 million assignments at E = 128.
 */
size_t moe_permute_noalloc_max_workspace(void);
nv4_status moe_permute_noalloc(const float *logits, int64_t T, int E, int k, int flags,
                               int32_t *topk_ids, float *topk_w,
                               int32_t *expert_offsets, int32_t *padded_offsets,
                               int32_t *row_token, int32_t *token_row,
                               const nv4_tensor *gather_src, nv4_tensor *gather_dst,
                               int32_t *dev_status, void *stream);

/*
 * nvfp4_grouped_gemm -- one grouped GEMM over experts, C = A_hat . B_hat^T per
 * expert, both operands NVFP4 (W4A4).  [LBP] "What W4A4 GEMM Actually Changes"
 * (both operands 4-bit, the GEMM runs on the 4-bit data); [MTE] "Development:
 * Aligning Numerics, Then Making NVFP4 Fast" (grouped GEMMs); [4BL] "Improving
 * Gradient Stability" (the product consumes DQ(Q(.)) of the operands).
 *
 * NV4_GROUP_M (forward and data gradients):
 *   A          [M_cap][K] rows grouped by expert: rows [offsets[e], offsets[e+1]).
 *              A->tscale per tensor or per row.  With a_rows != NULL, GEMM row r
 *              reads A row a_rows[r] (the permutation gather fused into the load;
 *              A then holds the un-permuted rows).
 *   B          [E*Nb][K]; expert e's matrix is rows [e*Nb, (e+1)*Nb);
 *              Nb = N (EPI_NONE) or 2N (EPI_SWIGLU: rows [gate_e (N); up_e (N)]).
 *              B->tscale: per tensor (SCALE_TENSOR); per expert (SCALE_SEGMENT,
 *              nseg == E); per expert and projection (SCALE_SEGMENT, nseg == 2E,
 *              EPI_SWIGLU only: gate_e has G[2e], up_e G[2e+1]); or per expert and
 *              K half (SCALE_SEGMENT_HALVES, nseg == E, EPI_NONE, (K/2) % 128 == 0,
 *              A scaled per tensor: products over K [0, K/2) take G[2e], over
 *              [K/2, K) G[2e+1]; the accumulator is rescaled once by
 *              fp32(G[2e] / G[2e+1]) at K/2, a single extra rounding).
 *   C          [M_cap][ldc] of ctype; rows [0, offsets[E]) are written.
 *   EPI_SWIGLU C = silu(gate) * up with silu(g) = g / (1 + exp(-g)), computed in
 *              FP32 after the tensor scales; amax_out (device FP32 [1], may be
 *              NULL) is raised with atomic max to max|C| of the stored values
 *              (the caller zero-fills it first), ready to feed nvfp4_quantize's
 *              amax_in.
 * NV4_GROUP_K (weight gradients):
 *   A [N][Kcap], B [M][Kcap] with expert e's contraction range
 *   [offsets[e], offsets[e+1]) (16-aligned, e.g. moe_permute's padded_offsets);
 *   C [E][N][ldc] (ldc >= M) gets A_e . B_e^T; an empty range gives zeros.
 *   Tensor scales per tensor.
 *   offsets    device int32 [E+1].
 * ws, ws_bytes   device workspace of nvfp4_grouped_gemm_workspace(A, B, group_mode) bytes
 *              (256-byte aligned; NULL or 0 is allowed when that query returns 0, and for
 *              GROUP_K with K % 64 == 0, where it only enables the tile counter below):
 *              - GROUP_K: workgroups take tiles from a counter in the first word of the
 *                workspace, the largest experts' first, which balances skewed expert
 *                sizes; without it every workgroup walks a fixed share of the tiles.
 *                Every tile is computed whole by one workgroup either way, so the output
 *                is bitwise the same.
 *              - K % 64 != 0 (either group mode): both operands are first copied into
 *                the workspace with K zero-padded to the next multiple of 64 (the extra
 *                blocks get scale 0 and add exact zeros to the FP32 sums), then the
 *                kernel runs on the copies.
 *              Calls that share a workspace must not overlap.
 * K (A->K == B->K) must be a positive multiple of 16 ([4BL] "Baseline": blocks of 16);
 * GROUP_K ranges must be 16-aligned.
 * B->f16 (decoded weights): with GROUP_M, a per-tensor A scale and K % 64 == 0 the
 * kernel reads B's elements from B->f16 instead of decoding codes and scales (the
 * same exact FP16 values; B->tscale still applies, per tensor, expert, projection or
 * K half as above).  The products are the same; only the grouping of K inside the
 * FP32 accumulation differs (stages of 64 instead of 128), so the two results agree
 * to FP32 rounding.  Otherwise B->f16 is ignored.
 * Errors: EINVAL, EALIGN (K not a positive multiple of 16, A->K != B->K, misaligned
 * codes), EUNSUPPORTED (SWIGLU with GROUP_K, row scales with GROUP_K, a B scale
 * grouping other than those above), EWORKSPACE (K % 64 != 0 without the workspace),
 * EHIP.
 */
size_t nvfp4_grouped_gemm_workspace(const nv4_tensor *A, const nv4_tensor *B, int group_mode);
nv4_status nvfp4_grouped_gemm(const nv4_tensor *A, const nv4_tensor *B, const int32_t *offsets, int E,
                              int64_t M_cap, int64_t N, const int32_t *a_rows,
                              int group_mode, int epilogue,
                              void *C, nv4_dtype ctype, int64_t ldc, float *amax_out,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * nvfp4_decode_f16 -- the exact FP16 values of an NVFP4 tensor without its decode
 * scale: out[r][k] = e2m1(code) * e4m3(block scale), which has at most 6
 * significant bits and lies in [2^-10, 2688], so FP16 holds it exactly.  [4BL]
 * "Improving Gradient Stability": a GEMM consumes the dequantised operand; the
 * expert weights change once per optimizer step, so their decoded values can be
 * kept (nv4_tensor.f16) instead of decoded inside every grouped GEMM.
 *   q      NVFP4 tensor [q->rows][q->K], K % 16 == 0 (any scale grouping: tscale is
 *          not read).
 *   out    device FP16 [q->rows][ldo], ldo >= K, ldo % 8 == 0, 16-byte aligned.
 * Errors: EINVAL (NULL pointers, bad sizes), EALIGN (K % 16, ldo % 8, misaligned
 * pointers), EHIP.
 */
nv4_status nvfp4_decode_f16(const nv4_tensor *q, void *out, int64_t ldo, void *stream);

/*
 * nv4_to_bf16 -- BF16 operands for the BF16 and dequantized backward.
 * [4BL] "Improving Gradient Stability": the dequantized backward runs the
 * backward GEMMs on BF16 operands holding DQ(Q(.)) of the exact NVFP4 tensors
 * the forward used, for weights and activations; [4BL] "Why is the NVFP4
 * pretraining recipe not sufficient for RL?": the conservative baseline keeps the
 * backward in BF16 on the unquantised tensors.
 *
 * The source is either x (BF16 [x_rows][ldx], ldx >= K, ldx % 8 == 0, 16-byte
 * aligned) or q (an NVFP4 tensor [q->rows][K] with its tscale grouping: per
 * tensor, per equal segment of q->rows/q->nseg rows, or per row; not
 * SCALE_SEGMENT_HALVES); exactly one is
 * non-NULL (with rows == 0 both may be NULL: nothing is read, and out may be NULL
 * when it has no elements).  The BF16 value of an NVFP4 element is
 *   bf16_rne(fp32(e2m1(q) * sf * G))
 * where e2m1(q) * sf is exact and the product with G is one FP32 rounding.
 *   rows, K          logical rows (after the gather) and columns; K % 16 == 0.
 *   row_index        device int32 [rows] or NULL (NV4_ROWS, NV4_COLS): logical row
 *                    r is source row row_index[r] (an index outside the source is
 *                    clamped into it).
 *   layout           NV4_ROWS: out [rows][K] (out_rows == rows, out_cols == K).
 *                    NV4_COLS: out [K][out_cols]; logical row r of segment s
 *                      (rows [seg_offsets[s], seg_offsets[s+1])) lands in column
 *                      seg_padded_offsets[s] + r - seg_offsets[s]; the rest of each
 *                      segment's 16-padded range is written as zeros; columns at
 *                      and after seg_padded_offsets[nseg] are not written.
 *                      out_cols >= rows + 15 * nseg, % 8.  The column operands of
 *                      the weight-gradient GEMMs (bf16_grouped_gemm, NV4_GROUP_K).
 *                    NV4_COLS_BATCHED: the source is nseg equal matrices of
 *                      m = rows/nseg rows (m % 16 == 0); out [nseg*K][m] holds each
 *                      transposed.  The transposed expert weights of the data
 *                      gradients.
 *   out              device BF16 [out_rows][out_cols], 16-byte aligned.
 * Errors: EINVAL (both or neither source, bad sizes, output shape mismatch),
 * EALIGN (K % 16, ldx, misaligned pointers), EUNSUPPORTED (row_index with
 * NV4_COLS_BATCHED), EHIP.
 */
nv4_status nv4_to_bf16(const void *x, int64_t x_rows, int64_t ldx, const nv4_tensor *q, int64_t rows, int64_t K,
                       const int32_t *row_index, int layout, int nseg, const int32_t *seg_offsets,
                       const int32_t *seg_padded_offsets, void *out, int64_t out_rows, int64_t out_cols,
                       void *stream);

/*
 * bf16_grouped_gemm -- nvfp4_grouped_gemm's grouping, row gather and epilogues on
 * BF16 operands (FP32 accumulation, no tensor scales).  [4BL] "Improving Gradient
 * Stability" (the backward GEMMs on BF16 operands), "Why is the NVFP4 pretraining
 * recipe not sufficient for RL?" (the BF16 baseline); [LBP] "Throughput Gains and
 * the Conditions That Produce Them" (the BF16 layer as the comparison point).
 *
 *   A [a_rows][K], B [b_rows][K]   BF16, row-major with row stride K, 16-byte
 *                    aligned, each below 4 GiB.
 *   K                a positive multiple of 32 (the kernel stages 32 elements).
 * NV4_GROUP_M: b_rows == E*N (EPI_NONE) or E*2N (EPI_SWIGLU: rows [gate_e; up_e]);
 *   expert e's rows [offsets[e], offsets[e+1]) of A (or A rows a_rows[r], the
 *   fused gather) times B_e^T into C [M_cap][ldc]; amax_out as in
 *   nvfp4_grouped_gemm.
 * NV4_GROUP_K: A [N][Kcap], B [M][Kcap] with Kcap = K; expert e contracts over
 *   [offsets[e], offsets[e+1]) (16-aligned, e.g. padded offsets, the layout
 *   nv4_to_bf16 NV4_COLS writes); C [E][N][ldc] gets A_e . B_e^T, an empty range
 *   zeros.  N is taken from a_rows.
 *   ws, ws_bytes   as for nvfp4_grouped_gemm (the GROUP_K tile schedule).
 * Errors: EINVAL, EALIGN (K not a positive multiple of 32, misaligned operands),
 * EUNSUPPORTED (SWIGLU or a row index with GROUP_K), EHIP.
 */
nv4_status bf16_grouped_gemm(const void *A, int64_t a_rows_n, const void *B, int64_t b_rows_n, int64_t K,
                             const int32_t *offsets, int E, int64_t M_cap, int64_t N, const int32_t *a_rows,
                             int group_mode, int epilogue, void *C, nv4_dtype ctype, int64_t ldc,
                             float *amax_out, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_combine -- weighted sum of each token's k expert outputs, back in token
 * order: out[t] = sum_{j=0..k-1} w[t][j] * Y[token_row[t][j]], j ascending, FP32.
 * [LBP] "What W4A4 GEMM Actually Changes" (expert routing); the weights are the
 * router weights from moe_permute.
 *
 *   Y, ytype, ldy    expert output rows [T*k][ldy] (BF16 or FP32).
 *   token_row        int32 [T][k] from moe_permute.
 *   topk_w           FP32 [T][k].
 *   out, otype       [T][H] (row stride H), BF16 (round to nearest even) or FP32.
 * Errors: EINVAL, EALIGN (H % 4, ldy % 4), EHIP.
 */
nv4_status moe_combine(const void *Y, nv4_dtype ytype, int64_t ldy, const int32_t *token_row,
                       const float *topk_w, int64_t T, int k, int64_t H,
                       void *out, nv4_dtype otype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NV4MOE_H */
