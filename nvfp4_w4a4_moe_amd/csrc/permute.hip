// Routing and permutation by expert for gfx950.
//
// "Low-Bit Precision Training ...", section "What W4A4 GEMM Actually Changes":
// expert routing concentrates activations on the chosen experts; "miniTE ...",
// section "Background: Same Weights Did Not Guarantee Same Policy": the expert
// work runs as grouped GEMMs, which need the routed rows of each expert to be
// contiguous.
//
// Router: top-k of the logits, larger first, ties to the lower expert id; the
// weight of a chosen expert is its softmax probability over all E logits (FP32,
// fixed-order reductions).  Permutation: a stable counting sort of the flat
// assignments f = t*k + j by expert, so the rows of one expert are in increasing
// (t, j) order.  The rank of every assignment is computed without atomics:
//   1. one wave per chunk of kPermuteChunk assignments ranks each assignment
//      among equal experts inside the chunk (wave ballots over the id bits,
//      chunk-local counters in LDS), and writes the chunk's expert histogram;
//   2. one wave per expert turns the histograms into per-(chunk, expert) bases,
//      one workgroup the expert totals into the expert offsets (exclusive prefix sums);
//   3. every assignment's row is base + local rank; a scatter writes the maps.
// The result is one exactly defined permutation, identical on every run.
#include <algorithm>
#include <mutex>

#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {
namespace {

constexpr int kMaxE = 1024;

// Wave-wide reductions over 64 lanes without LDS: DPP within rows of 16 lanes (the
// pairs (i, i^1), (i, i^2), then the half-row and row mirrors), then the gfx950
// row swaps across 16 and 32 lanes.  Every lane ends with the result.
template <int LANES = 64, class F>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, F op) {
  static_assert(LANES == 32 || LANES == 64, "reductions over 32-lane halves or the wave");
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(s16[0], s16[1]);
  if (LANES == 32) return v;  // each 32-lane half holds its own result
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(s32[0], s32[1]);
}
template <int LANES = 64>
__device__ __forceinline__ float wave_max_dpp(float v) {
  return __uint_as_float(wave_reduce_u32<LANES>(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  }));
}
template <int LANES = 64>
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return __uint_as_float(wave_reduce_u32<LANES>(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
  }));
}
template <int LANES = 64>
__device__ __forceinline__ int wave_min_dpp(int v) {
  return (int)wave_reduce_u32<LANES>((uint32_t)v, [](uint32_t x, uint32_t y) { return (uint32_t)min((int)x, (int)y); });
}

// LPT lanes per token (64: one token per wave; 32: two, one per half-wave), NPL
// logits per lane (expert e = lane-in-token + LPT * i): softmax statistics, then k
// rounds of an argmax over the token's lanes.  Each round: every lane's best untaken
// candidate (larger logit first, then lower id), the token's maximum value, and among
// the lanes holding it the lowest id (a ballot; a second reduction only when several
// lanes tie).  Lane j of the token keeps round j's id and logit; the k softmax
// weights are formed after the rounds, one per lane.  The kernel is bound by its VALU
// work: an exp and a division in every round cost a third of it (78 -> 60 us on the
// learner batch), and two tokens per wave share every reduction's instructions.
template <int NPL, int LPT>
__global__ __launch_bounds__(256) void k_topk(PermuteArgs a) {
  constexpr int TPW = kWave / LPT;  // tokens per wave
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPT, ll = lane % LPT;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  if (t0 >= a.T) return;  // uniform over the wave
  const int64_t t = t0 + sub;
  const bool valid = t < a.T;  // the second token of the last wave may not exist
  const int E = a.E;
  const float *lg = a.logits + t * E;
  float lv[NPL];
  float mx = -INFINITY;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = ll + LPT * i;
    lv[i] = -INFINITY;
    if (valid && e < E) {
      lv[i] = lg[e];
      nan |= lv[i] != lv[i];
      mx = fmaxf(mx, lv[i]);
    }
  }
  mx = wave_max_dpp<LPT>(mx);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = ll + LPT * i;
    if (valid && e < E) s += expf(lv[i] - mx);
  }
  s = wave_sum_dpp<LPT>(s);
  uint32_t taken = 0;
  int my_id = 0;
  float my_v = -INFINITY;
  for (int j = 0; j < a.k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = ll + LPT * i;
      // ids of one lane increase with i, so the first of equal values has the lowest id
      if (e < E && !((taken >> i) & 1u) && (lv[i] > bv || (bi == 0x7FFFFFFF && lv[i] == bv))) { bv = lv[i]; bi = e; }
    }
    const float vmax = wave_max_dpp<LPT>(bv);
    const uint64_t cand = __ballot(bi != 0x7FFFFFFF && bv == vmax);
    int wid;
    if (LPT == 64) {
      if (cand == 0) {
        wid = 0x7FFFFFFF;  // every remaining logit is NaN
      } else if ((cand & (cand - 1)) == 0) {
        wid = __builtin_amdgcn_readlane(bi, (int)__builtin_ctzll(cand));
      } else {
        wid = wave_min_dpp(((cand >> lane) & 1) ? bi : 0x7FFFFFFF);
      }
    } else {
      // the two halves' candidate lanes: one each (the usual case) is read directly
      const uint32_t c0 = (uint32_t)cand, c1 = (uint32_t)(cand >> 32);
      if ((c0 & (c0 - 1)) == 0 && (c1 & (c1 - 1)) == 0) {
        const int w0 = c0 ? __builtin_amdgcn_readlane(bi, (int)__builtin_ctz(c0)) : 0x7FFFFFFF;
        const int w1 = c1 ? __builtin_amdgcn_readlane(bi, 32 + (int)__builtin_ctz(c1)) : 0x7FFFFFFF;
        wid = sub ? w1 : w0;
      } else {
        wid = wave_min_dpp<LPT>(((cand >> lane) & 1) ? bi : 0x7FFFFFFF);
      }
    }
    if (wid < E && (wid % LPT) == ll) taken |= 1u << (wid / LPT);
    if (ll == j) { my_id = wid; my_v = vmax; }
  }
  float my_w = 0.0f;
  if (ll < a.k) my_w = expf(my_v - mx) / s;
  if (a.flags & NV4_RENORM) my_w = my_w / wave_sum_dpp<LPT>(my_w);  // lanes >= k hold 0
  if (valid && ll < a.k) {
    a.topk_ids[t * a.k + ll] = my_id;
    a.topk_w[t * a.k + ll] = my_w;
  }
  // any lane's NaN (each lane held only its own experts' logits)
  if (__ballot(nan) != 0 && lane == 0 && a.dev_status) atomicOr(a.dev_status, kDsNanLogit);
}

// one wave per chunk: rank of each assignment among the chunk's assignments to
// the same expert (in flat order), and the chunk's expert histogram
__global__ __launch_bounds__(64) void k_rank(PermuteArgs a, int nbits) {
  __shared__ int cnt[kMaxE];
  const int lane = threadIdx.x;
  const int E = a.E;
  for (int e = lane; e < E; e += kWave) cnt[e] = 0;
  __syncthreads();
  const int64_t R = a.T * a.k;
  const int64_t f0 = (int64_t)blockIdx.x * kPermuteChunk;
  const int64_t f1 = std::min<int64_t>(f0 + kPermuteChunk, R);
  bool badid = false;
  for (int64_t fb = f0; fb < f1; fb += kWave) {
    const int64_t f = fb + lane;
    const bool act = f < f1;
    int e = act ? a.topk_ids[f] : 0;
    if (e < 0 || e >= E) { badid |= act; e = 0; }
    uint64_t match = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      match &= bit ? bal : ~bal;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(match & below);
    const int base = cnt[e];
    __syncthreads();
    if (act) {
      a.local_rank[f] = base + rank;
      if ((match >> lane) == 1ull) cnt[e] = base + __popcll(match);  // highest lane of its group
    }
    __syncthreads();
  }
  for (int e = lane; e < E; e += kWave) a.chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
  if (badid && a.dev_status) atomicOr(a.dev_status, kDsBadExpert);
}

// Chunk histograms -> per-(chunk, expert) bases and expert offsets, in two kernels:
//   k_scan_chunks: one wave per expert turns its column of chunk counts into an
//     exclusive prefix over the chunks (in place) and leaves the expert's total in
//     expert_offsets[e];
//   k_scan_experts: one workgroup turns the totals into the exclusive offsets (and
//     the 16-padded ones).
// A row is then chunk base + expert offset + local rank (k_scatter).
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(v, o, kWave);
    if (lane >= o) v += x;
  }
  return v;
}

__global__ __launch_bounds__(64) void k_scan_chunks(PermuteArgs a, int nchunks) {
  const int E = a.E, e = blockIdx.x, lane = threadIdx.x;
  int run = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    int *p = a.chunk_counts + (int64_t)c * E + e;
    const int v = c < nchunks ? *p : 0;
    const int incl = wave_incl_scan(v, lane);
    if (c < nchunks) *p = run + incl - v;
    run += __shfl(incl, 63, kWave);
  }
  if (lane == 0) a.expert_offsets[e] = run;
}

__global__ __launch_bounds__(1024) void k_scan_experts(PermuteArgs a, int have_counts) {
  __shared__ int sc[kMaxE];
  __shared__ int sp[kMaxE];
  const int E = a.E;
  const int e = threadIdx.x;
  const int run = (e < E && have_counts) ? a.expert_offsets[e] : 0;
  const int prun = ((run + 15) >> 4) << 4;
  sc[e] = run;
  sp[e] = prun;
  __syncthreads();
  for (int o = 1; o < kMaxE; o <<= 1) {
    const int x = (e >= o) ? sc[e - o] : 0;
    const int y = (e >= o) ? sp[e - o] : 0;
    __syncthreads();
    sc[e] += x;
    sp[e] += y;
    __syncthreads();
  }
  if (e < E) {
    a.expert_offsets[e] = sc[e] - run;
    if (a.padded_offsets) a.padded_offsets[e] = sp[e] - prun;
    if (e == E - 1) {
      a.expert_offsets[E] = sc[e];
      if (a.padded_offsets) a.padded_offsets[E] = sp[e];
    }
  }
}

__global__ __launch_bounds__(256) void k_scatter(PermuteArgs a) {
  const int64_t R = a.T * a.k;
  const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= R) return;
  int e = a.topk_ids[f];
  if (e < 0 || e >= a.E) e = 0;
  const int64_t c = f / kPermuteChunk;
  const int r = a.chunk_counts[c * a.E + e] + a.expert_offsets[e] + a.local_rank[f];
  a.row_token[r] = (int)(f / a.k);
  a.token_row[f] = r;
}

// one wave per permuted row: copy the packed codes and scale bytes of its token
__global__ __launch_bounds__(256) void k_gather(PermuteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t R = a.T * a.k;
  if (r >= R) return;
  const int64_t t = a.row_token[r];
  const int64_t cb = a.gather_K >> 1, sb = a.gather_K >> 4;
  if ((cb & 15) == 0) {
    const uint4 *s = reinterpret_cast<const uint4 *>(a.src_codes + t * cb);
    uint4 *d = reinterpret_cast<uint4 *>(a.dst_codes + r * cb);
    for (int64_t i = lane; i < (cb >> 4); i += kWave) d[i] = s[i];
  } else {
    for (int64_t i = lane; i < cb; i += kWave) a.dst_codes[r * cb + i] = a.src_codes[t * cb + i];
  }
  if ((sb & 3) == 0) {
    const uint32_t *s = reinterpret_cast<const uint32_t *>(a.src_scales + t * sb);
    uint32_t *d = reinterpret_cast<uint32_t *>(a.dst_scales + r * sb);
    for (int64_t i = lane; i < (sb >> 2); i += kWave) d[i] = s[i];
  } else {
    for (int64_t i = lane; i < sb; i += kWave) a.dst_scales[r * sb + i] = a.src_scales[t * sb + i];
  }
}

}  // namespace

size_t permute_workspace_bytes(int64_t T, int E, int k) {
  const int64_t R = T * k;
  const int64_t nchunks = std::max<int64_t>(1, (R + kPermuteChunk - 1) / kPermuteChunk);
  const size_t a = (size_t)nchunks * E * sizeof(int32_t);
  const size_t b = (size_t)std::max<int64_t>(R, 1) * sizeof(int32_t);
  return ((a + 255) & ~(size_t)255) + ((b + 255) & ~(size_t)255);
}

// Workspace of moe_permute_noalloc: one array per device, for callers that cannot
// allocate.  Host code never passes `scratch` itself to a kernel (on the host it
// is a stand-in symbol, not a device address): the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) uint8_t scratch[kPermuteStaticBytes];

hipError_t permute_static_workspace(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_permute(const PermuteArgs &a, hipStream_t stream) {
  const int64_t R = a.T * a.k;
  if (R == 0) {
    // no assignment: all offsets are zero
    k_scan_experts<<<1, 1024, 0, stream>>>(a, 0);
    return hipGetLastError();
  }
  const int nchunks = (int)((R + kPermuteChunk - 1) / kPermuteChunk);
  int nbits = 0;
  while ((1 << nbits) < a.E) ++nbits;
  if (a.logits) {
    // four waves per workgroup; two tokens per wave up to 128 experts (k <= 32 <= LPT)
    const unsigned g1 = (unsigned)((a.T + 3) / 4), g2 = (unsigned)((a.T + 7) / 8);
    if (a.E <= 64) k_topk<2, 32><<<g2, 256, 0, stream>>>(a);
    else if (a.E <= 128) k_topk<4, 32><<<g2, 256, 0, stream>>>(a);
    else if (a.E <= 256) k_topk<4, 64><<<g1, 256, 0, stream>>>(a);
    else if (a.E <= 512) k_topk<8, 64><<<g1, 256, 0, stream>>>(a);
    else k_topk<16, 64><<<g1, 256, 0, stream>>>(a);
  }
  k_rank<<<nchunks, 64, 0, stream>>>(a, nbits);
  k_scan_chunks<<<a.E, 64, 0, stream>>>(a, nchunks);
  k_scan_experts<<<1, 1024, 0, stream>>>(a, 1);
  k_scatter<<<(unsigned)((R + 255) / 256), 256, 0, stream>>>(a);
  if (a.gather_K > 0) k_gather<<<(unsigned)((R + 3) / 4), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace nv4
