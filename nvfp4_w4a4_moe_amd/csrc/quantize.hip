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
//
// Stochastic rounding (the pretraining recipe's gradient rounding, same section
// "Why is the NVFP4 pretraining recipe not sufficient for RL?"), when asked for:
// the E2M1 step rounds |v| up to its upper grid neighbour exactly when
// u < (|v| - lo) / (hi - lo), u a 24-bit uniform per element from Philox4x64-10
// (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with
// counter (position >> 3, output row, stream, 0) and key (seed, 0); stream 0 for
// row-direction outputs, 1 for column-direction outputs.  Block scales stay
// round-to-nearest.
#include <algorithm>
#include <type_traits>

#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {
namespace {

constexpr int kThreads = 256;
constexpr int kXcdCount = 8;  // MI355X: workgroup i runs on XCD i % 8

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

// element offset of logical row `row` of x (through the optional row gather)
__device__ __forceinline__ int64_t row_off(const QuantArgs &a, int64_t row) {
  return (a.row_index ? (int64_t)a.row_index[row] : row) * a.ldx;
}

__device__ __forceinline__ const float *amax_src(const QuantArgs &a) {
  return a.amax_in ? a.amax_in : a.amax_acc;
}

__global__ void k_fill_zero(float *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Raw 8-element chunk (BF16: one 16-byte load; FP32: two).
template <bool F32>
struct Chunk {
  uint4 w[F32 ? 2 : 1];
};

// 16 bytes by a non-temporal load (the source is streamed once)
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void *p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// NT: non-temporal loads, for sources read once (measured on the learner batch: the X
// quantisation 19 % faster, the rows-and-columns passes 2-6 %); a gathered source
// whose rows repeat keeps ordinary loads, which let the repeats hit in the caches.
template <bool F32, bool NT = true>
__device__ __forceinline__ Chunk<F32> load_chunk(const void *x, int64_t off) {
  Chunk<F32> c;
  if (F32) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(x) + off);
    c.w[0] = NT ? ld16_nt(p) : p[0];
    c.w[F32 ? 1 : 0] = NT ? ld16_nt(p + 1) : p[1];
  } else {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
    c.w[0] = NT ? ld16_nt(p) : *p;
  }
  return c;
}

template <bool F32>
__device__ __forceinline__ void unpack_chunk(const Chunk<F32> &c, float v[8]) {
  if (F32) {
    v[0] = __uint_as_float(c.w[0].x); v[1] = __uint_as_float(c.w[0].y);
    v[2] = __uint_as_float(c.w[0].z); v[3] = __uint_as_float(c.w[0].w);
    v[4] = __uint_as_float(c.w[F32 ? 1 : 0].x); v[5] = __uint_as_float(c.w[F32 ? 1 : 0].y);
    v[6] = __uint_as_float(c.w[F32 ? 1 : 0].z); v[7] = __uint_as_float(c.w[F32 ? 1 : 0].w);
  } else {
    const uint4 u = c.w[0];
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xFFFF0000u);
    v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xFFFF0000u);
  }
}

// Position (row, chunk) of a lane's 8-element chunk in the flat chunk order of a
// row range; stepping by a fixed number of chunks needs no division.
struct Pos {
  int64_t row, ch;
};

__device__ __forceinline__ Pos pos_step(Pos p, int64_t dr, int64_t dc, int64_t kc) {
  p.ch += dc;
  p.row += dr;
  if (p.ch >= kc) { p.ch -= kc; p.row += 1; }
  return p;
}

// Group amax.  Workgroup (p, g) scans the chunks of group g's row range (an
// equal split of the rows, or [seg_offsets[g], seg_offsets[g+1])) in flat order,
// workgroup p taking every P-th run of 256 chunks, eight loads in flight per lane;
// waves reduce in registers and LDS, and one order-independent atomic max per
// workgroup goes to amax_acc[g].  Atomics on one address serialise in L2, so P
// stays near one workgroup per CU in total.
template <bool F32>
__global__ __launch_bounds__(kThreads) void k_amax_rows(QuantArgs a, int P) {
  constexpr int U = 8;
  __shared__ float red[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = blockIdx.x, g = blockIdx.y;
  int64_t r0, r1;
  if (a.scale_mode == NV4_SCALE_TENSOR) { r0 = 0; r1 = a.rows; }
  else if (a.seg_offsets) { r0 = a.seg_offsets[g]; r1 = a.seg_offsets[g + 1]; }
  else { const int64_t len = a.rows / a.ngroups; r0 = (int64_t)g * len; r1 = r0 + len; }  // equal segments
  const int64_t kc = a.K >> 3;
  const int64_t total = (r1 - r0) * kc;
  const int64_t stride = (int64_t)P * kThreads;
  const int64_t dr = stride / kc, dc = stride % kc;
  const int64_t c0 = (int64_t)p * kThreads + wave * 64 + lane;
  Pos pos = {r0 + c0 / kc, c0 % kc};
  float m = 0.0f;
  bool bad = false;
  for (int64_t base = (int64_t)p * kThreads + wave * 64; base < total; base += U * stride) {
    Chunk<F32> c[U];
    bool act[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      act[u] = base + u * stride + lane < total;
      c[u] = load_chunk<F32>(a.x, act[u] ? row_off(a, pos.row) + pos.ch * 8 : 0);
      pos = pos_step(pos, dr, dc, kc);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[8];
      unpack_chunk<F32>(c[u], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float av = act[u] ? fabsf(v[i]) : 0.0f;
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

// fp32(m / 6), correctly rounded.  For m >= 2^-122 the quotient is normal and one
// Newton correction of m * fp32(1/6) with an exact FMA remainder gives the
// correctly rounded quotient (Markstein, "Computation of elementary functions on
// the IBM RISC System/6000 processor", 1990; checked exhaustively over every
// FP32 m >= 2^-122).  Smaller nonzero m (subnormal quotients) take the division.
__device__ __forceinline__ float div6_rn(float m) {
  const float r6 = 0.16666667163372039794921875f;  // fp32(1/6)
  const float q0 = __fmul_rn(m, r6);
  const float rem = __builtin_fmaf(-q0, 6.0f, m);
  float q = __builtin_fmaf(rem, r6, q0);
  if (m < 0x1p-122f) q = __fdiv_rn(m, 6.0f);
  return q;
}

// Philox4x64-10: 10 rounds of two 64x64->128-bit products and a Feistel-like
// mix, the key bumped by the Weyl constants after every round.
struct Rand4 {
  uint64_t w[4];
};
// 128-bit product of x and the constant m from four 32x32+64->64-bit multiply-adds
// (v_mad_u64_u32), each carrying the previous partial sum:
//   t = x0 m0,  u = x0 m1 + t_hi,  w = x1 m0 + u_lo,  hi = x1 m1 + u_hi + w_hi,
//   lo = t_lo | w_lo << 32   (x m = t_lo + w_lo 2^32 + (x1 m1 + u_hi + w_hi) 2^64)
__device__ __forceinline__ void mulhilo64(uint64_t x, uint64_t m, uint64_t &hi, uint64_t &lo) {
  const uint32_t x0 = (uint32_t)x, x1 = (uint32_t)(x >> 32);
  const uint32_t m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
  const uint64_t t = (uint64_t)x0 * m0;
  const uint64_t u = (uint64_t)x0 * m1 + (t >> 32);
  const uint64_t w = (uint64_t)x1 * m0 + (uint32_t)u;
  lo = (uint32_t)t | (w << 32);
  hi = (uint64_t)x1 * m1 + ((u >> 32) + (w >> 32));
}
__device__ __forceinline__ Rand4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
  uint64_t k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(c0, kM0, hi0, lo0);
    mulhilo64(c2, kM1, hi1, lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return Rand4{{c0, c1, c2, c3}};
}

// the 24-bit uniform of element j (0..7) of the 8-element run a Philox block covers
__device__ __forceinline__ uint32_t uniform24(const Rand4 &r, int j) {
  const uint64_t w = r.w[j >> 1];
  return (uint32_t)((j & 1) ? (w >> 32) : (w & 0xFFFFFFFFull)) >> 8;
}

// E2M1 code of v by stochastic rounding with the uniform u24 * 2^-24: |v| saturates
// at 6; between grid neighbours lo <= |v| < hi it rounds up iff u < (|v| - lo) / (hi -
// lo).  |v| - lo is exact (lo = 0 or |v| <= 2 lo) and the gaps are powers of two, so
// the comparison is exact.  The sign comes from v (-0 gives code 8).
__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t u24) {
  const float a = fminf(fabsf(v), 6.0f);
  const uint32_t i = (uint32_t)(a >= 0.5f) + (a >= 1.0f) + (a >= 1.5f) + (a >= 2.0f) + (a >= 3.0f) +
                     (a >= 4.0f) + (a >= 6.0f);
  // grid gap around a: 0.5 below 2, 1 below 4, 2 above; lo = a rounded down to it
  // (exact: the scalings are by powers of two)
  const float gap = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
  const float inv_gap = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
  const float lo = __builtin_floorf(a * inv_gap) * gap;
  const float frac = __fmul_rn(a - lo, inv_gap);
  const float u = (float)u24 * 0x1p-24f;
  const uint32_t up = u < frac ? 1u : 0u;  // frac is 0 at the top of the grid (a = 6)
  return (__float_as_uint(v) >> 31 << 3) | (i + up);
}

// 8 codes (one dword, element 2i in the low nibble of byte i) of the products
// v[i] * inv by stochastic rounding, uniforms from one Philox block
__device__ __forceinline__ uint32_t pack_e2m1_sr8(const float v[8], float inv, const Rand4 &r) {
  uint32_t p = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) p |= e2m1_sr(__fmul_rn(v[j], inv), uniform24(r, j)) << (4 * j);
  return p;
}

// value of lane ^ 1 (quad permutation [1, 0, 3, 2] of the data-parallel primitives)
__device__ __forceinline__ float xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// Quantise one 8-element half-block held by this lane; the partner lane (lane ^ 1)
// holds the other half of the same 16-element block.  With inv_tab, fp32(S / sf)
// is read from a table of the 127 E4M3 values (the same correctly rounded
// quotients).  Returns the packed codes and the block scale byte.  With SR the
// codes round stochastically with the uniforms of Philox block `rnd`.
template <bool SR = false>
__device__ __forceinline__ uint32_t quant_half_block(const float v[8], float S, const float *inv_tab,
                                                     uint32_t &sf_out, bool &bad, const Rand4 *rnd = nullptr) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float av = fabsf(v[i]);
    bad |= !(av <= 3.402823466e38f);
    m = fmaxf(m, av);
  }
  m = fmaxf(m, xor1(m));
  const uint32_t sf = e4m3_from_f32(__fmul_rn(div6_rn(m), S));
  const float inv = inv_tab ? inv_tab[sf] : (sf ? __fdiv_rn(S, e4m3_to_f32(sf)) : 0.0f);
  sf_out = sf;
  if (SR) return pack_e2m1_sr8(v, inv, *rnd);
  uint32_t p = 0;
  p = pack_e2m1_pair<0>(p, __fmul_rn(v[0], inv), __fmul_rn(v[1], inv));
  p = pack_e2m1_pair<1>(p, __fmul_rn(v[2], inv), __fmul_rn(v[3], inv));
  p = pack_e2m1_pair<2>(p, __fmul_rn(v[4], inv), __fmul_rn(v[5], inv));
  p = pack_e2m1_pair<3>(p, __fmul_rn(v[6], inv), __fmul_rn(v[7], inv));
  return p;
}

// Write the decode scales G (and, when the amax came from amax_in, amax_out).
__device__ void write_group_scales(const QuantArgs &a) {
  const float *A = amax_src(a);
  for (int g = threadIdx.x; g < a.ngroups; g += blockDim.x) {
    float S = tensor_encode_scale(A[g]);
    a.tscale[g] = __fdiv_rn(1.0f, S);
    if (a.tscale2) a.tscale2[g] = __fdiv_rn(1.0f, S);
    if (a.amax_in && a.amax_acc) a.amax_acc[g] = a.amax_in[g];
  }
}

// No elements (rows == 0 or K == 0): only the groups' decode scales (and amax_out)
// are written.  The quantisation kernels would otherwise read x at offset 0 for
// their idle lanes, which an empty x does not have.
__global__ void k_group_scales(QuantArgs a) { write_group_scales(a); }

// Row layout, tensor or segment scales: every lane quantises 8 consecutive
// elements per chunk (one 16-byte BF16 load, one 4-byte code store); waves
// stride over the flat (row, chunk) order so that loads and stores are fully
// coalesced.  Each iteration quantises two chunks per lane while the loads of
// the next two are in flight.  The two lanes of a block are always both active
// or both inactive (K % 16 == 0 and runs start at multiples of 64 chunks).
// With one tensor scale, fp32(S / sf) comes from an LDS table.
template <bool F32, bool TENSOR, bool SR>
__global__ __launch_bounds__(kThreads) void k_quant_rows(QuantArgs a) {
  __shared__ float inv_tab[128];
  if (blockIdx.x == 0) write_group_scales(a);
  const float *A = amax_src(a);
  const float S_tensor = TENSOR ? tensor_encode_scale(A[0]) : 1.0f;
  if (TENSOR) {
    if (threadIdx.x < 128) inv_tab[threadIdx.x] = threadIdx.x ? __fdiv_rn(S_tensor, e4m3_to_f32(threadIdx.x)) : 0.0f;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int64_t kc = a.K >> 3;  // 8-element chunks per row (even)
  const int64_t total = a.rows * kc;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t dr = stride / kc, dc = stride % kc;
  const int64_t w0 = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 64;
  uint32_t *codes = reinterpret_cast<uint32_t *>(a.codes);
  const int64_t cstride = a.out_K >> 3, sstride = a.out_K >> 4;
  Pos q[2];
  q[0] = Pos{(w0 + lane) / kc, (w0 + lane) % kc};
  q[1] = pos_step(q[0], dr, dc, kc);
  Chunk<F32> cur[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    cur[u] = load_chunk<F32>(a.x, w0 + u * stride + lane < total ? row_off(a, q[u].row) + q[u].ch * 8 : 0);
  int64_t g_lo = 0, g_hi = 0;  // row range of the group whose scale S holds
  float S = S_tensor;
  bool bad = false;
  for (int64_t base = w0; base < total; base += 2 * stride) {
    Pos nq[2];
    Chunk<F32> nxt[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      nq[u] = pos_step(pos_step(q[u], dr, dc, kc), dr, dc, kc);
      const bool nact = base + (2 + u) * stride + lane < total;
      nxt[u] = load_chunk<F32>(a.x, nact ? row_off(a, nq[u].row) + nq[u].ch * 8 : 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool act = base + u * stride + lane < total;
      float v[8];
      unpack_chunk<F32>(cur[u], v);
      uint32_t sf, p;
      Rand4 rnd;
      if (SR) rnd = philox4x64_10((uint64_t)q[u].ch, (uint64_t)q[u].row, 0, 0, a.sr_seed);
      if (TENSOR) {
        p = quant_half_block<SR>(v, S_tensor, inv_tab, sf, bad, &rnd);
      } else {
        const int64_t row = act ? q[u].row : 0;
        if (row < g_lo || row >= g_hi) {  // entered another group: its row range and scale
          const int g = row_group(a, row);
          if (a.scale_mode == NV4_SCALE_ROW) { g_lo = row; g_hi = row + 1; }
          else if (a.seg_offsets) { g_lo = a.seg_offsets[g]; g_hi = a.seg_offsets[g + 1]; }
          else { g_lo = (int64_t)g * (a.rows / a.nseg); g_hi = g_lo + a.rows / a.nseg; }
          S = tensor_encode_scale(A[g]);
        }
        p = quant_half_block<SR>(v, S, nullptr, sf, bad, &rnd);
      }
      if (act) {
        codes[q[u].row * cstride + q[u].ch] = p;
        if ((q[u].ch & 1) == 0) a.scales[q[u].row * sstride + (q[u].ch >> 1)] = (uint8_t)sf;
      }
      q[u] = nq[u];
      cur[u] = nxt[u];
    }
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

// Row layout with one scale per row (the per-token variant): one wave per row, amax
// and quantisation fused.  Rows of up to NC * 512 elements stay in registers between
// the row-amax reduction and the quantisation (one read of x), and the next row's
// loads are in flight while the current row is quantised.  NC = 0: longer rows, read
// twice (the second time from cache).
template <bool F32, bool SR, int NC>
__global__ __launch_bounds__(kThreads) void k_quant_rows_per_row(QuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  bool bad = false;
  auto store = [&](int64_t row, int64_t k, uint32_t p, uint32_t sf) {
    if (k < a.K) {
      reinterpret_cast<uint32_t *>(a.codes)[row * (a.out_K >> 3) + (k >> 3)] = p;
      if (((k >> 3) & 1) == 0) a.scales[row * (a.out_K >> 4) + (k >> 4)] = (uint8_t)sf;
    }
  };
  auto finish_scale = [&](int64_t row, float A) {
    const float S = tensor_encode_scale(A);
    if (lane == 0) {
      a.tscale[row] = __fdiv_rn(1.0f, S);
      if (a.amax_acc) a.amax_acc[row] = A;
    }
    return S;
  };
  if constexpr (NC > 0) {
    const int nc = (int)((a.K + 511) >> 9);  // 512-element rounds of the wave per row (<= NC)
    auto load_row = [&](int64_t row, Chunk<F32> (&c)[NC]) {
      const int64_t base = row_off(a, row < a.rows ? row : 0);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int64_t k = (int64_t)i * 512 + lane * 8;
        if (i < nc) c[i] = load_chunk<F32>(a.x, base + (k < a.K ? k : (int64_t)i * 512));
      }
    };
    Chunk<F32> cur[NC], nxt[NC];
    if (wave < a.rows) load_row(wave, cur);
    for (int64_t row = wave; row < a.rows; row += nwaves) {
      if (row + nwaves < a.rows) load_row(row + nwaves, nxt);
      float A;
      if (a.amax_in) {
        A = a.amax_in[row];
      } else {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          if (i < nc && (int64_t)i * 512 + lane * 8 < a.K) {
            float v[8];
            unpack_chunk<F32>(cur[i], v);
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
          }
        }
        A = wave_max(m);
      }
      const float S = finish_scale(row, A);
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        if (i < nc) {
          const int64_t k = (int64_t)i * 512 + lane * 8;
          float v[8];
          unpack_chunk<F32>(cur[i], v);
          uint32_t sf;
          Rand4 rnd;
          if (SR) rnd = philox4x64_10((uint64_t)(k >> 3), (uint64_t)row, 0, 0, a.sr_seed);
          store(row, k, quant_half_block<SR>(v, S, nullptr, sf, bad, &rnd), sf);
        }
      }
#pragma unroll
      for (int i = 0; i < NC; ++i) cur[i] = nxt[i];
    }
  } else {
    for (int64_t row = wave; row < a.rows; row += nwaves) {
      const int64_t base = row_off(a, row);
      float A;
      if (a.amax_in) {
        A = a.amax_in[row];
      } else {
        float m = 0.0f;
        for (int64_t k = (int64_t)lane * 8; k < a.K; k += 512) {
          float v[8];
          unpack_chunk<F32>(load_chunk<F32>(a.x, base + k), v);
#pragma unroll
          for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
        }
        A = wave_max(m);
      }
      const float S = finish_scale(row, A);
      for (int64_t k0 = 0; k0 < a.K; k0 += 512) {
        const int64_t k = k0 + (int64_t)lane * 8;
        float v[8];
        unpack_chunk<F32>(load_chunk<F32>(a.x, base + (k < a.K ? k : k0)), v);
        uint32_t sf;
        Rand4 rnd;
        if (SR) rnd = philox4x64_10((uint64_t)(k >> 3), (uint64_t)row, 0, 0, a.sr_seed);
        store(row, k, quant_half_block<SR>(v, S, nullptr, sf, bad, &rnd), sf);
      }
    }
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

// A = max |x[i]| over n FP32 values (the tensor amax from recorded per-row amaxes)
__global__ __launch_bounds__(kThreads) void k_amax_vec(const float *x, int64_t n, float *amax, int32_t *dev_status) {
  float m = 0.0f;
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) {
    const float v = fabsf(x[i]);
    bad |= !(v <= 3.402823466e38f);
    m = fmaxf(m, v);
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) atomic_max_nonneg(amax, m);
  if (bad && dev_status) atomicOr(dev_status, kDsNonFinite);
}

// Column layouts (transposed operands of the backward GEMMs).  Output row `c`
// (a column of x) holds 16-element blocks along positions p of the new K; block
// p/16 takes 16 consecutive rows of one segment (zero beyond the segment's end):
//   NV4_COLS          segment s owns positions [pad[s], pad[s+1]) and rows
//                     [off[s], off[s+1]); output row c; positions past pad[nseg]
//                     are not written.
//   NV4_COLS_BATCHED  matrix s (rows [s*m, (s+1)*m)) -> output rows s*C + c,
//                     positions [0, m).
// One workgroup transposes a tile of P positions x C columns through LDS:
//   1. coalesced loads of the tile's source rows, 8 elements per lane and pass (all
//      passes in flight together), zero for padding;
//   2. with ROWS_TOO (NV4_ROWS_AND_COLS) the row-direction quantisation of the
//      tile's rows straight from those registers (the two lanes of a 16-element
//      block exchange their half maxima), so the source is read once for both
//      operands of a tensor that feeds a data gradient and a weight gradient;
//   3. the tile into LDS [position][column], 16-byte units of a row XOR-permuted by
//      the row so that reads along rows and down columns spread over the banks;
//   4. column blocks: each thread reads 16 rows x (2 or 4) columns (one 4- or
//      8-byte LDS read per row), block amax, E4M3 scale, 16 E2M1 codes per column,
//      into an LDS out-tile;
//   5. coalesced stores: 8 lanes write one output row's P/2 code bytes.
constexpr int kSegLds = 256;       // segment offsets staged in LDS up to this many segments
constexpr int kOutPitch = 72;       // LDS out-tile row pitch for 64 code bytes (+8 breaks bank aliasing)
constexpr int kScalePitch = 12;

template <bool F32, int P, int C, bool ROWS_TOO, bool SR, bool NT = true>
__global__ __launch_bounds__(kThreads) void k_quant_cols(QuantArgs a, int ptiles_per_seg, int gx, int64_t ntiles) {
  typedef typename std::conditional<F32, float, uint16_t>::type T;
  static_assert(P == 128, "tiles of 128 positions (8 blocks)");
  constexpr int NB = P / 16;                          // blocks per column per tile
  constexpr int kRowBytes = C * (int)sizeof(T);       // bytes of a tile row
  constexpr int kUnits = kRowBytes / 16;              // 16-byte units per tile row (a power of two)
  static_assert((kUnits & (kUnits - 1)) == 0, "row units must be a power of two");
  constexpr int kLanesPerRow = C / 8;                 // 8-element chunks per tile row
  constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  constexpr int kPasses = P / kRowsPerPass;
  constexpr int kPatchCols = C * NB / kThreads;       // columns per thread in the column phase
  constexpr int kPatchGroups = C / kPatchCols;        // column groups per block row
  constexpr int kReadBytes = kPatchCols * (int)sizeof(T);
  static_assert(kReadBytes == 4 || kReadBytes == 8, "column reads of 4 or 8 bytes");
  static_assert(kPatchGroups * NB == kThreads, "one column patch per thread");
  // The column output tile reuses the input tile's LDS once every read of the input
  // is done (the column results wait in registers), so that more workgroups fit on
  // a CU and keep more loads in flight.
  struct OutTile {
    uint8_t codes[C][kOutPitch];
    uint8_t scales[C][kScalePitch];
  };
  static_assert(sizeof(OutTile) <= (size_t)P * kRowBytes, "output tile fits in the input tile");
  __shared__ __attribute__((aligned(16))) uint8_t tile[P * kRowBytes];
  OutTile &otile = *reinterpret_cast<OutTile *>(&tile[0]);
  auto &ocodes = otile.codes;
  auto &oscales = otile.scales;
  __shared__ int64_t bsrc[NB];
  __shared__ int bnum[NB], bgrp[NB];
  __shared__ float inv_tab[128];
  __shared__ int seg_pad[kSegLds + 1], seg_off[kSegLds + 1];
  // byte offset of 16-byte unit u of tile row `row`
  auto unit_off = [](int row, int u) -> int { return row * kRowBytes + ((u ^ (row & (kUnits - 1))) << 4); };

  // Tile t = by * gx + bx (column tile bx, position tile by).  Workgroup g runs on XCD
  // g % 8 (the hardware's round-robin).  Tiles write scale bytes in 8-byte pieces of
  // 64-byte lines (per output row and tile); pieces of one line merge in an XCD's L2
  // before being written back only if they come from the same XCD, close in time.
  // Column scales: the next position tile (t + gx) holds the neighbouring pieces, and
  // with gx % 8 == 0 tile t on workgroup t already puts it on the same XCD, four tiles
  // later.  Row scales (NV4_ROWS_AND_COLS): the neighbouring pieces are in the other
  // column tiles of the band (t + 1, ...).  So the tiles go to the XCDs in 8 contiguous
  // chunks, one per XCD, for the rows-and-columns passes and whenever gx % 8 != 0
  // (measured on the learner batch: the rows-and-columns pass of dY2, gx = 16, writes
  // 1231 instead of 1412 MB for 1210 MB of output and runs 5 % faster, those of the
  // SwiGLU output and dY13, gx = 6 and 12, 5 % faster).
  // Gathered rows (X in expert order, each token's row in k segments): the tiles are
  // taken column tile by column tile (t = bx * gy + by), so that the k repeats of a
  // row's C columns fall within one column tile's pass over the positions and are
  // read from the caches (the 64-column slab of the learner batch's X is 8 MB); in
  // chunks, so that position-neighbours stay on one XCD (0.64 -> 0.56 ms; the
  // position-major order in chunks was 2 % slower than in the plain order).
  int64_t t = blockIdx.x;
  const bool gathered = !ROWS_TOO && a.row_index != nullptr;
  if (gathered || ROWS_TOO || gx % kXcdCount) {
    const int64_t chunk = (ntiles + kXcdCount - 1) / kXcdCount;
    t = (int64_t)(blockIdx.x % kXcdCount) * chunk + blockIdx.x / kXcdCount;
  }
  if (t >= ntiles) return;  // uniform over the workgroup
  const int64_t gy = ntiles / gx;  // position tiles
  const int64_t bx = gathered ? t / gy : t % gx, by = gathered ? t % gy : t / gx;
  if (blockIdx.x == 0) write_group_scales(a);
  const float *A = amax_src(a);
  const int64_t Ccols = a.K;  // columns of x
  const int64_t c0 = bx * C;
  const bool batched = a.layout == NV4_COLS_BATCHED;
  int s_tile = 0;
  int64_t p0, plimit, orow0;
  if (batched) {
    s_tile = (int)(by / ptiles_per_seg);
    p0 = (by % ptiles_per_seg) * P;
    plimit = a.rows / a.nseg;
    orow0 = (int64_t)s_tile * Ccols + c0;
  } else {
    p0 = by * P;
    plimit = a.seg_padded_offsets[a.nseg];
    orow0 = c0;
  }
  if (p0 >= plimit) return;  // uniform over the workgroup
  // NV4_COLS: the segments' offsets, searched below, from LDS when they fit (one
  // coalesced load instead of a chain of dependent loads)
  const bool seg_in_lds = !batched && a.nseg <= kSegLds;
  if (seg_in_lds) {
    for (int i = threadIdx.x; i <= a.nseg; i += kThreads) {
      seg_pad[i] = a.seg_padded_offsets[i];
      seg_off[i] = a.seg_offsets[i];
    }
    __syncthreads();
  }
  // SCALE_SEGMENT_HALVES (batched only): positions [0, m/2) of matrix s take group
  // 2s, [m/2, m) group 2s + 1 (the first and second half of the matrix's rows)
  const bool halves = a.scale_mode == NV4_SCALE_SEGMENT_HALVES;
  const bool seg_scales = a.scale_mode == NV4_SCALE_SEGMENT || halves;
  // per-block source rows: start, count (0..16), scale group
  if (threadIdx.x < NB) {
    const int j = threadIdx.x;
    const int64_t p = p0 + 16 * j;
    int64_t start = 0;
    int n = 0, g = 0;
    if (p < plimit) {
      if (batched) {
        start = (int64_t)s_tile * plimit + p;
        n = 16;
        g = halves ? 2 * s_tile + (p >= plimit / 2 ? 1 : 0) : (seg_scales ? s_tile : 0);
      } else {
        const int *pad = seg_in_lds ? seg_pad : a.seg_padded_offsets;
        const int *off = seg_in_lds ? seg_off : a.seg_offsets;
        int lo = 0, hi = a.nseg - 1;  // last segment s with pad[s] <= p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (pad[mid] <= p) lo = mid; else hi = mid - 1;
        }
        start = off[lo] + (p - pad[lo]);
        n = (int)std::min<int64_t>(16, std::max<int64_t>(0, off[lo + 1] - start));
        g = seg_scales ? lo : 0;
      }
    }
    bsrc[j] = start;
    bnum[j] = n;
    bgrp[j] = g;
  }
  // one tensor scale for the whole tile: 1 / block scale from a table
  const bool straddle = halves && p0 < plimit / 2 && p0 + P > plimit / 2;
  const bool uniform = (!seg_scales || batched) && !straddle;
  const int tile_group = !seg_scales ? 0 : (halves ? 2 * s_tile + (p0 >= plimit / 2 ? 1 : 0) : s_tile);
  const float S_tile = tensor_encode_scale(A[uniform ? tile_group : 0]);
  if (uniform && threadIdx.x < 128)
    inv_tab[threadIdx.x] = threadIdx.x ? __fdiv_rn(S_tile, e4m3_to_f32(threadIdx.x)) : 0.0f;
  __syncthreads();

  bool bad = false;
  // 1. load the tile: lane (lr, lch) takes 8 elements at column c0 + 8 lch of tile rows
  // lr + i * kRowsPerPass
  const int lr = threadIdx.x / kLanesPerRow, lch = threadIdx.x % kLanesPerRow;
  const bool col_ok = c0 + lch * 8 < Ccols;
  Chunk<F32> v[kPasses];
#pragma unroll
  for (int i = 0; i < kPasses; ++i) {
    const int pp = i * kRowsPerPass + lr;
    const int j = pp >> 4, r = pp & 15;
    v[i] = Chunk<F32>{};
    if (col_ok && r < bnum[j]) v[i] = load_chunk<F32, NT>(a.x, row_off(a, bsrc[j] + r) + c0 + lch * 8);
  }
  // 2. row blocks of the tile's valid rows (tensor scale) from the loaded registers:
  // lanes 2m and 2m + 1 of a row hold the two halves of one 16-element block
  if (ROWS_TOO) {
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const int pp = i * kRowsPerPass + lr;
      const int j = pp >> 4, r = pp & 15;
      const bool ok = col_ok && r < bnum[j];
      const int64_t orow = bsrc[j] + r;  // logical row of x
      float vv[8];
      unpack_chunk<F32>(v[i], vv);
      Rand4 rnd;
      if (SR) rnd = philox4x64_10((uint64_t)((c0 + lch * 8) >> 3), (uint64_t)orow, 0, 0, a.sr_seed);
      uint32_t sf;
      bool bad_row = false;
      const uint32_t p = quant_half_block<SR>(vv, S_tile, inv_tab, sf, bad_row, &rnd);
      if (ok) {
        bad |= bad_row;
        reinterpret_cast<uint32_t *>(a.codes2 + orow * (Ccols >> 1))[(c0 >> 3) + lch] = p;
        if ((lch & 1) == 0) a.scales2[orow * (Ccols >> 4) + ((c0 + lch * 8) >> 4)] = (uint8_t)sf;
      }
    }
  }
  // 3. the tile into LDS
#pragma unroll
  for (int i = 0; i < kPasses; ++i) {
    const int pp = i * kRowsPerPass + lr;
#pragma unroll
    for (int w = 0; w < (F32 ? 2 : 1); ++w)
      *reinterpret_cast<uint4 *>(&tile[unit_off(pp, lch * (F32 ? 2 : 1) + w)]) = v[i].w[w];
  }
  __syncthreads();

  // rnd0 / rnd1: the Philox blocks of the 16 elements' positions (SR only)
  auto quant16 = [&](const float vv[16], float S, bool use_tab, uint32_t &lo, uint32_t &hi, const Rand4 &rnd0,
                     const Rand4 &rnd1) -> uint32_t {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float av = fabsf(vv[i]);
      bad |= !(av <= 3.402823466e38f);
      m = fmaxf(m, av);
    }
    const uint32_t sf = e4m3_from_f32(__fmul_rn(div6_rn(m), S));
    const float inv = use_tab ? inv_tab[sf] : (sf ? __fdiv_rn(S, e4m3_to_f32(sf)) : 0.0f);
    if (SR) {
      lo = pack_e2m1_sr8(vv, inv, rnd0);
      hi = pack_e2m1_sr8(vv + 8, inv, rnd1);
      return sf;
    }
    lo = 0;
    hi = 0;
    lo = pack_e2m1_pair<0>(lo, __fmul_rn(vv[0], inv), __fmul_rn(vv[1], inv));
    lo = pack_e2m1_pair<1>(lo, __fmul_rn(vv[2], inv), __fmul_rn(vv[3], inv));
    lo = pack_e2m1_pair<2>(lo, __fmul_rn(vv[4], inv), __fmul_rn(vv[5], inv));
    lo = pack_e2m1_pair<3>(lo, __fmul_rn(vv[6], inv), __fmul_rn(vv[7], inv));
    hi = pack_e2m1_pair<0>(hi, __fmul_rn(vv[8], inv), __fmul_rn(vv[9], inv));
    hi = pack_e2m1_pair<1>(hi, __fmul_rn(vv[10], inv), __fmul_rn(vv[11], inv));
    hi = pack_e2m1_pair<2>(hi, __fmul_rn(vv[12], inv), __fmul_rn(vv[13], inv));
    hi = pack_e2m1_pair<3>(hi, __fmul_rn(vv[14], inv), __fmul_rn(vv[15], inv));
    return sf;
  };

  // 4. column blocks: thread (block row jb, column group cg) takes columns
  // cg * kPatchCols + [0, kPatchCols) of positions 16 jb + [0, 16)
  const int jb = threadIdx.x / kPatchGroups, cg = threadIdx.x % kPatchGroups;
  uint32_t col_lo[kPatchCols], col_hi[kPatchCols], col_sf[kPatchCols];
  {
    typedef typename std::conditional<kReadBytes == 8, uint2, uint32_t>::type RT;
    const int cb = cg * kReadBytes;  // byte column of the patch inside a tile row
    RT raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 16 * jb + i;
      raw[i] = *reinterpret_cast<const RT *>(&tile[unit_off(row, cb >> 4) + (cb & 15)]);
    }
    const float S = uniform ? S_tile : tensor_encode_scale(A[bgrp[jb]]);
#pragma unroll
    for (int q = 0; q < kPatchCols; ++q) {
      float vv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t *w = reinterpret_cast<const uint32_t *>(&raw[i]);
        vv[i] = F32 ? __uint_as_float(w[q])
                    : __uint_as_float((q & 1) ? (w[q >> 1] & 0xFFFF0000u) : (w[q >> 1] << 16));
      }
      uint32_t lo, hi;
      Rand4 r0, r1;
      if (SR) {  // output row orow0 + c, positions p0 + 16 jb + [0, 16), stream 1
        const int c = cg * kPatchCols + q;
        const uint64_t pc = (uint64_t)((p0 >> 3) + 2 * jb);
        r0 = philox4x64_10(pc, (uint64_t)(orow0 + c), 1, 0, a.sr_seed);
        r1 = philox4x64_10(pc + 1, (uint64_t)(orow0 + c), 1, 0, a.sr_seed);
      }
      col_sf[q] = quant16(vv, S, uniform, lo, hi, r0, r1);
      col_lo[q] = lo;
      col_hi[q] = hi;
    }
  }
  __syncthreads();
  {  // every read of the input tile is done: its LDS becomes the output tile
#pragma unroll
    for (int q = 0; q < kPatchCols; ++q) {
      const int c = cg * kPatchCols + q;
      *reinterpret_cast<uint2 *>(&ocodes[c][8 * jb]) = make_uint2(col_lo[q], col_hi[q]);
      oscales[c][jb] = (uint8_t)col_sf[q];
    }
    __syncthreads();
  }

  // 5. coalesced stores: 8 lanes per output row, one block (8 code bytes) each
  {
    const int j = threadIdx.x & 7, rr = threadIdx.x >> 3;
    const bool blk_ok = p0 + 16 * j < plimit;
    const int64_t cstride = a.out_K >> 1, sstride = a.out_K >> 4;
#pragma unroll
    for (int pass = 0; pass < C / 32; ++pass) {
      const int c = pass * 32 + rr;
      if (blk_ok && c0 + c < Ccols) {
        const int64_t orow = orow0 + c;
        *reinterpret_cast<uint2 *>(a.codes + orow * cstride + (p0 >> 1) + 8 * j) =
            *reinterpret_cast<const uint2 *>(&ocodes[c][8 * j]);
        a.scales[orow * sstride + (p0 >> 4) + j] = oscales[c][j];
      }
    }
  }
  if (bad && a.dev_status) atomicOr(a.dev_status, kDsNonFinite);
}

template <bool SR>
hipError_t launch_quantize_t(const QuantArgs &a, hipStream_t stream) {
  const int cus = device_cu_count();
  const int per_row = a.scale_mode == NV4_SCALE_ROW;
  const bool f32 = a.x_is_f32 != 0;
  if (a.rows == 0 || a.K == 0) {
    if (a.ngroups > 0) {
      if (!a.amax_in) k_fill_zero<<<(a.ngroups + 255) / 256, 256, 0, stream>>>(a.amax_acc, a.ngroups);
      k_group_scales<<<1, kThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
  }
  // group amax pass (tensor / segment scales without a supplied amax)
  if (!a.amax_in && !per_row) {
    k_fill_zero<<<(a.ngroups + 255) / 256, 256, 0, stream>>>(a.amax_acc, a.ngroups);
    if (a.rows > 0) {
      // about one workgroup per CU in total, split over the groups, at most one
      // per 2048 chunks of a group
      const int groups = a.ngroups;
      const int64_t chunks_per_group = (a.rows + groups - 1) / groups * (a.K >> 3);
      const int P = (int)std::max<int64_t>(1, std::min<int64_t>(cus / groups, (chunks_per_group + 2047) / 2048));
      if (f32) k_amax_rows<true><<<dim3(P, groups), kThreads, 0, stream>>>(a, P);
      else k_amax_rows<false><<<dim3(P, groups), kThreads, 0, stream>>>(a, P);
    }
  }
  if (a.layout == NV4_ROWS) {
    if (per_row) {
      const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((a.rows + 3) / 4, (int64_t)cus * 16));
      // register cache of 2, 4 or 8 rounds of 512 elements, or none for longer rows
      const int64_t nc = (a.K + 511) / 512;
      auto go = [&](auto ncc) {
        constexpr int N = decltype(ncc)::value;
        if (f32) k_quant_rows_per_row<true, SR, N><<<grid, kThreads, 0, stream>>>(a);
        else k_quant_rows_per_row<false, SR, N><<<grid, kThreads, 0, stream>>>(a);
      };
      if (nc <= 2) go(std::integral_constant<int, 2>{});
      else if (nc <= 4) go(std::integral_constant<int, 4>{});
      else if (nc <= 8) go(std::integral_constant<int, 8>{});
      else go(std::integral_constant<int, 0>{});
    } else {
      const int64_t chunks = a.rows * (a.K >> 3);
      const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((chunks + 2 * kThreads - 1) / (2 * kThreads), (int64_t)cus * 8));
      const bool tensor = a.scale_mode == NV4_SCALE_TENSOR;
      if (f32) {
        if (tensor) k_quant_rows<true, true, SR><<<grid, kThreads, 0, stream>>>(a);
        else k_quant_rows<true, false, SR><<<grid, kThreads, 0, stream>>>(a);
      } else {
        if (tensor) k_quant_rows<false, true, SR><<<grid, kThreads, 0, stream>>>(a);
        else k_quant_rows<false, false, SR><<<grid, kThreads, 0, stream>>>(a);
      }
    }
  } else {
    // tiles of 128 positions x 64 columns, or 128 columns for BF16 rows and columns
    // together (the row blocks need 64 columns per thread); NV4_COLS: an upper
    // bound of the padded positions (rows + 15 per segment), tiles past the actual
    // end exit at once.  (Measured on the learner batch: the gathered column
    // quantisation of X takes 0.71 ms with 64 columns, 0.85 ms with 128, 0.92 ms
    // with 32 and 1.26 ms with 256; rows and columns together are 20 % slower with
    // 64 columns than with 128.)
    constexpr int P = 128;
    const bool both = a.layout == NV4_ROWS_AND_COLS;
    const int C = (!f32 && both) ? 128 : 64;
    const unsigned gx = (unsigned)std::max<int64_t>(1, (a.K + C - 1) / C);
    int ptiles;
    unsigned gy;
    if (a.layout == NV4_COLS_BATCHED) {
      ptiles = (int)((a.rows / a.nseg + P - 1) / P);
      gy = (unsigned)(ptiles * a.nseg);
    } else {
      ptiles = 0;
      gy = (unsigned)std::max<int64_t>(1, (a.rows + 15 * (int64_t)a.nseg + P - 1) / P);
    }
    // one workgroup per tile, in a 1-D grid rounded up to a multiple of the XCD count
    const int64_t ntiles = (int64_t)gx * gy;
    const unsigned grid = (unsigned)(((ntiles + kXcdCount - 1) / kXcdCount) * kXcdCount);
    if (f32) {
      if (both) k_quant_cols<true, P, 64, true, SR><<<grid, kThreads, 0, stream>>>(a, ptiles, (int)gx, ntiles);
      else k_quant_cols<true, P, 64, false, SR><<<grid, kThreads, 0, stream>>>(a, ptiles, (int)gx, ntiles);
    } else {
      if (both) k_quant_cols<false, P, 128, true, SR><<<grid, kThreads, 0, stream>>>(a, ptiles, (int)gx, ntiles);
      else if (a.row_index)  // gathered rows (X in expert order) repeat: ordinary loads
        k_quant_cols<false, P, 64, false, SR, false><<<grid, kThreads, 0, stream>>>(a, ptiles, (int)gx, ntiles);
      else k_quant_cols<false, P, 64, false, SR><<<grid, kThreads, 0, stream>>>(a, ptiles, (int)gx, ntiles);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_amax_vec(const float *x, int64_t n, float *amax, int32_t *dev_status, hipStream_t stream) {
  k_fill_zero<<<1, 64, 0, stream>>>(amax, 1);
  if (n > 0) {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n + kThreads - 1) / kThreads, 256));
    k_amax_vec<<<grid, kThreads, 0, stream>>>(x, n, amax, dev_status);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs &a, hipStream_t stream) {
  return a.sr ? launch_quantize_t<true>(a, stream) : launch_quantize_t<false>(a, stream);
}

}  // namespace nv4
