// Grouped NVFP4 x NVFP4 GEMM for gfx950 (W4A4 expert GEMMs).
//
// "Low-Bit Precision Training ...", section "What W4A4 GEMM Actually Changes":
// both operands are 4-bit and the GEMM consumes them directly.  "miniTE ...",
// section "Development: Aligning Numerics, Then Making NVFP4 Fast": the expert
// work is a grouped GEMM.  "The 4-bitter Lesson", section "Improving Gradient
// Stability": the product is taken with the dequantised operands DQ(Q(.)).
//
// Design for CDNA4.  gfx950's scaled FP4 matrix instructions take power-of-two
// (E8M0) scales per 32 elements, while NVFP4 scales are E4M3 per 16 elements, so
// they cannot apply NVFP4 block scales exactly.  Instead every operand element
// is decoded exactly to FP16: e2m1 * e4m3 has at most 6 significant bits and
// lies in [2^-10, 2688], so the FP4->FP16 converter (scale 1) followed by a
// packed FP16 multiply by the block scale never rounds.  The FP16 MFMA
// (v_mfma_f32_32x32x16_f16) forms exact products and accumulates in FP32; the
// FP32 tensor scales G_a * G_b are applied in the epilogue.
//
// Data flow per workgroup tile (persistent workgroups walk the tiles):
//   HBM -> registers (16-byte loads of packed codes, 8-byte loads of scale bytes)
//   -> LDS (packed, XOR-swizzled 16-byte chunks, double buffered)
//   -> each wave reads its fragments (one 16-byte read per 64 K per fragment row)
//   -> decode to FP16 in registers -> MFMA.
// K permutation: inside each 64-wide K slice, lane half h of an MFMA operand
// supplies elements h*32 + s*8 + [0, 8) in MFMA step s, for both A and B, so that
// one 16-byte LDS read gives a lane all 32 codes it needs for the slice.  Any
// permutation of K applied to both operands leaves the dot product unchanged.
//
// Tile order: the logical tile index is split so that the workgroups of one XCD
// (hardware assigns workgroup i to XCD i % 8) take consecutive tiles, which share
// the A rows (same M tile) and the expert's B matrix in that XCD's L2.
#include <algorithm>

#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kXcds = 8;

template <int WAVES_M, int WAVES_N, int FM, int FN>
struct TileCfg {
  static constexpr int kWavesM = WAVES_M, kWavesN = WAVES_N, kFM = FM, kFN = FN;
  static constexpr int BM = WAVES_M * FM * 32;
  static constexpr int BN = WAVES_N * FN * 32;  // rows of B per tile
  static constexpr int BK = 128;                // K per LDS stage
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kRowBytes = BK / 2;      // packed codes per row per stage
  static constexpr int kScBytes = BK / 16;      // scale bytes per row per stage
  static constexpr int kStageBytes = (BM + BN) * (kRowBytes + kScBytes);
};

// an index into A taken from the caller: clamp into [0, rows) so that an index
// outside the contract cannot read outside the buffer
__device__ __forceinline__ int64_t min_row(int32_t idx, int64_t rows) {
  return idx < 0 ? 0 : (idx >= rows ? rows - 1 : idx);
}

// LDS position of 16-byte chunk q (0..3) of tile row r
__device__ __forceinline__ int swz(int q, int r) { return q ^ ((r >> 1) & 3); }

struct TileJob {
  int e;
  int64_t m0, m_end;   // GROUP_M: rows of A/C; GROUP_K: rows of A (N dimension)
  int64_t n0;          // first B row of the tile (GROUP_K: first row of B)
  int64_t k_lo, k_hi;  // contraction range
};

// Per-expert tile counts -> exclusive prefix in LDS (one pass per workgroup).
template <int NT>
__device__ void expert_tile_prefix(const int32_t *offsets, int E, int BM, int *tstart, int *scratch) {
  const int tid = threadIdx.x;
  const int per = (E + NT - 1) / NT;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      const int n = offsets[e + 1] - offsets[e];
      local += (n + BM - 1) / BM;
    }
  }
  scratch[tid] = local;
  __syncthreads();
  for (int o = 1; o < NT; o <<= 1) {
    const int x = tid >= o ? scratch[tid - o] : 0;
    __syncthreads();
    scratch[tid] += x;
    __syncthreads();
  }
  int run = scratch[tid] - local;
  for (int i = 0; i < per; ++i) {
    const int e = tid * per + i;
    if (e < E) {
      tstart[e] = run;
      const int n = offsets[e + 1] - offsets[e];
      run += (n + BM - 1) / BM;
    }
  }
  if (tid == NT - 1) tstart[E] = scratch[tid];
  __syncthreads();
}

template <class Cfg, int GROUP, int EPI, bool OUT_F32, bool A_ROW_SCALE>
__global__ __launch_bounds__(Cfg::kThreads) void k_gemm(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  constexpr int RB = Cfg::kRowBytes, SB = Cfg::kScBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Cfg::kStageBytes];
  __shared__ int tstart[kMaxExperts + 1];
  __shared__ int scratch[NT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5, l32 = lane & 31;
  const int E = g.E;
  const int64_t K = g.K;
  const int64_t ldA = K >> 1, ldAs = K >> 4;  // bytes per row: codes, scales

  // ---- tile space
  int64_t total;
  int ntn;
  if (GROUP == NV4_GROUP_M) {
    expert_tile_prefix<NT>(g.offsets, E, BM, tstart, scratch);
    ntn = (int)(EPI == NV4_EPI_SWIGLU ? (g.N + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN);
    total = (int64_t)tstart[E] * ntn;
  } else {
    // GROUP_K: A [N][K], B [M][K]; per expert (N/BM) x (M/BN) tiles
    const int tn = (int)((g.a_rows + BM - 1) / BM);
    const int tm = (int)((g.b_rows + BN - 1) / BN);
    ntn = tm;
    total = (int64_t)E * tn * tm;
  }
  const int G = gridDim.x;
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;

  const float a_ts = (!A_ROW_SCALE) ? g.a_tscale[0] : 1.0f;
  float amax_run = 0.0f;

  for (int64_t it = 0;; ++it) {
    const int64_t L = it * G + (int64_t)xcd * per_xcd + slot;
    if (L >= total) break;
    TileJob job;
    int64_t nt_idx;
    if (GROUP == NV4_GROUP_M) {
      const int64_t mt = L / ntn;
      nt_idx = L - mt * ntn;
      int lo = 0, hi = E - 1;  // last expert with tstart[e] <= mt
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tstart[mid] <= mt) lo = mid; else hi = mid - 1;
      }
      job.e = lo;
      job.m0 = g.offsets[lo] + (mt - tstart[lo]) * BM;
      job.m_end = std::min<int64_t>(g.offsets[lo + 1], g.M_cap);  // never past the caller's C rows
      job.n0 = nt_idx;  // resolved per row below
      job.k_lo = 0;
      job.k_hi = K;
    } else {
      const int tn = (int)((g.a_rows + BM - 1) / BM);
      const int64_t per_e = (int64_t)tn * ntn;
      job.e = (int)(L / per_e);
      const int64_t r = L - job.e * per_e;
      const int64_t tni = r / ntn;
      nt_idx = r - tni * ntn;
      job.m0 = tni * BM;
      job.m_end = g.a_rows;
      job.n0 = nt_idx * BN;
      job.k_lo = g.offsets[job.e];
      job.k_hi = g.offsets[job.e + 1];
    }

    // ---- per-thread load assignments (fixed for the tile)
    // codes: (BM + BN) rows x 4 chunks of 16 bytes
    constexpr int kChunks = (BM + BN) * 4;
    constexpr int kChunkIters = (kChunks + NT - 1) / NT;
    const uint8_t *src_c[kChunkIters];
    int lds_c[kChunkIters];
    bool ok_c[kChunkIters];
#pragma unroll
    for (int i = 0; i < kChunkIters; ++i) {
      const int id = tid + i * NT;
      const int row = id >> 2, q = id & 3;
      src_c[i] = nullptr;
      lds_c[i] = 0;
      ok_c[i] = false;
      if (id < kChunks) {
        if (row < BM) {
          const int64_t gr = job.m0 + row;
          if (gr < job.m_end) {
            int64_t pr = gr;
            if (GROUP == NV4_GROUP_M && g.a_rows_index) pr = min_row(g.a_rows_index[gr], g.a_rows);
            src_c[i] = g.a_codes + pr * ldA + q * 16;
            ok_c[i] = true;
          }
          lds_c[i] = row * RB + swz(q, row) * 16;
        } else {
          const int br = row - BM;
          int64_t grow = -1;
          if (GROUP == NV4_GROUP_M) {
            if (EPI == NV4_EPI_SWIGLU) {
              const int wv = br / (FN * 32), f = (br % (FN * 32)) / 32;
              const int half = FN / 2;
              const int64_t col = nt_idx * (BN / 2) + wv * (half * 32) + (f % half) * 32 + (br & 31);
              if (col < g.N) grow = (int64_t)job.e * 2 * g.N + (f >= half ? g.N : 0) + col;
            } else {
              const int64_t col = nt_idx * BN + br;
              if (col < g.N) grow = (int64_t)job.e * g.N + col;
            }
          } else {
            const int64_t col = job.n0 + br;
            if (col < g.b_rows) grow = col;
          }
          if (grow >= 0) {
            src_c[i] = g.b_codes + grow * ldA + q * 16;
            ok_c[i] = true;
          }
          lds_c[i] = BM * RB + br * RB + swz(q, br) * 16;
        }
      }
    }
    // scale bytes: (BM + BN) rows x 8 bytes (two dwords)
    constexpr int kScIters = ((BM + BN) + NT - 1) / NT;
    const uint8_t *src_s[kScIters];
    int lds_s[kScIters];
#pragma unroll
    for (int i = 0; i < kScIters; ++i) {
      const int row = tid + i * NT;
      src_s[i] = nullptr;
      lds_s[i] = -1;
      if (row < BM + BN) {
        if (row < BM) {
          const int64_t gr = job.m0 + row;
          if (gr < job.m_end) {
            int64_t pr = gr;
            if (GROUP == NV4_GROUP_M && g.a_rows_index) pr = min_row(g.a_rows_index[gr], g.a_rows);
            src_s[i] = g.a_scales + pr * ldAs;
          }
        } else {
          const int br = row - BM;
          int64_t grow = -1;
          if (GROUP == NV4_GROUP_M) {
            if (EPI == NV4_EPI_SWIGLU) {
              const int wv = br / (FN * 32), f = (br % (FN * 32)) / 32;
              const int half = FN / 2;
              const int64_t col = nt_idx * (BN / 2) + wv * (half * 32) + (f % half) * 32 + (br & 31);
              if (col < g.N) grow = (int64_t)job.e * 2 * g.N + (f >= half ? g.N : 0) + col;
            } else {
              const int64_t col = nt_idx * BN + br;
              if (col < g.N) grow = (int64_t)job.e * g.N + col;
            }
          } else {
            const int64_t col = job.n0 + br;
            if (col < g.b_rows) grow = col;
          }
          if (grow >= 0) src_s[i] = g.b_scales + grow * ldAs;
        }
        lds_s[i] = (BM + BN) * RB + row * SB;
      }
    }

    // ---- K range in stages of BK (stage starts 128-aligned; blocks outside [k_lo, k_hi) are masked)
    const int64_t kb0 = (job.k_lo / BK) * BK;
    const int nk = job.k_hi > job.k_lo ? (int)((job.k_hi - kb0 + BK - 1) / BK) : 0;

    uint4 rc[kChunkIters];
    uint2 rs[kScIters];
    auto gload = [&](int kt) {
      const int64_t k0 = kb0 + (int64_t)kt * BK;
#pragma unroll
      for (int i = 0; i < kChunkIters; ++i) {
        const int q = (tid + i * NT) & 3;
        const int64_t kk = k0 + q * 32;
        if (ok_c[i] && kk < K) rc[i] = *reinterpret_cast<const uint4 *>(src_c[i] + (k0 >> 1));
        else rc[i] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kScIters; ++i) {
        uint2 v = make_uint2(0, 0);
        if (src_s[i]) {
          const uint32_t *p = reinterpret_cast<const uint32_t *>(src_s[i] + (k0 >> 4));
          if (k0 < K) v.x = p[0];
          if (k0 + 64 < K) v.y = p[1];
          // mask blocks outside [k_lo, k_hi): their scale becomes 0, so they decode to 0
          if (GROUP == NV4_GROUP_K) {
            uint32_t mlo = 0, mhi = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int64_t kbl = k0 + b * 16, kbh = k0 + 64 + b * 16;
              if (kbl >= job.k_lo && kbl < job.k_hi) mlo |= 0xFFu << (8 * b);
              if (kbh >= job.k_lo && kbh < job.k_hi) mhi |= 0xFFu << (8 * b);
            }
            v.x &= mlo;
            v.y &= mhi;
          }
        }
        rs[i] = v;
      }
    };
    auto sstore = [&](int buf) {
      uint8_t *base = lds + buf * Cfg::kStageBytes;
#pragma unroll
      for (int i = 0; i < kChunkIters; ++i)
        if (tid + i * NT < kChunks) *reinterpret_cast<uint4 *>(base + lds_c[i]) = rc[i];
#pragma unroll
      for (int i = 0; i < kScIters; ++i)
        if (lds_s[i] >= 0) *reinterpret_cast<uint2 *>(base + lds_s[i]) = rs[i];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
      gload(0);
      sstore(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) gload(kt + 1);
      const uint8_t *base = lds + (kt & 1) * Cfg::kStageBytes;
      const uint8_t *sbase = base + (BM + BN) * RB;
#pragma unroll
      for (int sub = 0; sub < BK / 64; ++sub) {
        uint4 ca[FM], cb[FN];
        f16x2 sa[FM], sbv[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * FM * 32 + i * 32 + l32;
          ca[i] = *reinterpret_cast<const uint4 *>(base + row * RB + swz(sub * 2 + h, row) * 16);
          const uint32_t s2 = *reinterpret_cast<const uint16_t *>(sbase + row * SB + sub * 4 + 2 * h);
          sa[i] = e4m3x2_to_f16(s2);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * FN * 32 + j * 32 + l32;
          cb[j] = *reinterpret_cast<const uint4 *>(base + BM * RB + row * RB + swz(sub * 2 + h, row) * 16);
          const uint32_t s2 = *reinterpret_cast<const uint16_t *>(sbase + (BM + row) * SB + sub * 4 + 2 * h);
          sbv[j] = e4m3x2_to_f16(s2);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          f16x8 av[FM], bv[FN];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const uint32_t w = s == 0 ? ca[i].x : s == 1 ? ca[i].y : s == 2 ? ca[i].z : ca[i].w;
            const _Float16 sc = (s < 2) ? sa[i][0] : sa[i][1];
            av[i] = decode8_f16(w, f16x2{sc, sc});
          }
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const uint32_t w = s == 0 ? cb[j].x : s == 1 ? cb[j].y : s == 2 ? cb[j].z : cb[j].w;
            const _Float16 sc = (s < 2) ? sbv[j][0] : sbv[j][1];
            bv[j] = decode8_f16(w, f16x2{sc, sc});
          }
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
      }
      if (kt + 1 < nk) sstore((kt + 1) & 1);
      __syncthreads();
    }

    // ---- epilogue
    float b_ts = 1.0f;
    if (GROUP == NV4_GROUP_M) b_ts = g.b_scale_mode == NV4_SCALE_SEGMENT ? g.b_tscale[job.e] : g.b_tscale[0];
    else b_ts = g.b_tscale[0];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rloc = wm * FM * 32 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const int64_t grow = job.m0 + rloc;
        if (grow >= job.m_end) continue;
        float sc = a_ts * b_ts;
        if (A_ROW_SCALE) {
          int64_t pr = grow;
          if (g.a_rows_index) pr = min_row(g.a_rows_index[grow], g.a_rows);
          sc = g.a_tscale[pr] * b_ts;
        }
        if (EPI == NV4_EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            const int64_t col = nt_idx * (BN / 2) + wn * (FN / 2 * 32) + j * 32 + l32;
            if (col >= g.N) continue;
            const float gt = acc[i][j][r] * sc;
            const float up = acc[i][j + FN / 2][r] * sc;
            const float hv = gt / (1.0f + expf(-gt)) * up;
            float stored;
            if (OUT_F32) {
              reinterpret_cast<float *>(g.C)[grow * g.ldc + col] = hv;
              stored = hv;
            } else {
              const uint32_t b16 = f32_to_bf16_rne(hv);
              reinterpret_cast<uint16_t *>(g.C)[grow * g.ldc + col] = (uint16_t)b16;
              stored = bf16_bits_to_f32(b16);
            }
            amax_run = fmaxf(amax_run, fabsf(stored));
          }
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            int64_t col, off;
            if (GROUP == NV4_GROUP_M) {
              col = nt_idx * BN + wn * FN * 32 + j * 32 + l32;
              if (col >= g.N) continue;
              off = grow * g.ldc + col;
            } else {
              col = job.n0 + wn * FN * 32 + j * 32 + l32;
              if (col >= g.b_rows) continue;
              off = ((int64_t)job.e * g.a_rows + grow) * g.ldc + col;
            }
            const float v = acc[i][j][r] * sc;
            if (OUT_F32) reinterpret_cast<float *>(g.C)[off] = v;
            else reinterpret_cast<uint16_t *>(g.C)[off] = (uint16_t)f32_to_bf16_rne(v);
          }
        }
      }
    }
  }
  if (EPI == NV4_EPI_SWIGLU && g.amax_out) {
    const float w = wave_max(amax_run);
    if (lane == 0) atomic_max_nonneg(g.amax_out, w);
  }
}

using Cfg128 = TileCfg<2, 2, 2, 2>;

template <int GROUP, int EPI, bool OUT_F32, bool ROWS>
hipError_t launch_cfg(const GemmArgs &g, hipStream_t stream) {
  const int cus = device_cu_count();
  int grid = cus * 4;
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  k_gemm<Cfg128, GROUP, EPI, OUT_F32, ROWS><<<grid, Cfg128::kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmArgs &g, hipStream_t stream) {
  const bool rows = g.a_scale_mode == NV4_SCALE_ROW;
  if (g.group_mode == NV4_GROUP_K) {
    return g.c_is_f32 ? launch_cfg<NV4_GROUP_K, NV4_EPI_NONE, true, false>(g, stream)
                      : launch_cfg<NV4_GROUP_K, NV4_EPI_NONE, false, false>(g, stream);
  }
  if (g.epilogue == NV4_EPI_SWIGLU) {
    if (rows) return g.c_is_f32 ? launch_cfg<NV4_GROUP_M, NV4_EPI_SWIGLU, true, true>(g, stream)
                                : launch_cfg<NV4_GROUP_M, NV4_EPI_SWIGLU, false, true>(g, stream);
    return g.c_is_f32 ? launch_cfg<NV4_GROUP_M, NV4_EPI_SWIGLU, true, false>(g, stream)
                      : launch_cfg<NV4_GROUP_M, NV4_EPI_SWIGLU, false, false>(g, stream);
  }
  if (rows) return g.c_is_f32 ? launch_cfg<NV4_GROUP_M, NV4_EPI_NONE, true, true>(g, stream)
                              : launch_cfg<NV4_GROUP_M, NV4_EPI_NONE, false, true>(g, stream);
  return g.c_is_f32 ? launch_cfg<NV4_GROUP_M, NV4_EPI_NONE, true, false>(g, stream)
                    : launch_cfg<NV4_GROUP_M, NV4_EPI_NONE, false, false>(g, stream);
}

}  // namespace nv4
