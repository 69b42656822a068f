// Grouped NVFP4 x NVFP4 GEMM for gfx950 (W4A4 expert GEMMs): the kernel template and
// its launcher.  Each group of instantiations is compiled in a translation unit of
// its own (gemm_*.hip), so that the library builds in parallel; gemm.hip dispatches.
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
// K permutation: inside each 128-wide K stage, lane half h of an MFMA operand
// supplies elements h*64 + sub*32 + s*8 + [0, 8) in MFMA step 4*sub + s, for both A
// and B.  One 16-byte LDS read gives a lane the 32 codes of a slice `sub`, and one
// 4-byte read the scale bytes of all four of its blocks in the stage.  Any
// permutation of K applied to both operands leaves the dot product unchanged.
//
// Decoded weights (B given as its exact FP16 values e2m1 * e4m3, GROUP_M only): A stays
// NVFP4 and is decoded as above, B is read from LDS as it is.  Stages of 64 (an FP16 B
// stage of 128 would not fit twice in LDS next to A), 64 x 128 wave tiles so that
// each wave decodes two A fragments per eight MFMAs.  The products are the same; the
// grouping of K in the FP32 sums differs.
//
// BF16 operands (the unquantised layer and the BF16 / dequantized backward of
// "The 4-bitter Lesson", section "Improving Gradient Stability") use the same
// kernel with the decode removed: stages of 32 BF16 elements (64 bytes per row,
// the same LDS layout as a stage of 128 FP4 codes), one 16-byte LDS read per
// fragment row per MFMA step, v_mfma_f32_32x32x16_bf16, no tensor scales.  Tiles
// of 128 x 256 per workgroup (four 64 x 128 wave tiles) with two workgroups per CU,
// so that one workgroup's barrier and load waits overlap the other's MFMAs.
//
// Tile order: the logical tile index is split so that the workgroups of one XCD
// (hardware assigns workgroup i to XCD i % 8) take consecutive tiles, which share
// the A rows (same M tile) and the expert's B matrix in that XCD's L2.
#pragma once

#include <algorithm>
#include <type_traits>

#include "nv4_device.h"
#include "nv4_internal.h"
#include "../../include/nv4moe.h"

namespace nv4 {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kXcds = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int WAVES_M, int WAVES_N, int FM, int FN, int WAVES_PER_SIMD = 1, int STAGES = 2, bool BF16 = false,
          bool WF16 = false>
struct TileCfg {
  static constexpr bool kBf16 = BF16;                   // operands BF16 (else NVFP4)
  static constexpr bool kWf16 = WF16;                   // A NVFP4, B exact FP16 values (decoded weights)
  static constexpr int kWavesM = WAVES_M, kWavesN = WAVES_N, kFM = FM, kFN = FN;
  static constexpr int kWavesPerSimd = WAVES_PER_SIMD;  // occupancy the registers are budgeted for
  static constexpr int kStages = STAGES;                // LDS ring depth (prefetch distance STAGES - 1)
  static constexpr int BM = WAVES_M * FM * 32;
  static constexpr int BN = WAVES_N * FN * 32;  // rows of B per tile
  static constexpr int BK = BF16 ? 32 : (WF16 ? 64 : 128);  // K per LDS stage
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int kRowBytes = BF16 ? BK * 2 : BK / 2;  // A element bytes per row per stage
  static constexpr int kScBytes = BF16 ? 0 : BK / 16;       // A scale bytes per row per stage
  static constexpr int kRowBytesB = (BF16 || WF16) ? BK * 2 : BK / 2;  // B element bytes per row per stage
  static constexpr int kScBytesB = (BF16 || WF16) ? 0 : BK / 16;       // B scale bytes per row per stage
  static constexpr int kStageBytes = BM * (kRowBytes + kScBytes) + BN * (kRowBytesB + kScBytesB);
};

// an index into A taken from the caller: clamp into [0, rows) so that an index
// outside the contract cannot read outside the buffer
__device__ __forceinline__ int64_t min_row(int32_t idx, int64_t rows) {
  return idx < 0 ? 0 : (idx >= rows ? rows - 1 : idx);
}

typedef __attribute__((address_space(3))) void *lds_ptr;
// LDS DMA of N bytes per lane from the raw buffer [base, base + bytes) at byte
// offset voff; lane i lands at dst + i * N.  Reads outside the buffer return zeros.
// (Device-only helper: the buffer-resource type exists only on the GPU target.)
__device__ __forceinline__ void dma16_to_lds(const void *base, uint32_t bytes, uint8_t *dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000), (lds_ptr)dst, 16,
      voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void *base, uint32_t bytes, uint8_t *dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000), (lds_ptr)dst, 4,
      voff, 0, 0, 0);
}

// wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left open)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence waits
// for every outstanding memory operation, including LDS DMA of stages that are
// still being prefetched.  Callers wait explicitly for what they need first.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer stores of one C row: `base` is the row's first byte and `bytes` the part of
// the tile's rows that lies at or after it, so a store whose byte offset falls
// outside [0, bytes) is dropped by the hardware (rows past the tile's valid rows,
// columns flagged invalid by an offset of 2^31).  Device-only helpers: the buffer
// resource type exists only on the GPU target.
// (base and bytes are the same for the whole wave; reading them from the first
// lane keeps the buffer descriptor in scalar registers)
__device__ __forceinline__ void *uniform_ptr(void *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void store_row_b32(void *base, uint32_t bytes, uint32_t voff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(
      __builtin_bit_cast(uint32_t, v),
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                        0x00020000),
      voff, 0, 2);  // non-temporal: FP32 results are read by the next kernel, not here
}
__device__ __forceinline__ void store_row_b16(void *base, uint32_t bytes, uint32_t voff, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(
      v,
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(base), (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                        0x00020000),
      voff, 0, 0);
}
// FP32 -> BF16 bits, round to nearest even (the gfx950 converter)
__device__ __forceinline__ uint16_t bf16_of(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// LDS position of 16-byte chunk q (0..3) of tile row r (rows are 64 bytes).  A
// fragment read has 16 consecutive rows read the same chunk in one LDS pass
// (64 banks of 4 bytes); XOR-ing the chunk with bits 2..3 of the row gives those
// 16 rows 16 distinct (row mod 4, position) bank groups.
__device__ __forceinline__ int swz(int q, int r) { return q ^ ((r >> 2) & 3); }

// A value the whole wave agrees on, as a scalar (lets the compiler keep it, and
// everything derived from it, in scalar registers)
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct TileJob {
  int e;
  bool gather;         // A rows come through the caller's row index
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


// Physical row of A for tile row r (-1 when outside the tile's range).
__device__ __forceinline__ int64_t a_row_of(const GemmArgs &g, const TileJob &job, int r) {
  const int64_t gr = job.m0 + r;
  if (gr >= job.m_end) return -1;
  if (job.gather) return min_row(g.a_rows_index[gr], g.a_rows);
  return gr;
}

// Physical row of B for B-tile row r (-1 when outside N).  With the SwiGLU
// epilogue a wave's FN fragments hold FN/2 gate fragments followed by the FN/2
// up fragments of the same output columns.
template <int GROUP, int EPI, int FN, int BN>
__device__ __forceinline__ int64_t b_row_of(const GemmArgs &g, const TileJob &job, int64_t nt_idx, int r) {
  if (GROUP == NV4_GROUP_K) {
    const int64_t col = job.n0 + r;
    return col < g.b_rows ? col : -1;
  }
  if (EPI == NV4_EPI_SWIGLU) {
    constexpr int half = FN / 2;
    const int wv = r / (FN * 32), f = (r % (FN * 32)) / 32;
    const int64_t col = nt_idx * (BN / 2) + wv * (half * 32) + (f % half) * 32 + (r & 31);
    if (col >= g.N) return -1;
    return (int64_t)job.e * 2 * g.N + (f >= half ? g.N : 0) + col;
  }
  const int64_t col = nt_idx * BN + r;
  return col < g.N ? (int64_t)job.e * g.N + col : -1;
}

// KSPLIT: B carries one decode scale per expert and K half (SCALE_SEGMENT_HALVES, GROUP_M,
// (K/2) % BK == 0): the accumulators hold the first half's products scaled by
// G[2e] / G[2e+1] when the second half starts, and G[2e+1] is applied at the end.
template <class Cfg, int GROUP, int EPI, bool OUT_F32, bool A_ROW_SCALE, bool KSPLIT = false>
__global__ __launch_bounds__(Cfg::kThreads) __attribute__((amdgpu_waves_per_eu(Cfg::kWavesPerSimd)))
void k_gemm(GemmArgs g) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::kThreads, NW = NT / 64;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  constexpr int RB = Cfg::kRowBytes, SB = Cfg::kScBytes;
  // LDS DMA plan: codes in 1 KB blocks of 16 rows, scales in 256-byte blocks of 32
  // rows (A rows first, then B rows); wave w issues blocks w, w + NW, ...
  constexpr bool BF = Cfg::kBf16;
  // WF: A NVFP4 stages of 64 codes (32 bytes, 4 scale bytes per row), B exact FP16
  // values (128 bytes per row); 1 KB DMA blocks of 32 A rows or 8 B rows, A scales in
  // 256-byte blocks of 64 rows
  constexpr bool WF = Cfg::kWf16;
  static_assert(!WF || (GROUP == NV4_GROUP_M && FM == 2 && FN == 4), "FP16 B: GROUP_M, 64 x 128 wave tiles");
  constexpr int kCodeBlocksA = WF ? BM * RB / 1024 : 0;
  constexpr int kCodeBlocks = WF ? kCodeBlocksA + BN * Cfg::kRowBytesB / 1024 : (BM + BN) / 16;
  constexpr int kScBlocks = BF ? 0 : (WF ? BM * SB / 256 : (BM + BN) / 32);
  constexpr int kCodeIters = (kCodeBlocks + NW - 1) / NW;
  constexpr int kScIters = BF ? 1 : (kScBlocks + NW - 1) / NW;
  // DMAs every wave issues per stage (the vmcnt wait uses the smallest count)
  constexpr int kDmaMin = kCodeBlocks / NW + kScBlocks / NW;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile rows must be multiples of 32");
  constexpr int kScBase = WF ? BM * RB + BN * Cfg::kRowBytesB : (BM + BN) * RB;
  constexpr int S = Cfg::kStages;
  static_assert(S >= 2 && S <= 4, "LDS ring of 2 to 4 stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[Cfg::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[Cfg::kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[S > 2 ? Cfg::kStageBytes : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[S > 3 ? Cfg::kStageBytes : 16];
  __shared__ int tstart[kMaxExperts + 1];
  __shared__ int scratch[NT];
  // per-row A scales of the tile (per-token mode), double-buffered by tile parity: a
  // wave writes the next tile's scales while others may still read this tile's
  __shared__ float row_scale[A_ROW_SCALE ? 2 : 1][A_ROW_SCALE ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform over the wave (scalar)
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5, l32 = lane & 31;
  const int E = g.E;
  const int64_t K = g.K;
  const int64_t ldA = BF ? K * 2 : K >> 1, ldAs = K >> 4;  // bytes per row: elements (codes), scales
  const int64_t ldB = (BF || WF) ? K * 2 : K >> 1;          // bytes per B row
  // buffer resources: loads past num_records return zeros (operands are < 4 GiB)
  const uint32_t na_c = (uint32_t)(g.a_rows * ldA), na_s = (uint32_t)(g.a_rows * ldAs);
  const uint32_t nb_c = (uint32_t)(g.b_rows * ldB), nb_s = (uint32_t)(g.b_rows * ldAs);
  const void *b_elems = WF ? static_cast<const void *>(g.b_f16) : static_cast<const void *>(g.b_codes);

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
    if (g.tile_counter) {
      // Dynamic schedule: a tile's work grows with its expert's rows, so workgroups
      // take tiles from a counter, largest experts first (tstart holds the experts in
      // decreasing row count, ties by id).  Every tile is still computed whole by
      // one workgroup, so the result does not depend on which one.
      for (int e = tid; e < E; e += NT) {
        const int n = g.offsets[e + 1] - g.offsets[e];
        int rank = 0;
        for (int f = 0; f < E; ++f) {
          const int m = g.offsets[f + 1] - g.offsets[f];
          rank += (m > n) || (m == n && f < e);
        }
        tstart[rank] = e;
      }
      __syncthreads();
    }
  }
  const int G = gridDim.x;
  const int per_xcd = G / kXcds;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;

  const float a_ts = (!A_ROW_SCALE && !Cfg::kBf16) ? g.a_tscale[0] : 1.0f;
  float amax_run = 0.0f;

  // Dynamic schedule: thread 0 takes the first tile here and, during every tile,
  // the next one; the index travels through an LDS slot that alternates with the
  // iteration (written before the barrier that ends the K loop, read after it, never
  // rewritten while a wave may still read it).
  const bool dyn = GROUP == NV4_GROUP_K && g.tile_counter != nullptr;
  if (dyn) {
    if (tid == 0) scratch[0] = atomicAdd(g.tile_counter, 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slot is written
    block_barrier();
  }
  // ---- epilogue of a finished tile (job ej, column tile en, B scales eg / eu, row
  // scales of iteration eit): tensor scales, optional SwiGLU, store
  constexpr int NJ = EPI == NV4_EPI_SWIGLU ? FN / 2 : FN;
  constexpr int ESZ = OUT_F32 ? 4 : 2;
  f32x16 acc[FM][FN];
  TileJob ej{};
  int64_t en = 0;
  float eg = 1.0f, eu = 1.0f;
  auto epilogue = [&](int64_t eit) {
    const int ldc = (int)g.ldc;
    int colw, ncols;  // first output column of this wave's fragment 0 (before the lane), column count
    if (EPI == NV4_EPI_SWIGLU) {
      colw = (int)en * (BN / 2) + wn * (FN / 2 * 32);
      ncols = (int)g.N;
    } else if (GROUP == NV4_GROUP_M) {
      colw = (int)en * BN + wn * FN * 32;
      ncols = (int)g.N;
    } else {
      colw = (int)ej.n0 + wn * FN * 32;
      ncols = (int)g.b_rows;
    }
    const int rows_valid = (int)std::min<int64_t>(ej.m_end - ej.m0, BM) - wm * FM * 32;
    // this wave's rows start at tile row wm*FM*32; lane half h adds 4 rows
    char *cw = static_cast<char *>(g.C) +
               ((int64_t)(GROUP == NV4_GROUP_K ? ej.e * g.a_rows : 0) + ej.m0 + wm * FM * 32) * g.ldc * ESZ;
    // lane offsets: row q (0..3) of a 4-row group plus 4 rows for lane half h, column
    // of fragment j (an invalid column gets an offset past any buffer)
    uint32_t voff[4][NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = colw + j * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        voff[q][j] = col < ncols ? (uint32_t)(((q + h * 4) * ldc + col) * ESZ) : 0x80000000u;
    }
    const float sc = a_ts * eg, sc_up = a_ts * eu;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ru = i * 32 + g4 * 8;  // first row of the group for lane half 0
        // bytes from row ru to the end of the valid rows, at most 8 rows (the group's
        // offsets stay below 8 rows)
        const int left = std::min(std::max(rows_valid - ru, 0), 8);
        char *rb = cw + (int64_t)ru * g.ldc * ESZ;
        const uint32_t nb = (uint32_t)(left * ldc * ESZ);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = g4 * 4 + q;
          float rsc = sc, rsc_up = sc_up;
          if (A_ROW_SCALE) {
            const float ra = row_scale[eit & 1][wm * FM * 32 + ru + q + h * 4];
            rsc = ra * eg;
            rsc_up = ra * eu;
          }
          if (EPI == NV4_EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              const float gt = acc[i][j][r] * rsc;
              const float up = acc[i][j + FN / 2][r] * rsc_up;
              // silu(g) * u with the hardware exp2 and reciprocal (relative error ~1e-7)
              const float hv = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
              float stored;
              if (OUT_F32) {
                store_row_b32(rb, nb, voff[q][j], hv);
                stored = hv;
              } else {
                const uint16_t b16 = bf16_of(hv);
                store_row_b16(rb, nb, voff[q][j], b16);
                stored = bf16_bits_to_f32(b16);
              }
              // rows and columns outside the tile hold exact zeros (zero operands)
              amax_run = fmaxf(amax_run, fabsf(stored));
            }
          } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              const float v = acc[i][j][r] * rsc;
              if (OUT_F32) store_row_b32(rb, nb, voff[q][j], v);
              else store_row_b16(rb, nb, voff[q][j], bf16_of(v));
            }
          }
        }
      }
    }
  };
  // FP32 GROUP_M outputs (the down projection: K = I, six stages of 128 per tile, then
  // 256 KB of stores) issue a tile's C stores in the next iteration, after the next
  // tile's first LDS DMA, so that they drain while its first stage computes (GEMM2
  // 4 % faster on the learner batch; the BF16-output GEMMs were 0.5-2.5 % slower that
  // way and keep the stores at the end of the tile).
  constexpr bool kLate = OUT_F32 && GROUP == NV4_GROUP_M;
  constexpr int kEpiStores = FM * 16 * NJ;  // buffer stores every wave issues per tile
  constexpr int kPostEpiWait = kEpiStores < 63 ? kEpiStores : 63;
  for (int64_t it = 0;; ++it) {
    const int64_t L = dyn ? (int64_t)__builtin_amdgcn_readfirstlane(scratch[it & 1])
                          : it * G + (int64_t)xcd * per_xcd + slot;
    const bool have = L < total;  // uniform
    if (!kLate && !have) break;
    int next_tile = 0;
    if (have && dyn && tid == 0) next_tile = atomicAdd(g.tile_counter, 1);
    TileJob job{};  // with no tile: an empty K range, no DMA, rows that load nothing
    int64_t nt_idx = 0;
    if (!have) {
    } else if (GROUP == NV4_GROUP_M) {
      const int64_t mt = L / ntn;
      nt_idx = L - mt * ntn;
      int lo = 0, hi = E - 1;  // last expert with tstart[e] <= mt (it owns >= 1 tile)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tstart[mid] <= mt) lo = mid; else hi = mid - 1;
      }
      job.e = lo;
      job.m0 = g.offsets[lo] + (mt - tstart[lo]) * BM;
      job.m_end = std::min<int64_t>(g.offsets[lo + 1], g.M_cap);  // never past the caller's C rows
      job.n0 = nt_idx;
      job.k_lo = 0;
      job.k_hi = K;
      job.gather = g.a_rows_index != nullptr;
    } else {
      job.gather = false;
      const int tn = (int)((g.a_rows + BM - 1) / BM);
      const int64_t per_e = (int64_t)tn * ntn;
      const int rank = (int)(L / per_e);
      job.e = g.tile_counter ? tstart[rank] : rank;
      const int64_t r = L - (int64_t)rank * per_e;
      const int64_t tni = r / ntn;
      nt_idx = r - tni * ntn;
      job.m0 = tni * BM;
      job.m_end = g.a_rows;
      job.n0 = nt_idx * BN;
      job.k_lo = g.offsets[job.e];
      job.k_hi = g.offsets[job.e + 1];
    }
    // the tile is the same for the whole wave (the expert search read LDS)
    job.e = __builtin_amdgcn_readfirstlane(job.e);
    job.m0 = uniform64(job.m0);
    job.m_end = uniform64(job.m_end);
    job.n0 = uniform64(job.n0);
    job.k_lo = uniform64(job.k_lo);
    job.k_hi = uniform64(job.k_hi);
    nt_idx = uniform64(nt_idx);

    if (A_ROW_SCALE) {
      // the tile's row scales, fetched now so that the epilogue reads them from LDS
      // (every wave's writes are complete by the barrier that ends the K loop)
      for (int t = tid; t < BM; t += NT) {
        const int64_t grow = job.m0 + t;
        float v = 0.0f;
        if (grow < job.m_end) v = g.a_tscale[job.gather ? min_row(g.a_rows_index[grow], g.a_rows) : grow];
        row_scale[it & 1][t] = v;
      }
    }

    // ---- this lane's DMA sources: byte offsets into the operand; rows outside the
    // tile's range point past the end of the operand, so they load as zeros.
    uint32_t c_off[kCodeIters];
#pragma unroll
    for (int j = 0; j < kCodeIters; ++j) {
      if constexpr (WF) {
        const int blk = j * NW + wave;
        if (blk < kCodeBlocksA) {  // 32 A rows of 32 code bytes: lane -> row lane/2, chunk lane%2
          const int r = blk * 32 + (lane >> 1);
          const int64_t pr = a_row_of(g, job, r);
          c_off[j] = pr >= 0 ? (uint32_t)(pr * ldA) + (lane & 1) * 16 : na_c;
        } else {  // 8 B rows of 128 value bytes; the lane's slot holds chunk slot ^ (row % 8)
          const int r = (blk - kCodeBlocksA) * 8 + (lane >> 3);
          const int q = (lane & 7) ^ (r & 7);
          int64_t pr = -1;
          if (r < BN) pr = b_row_of<GROUP, EPI, FN, BN>(g, job, nt_idx, r);
          c_off[j] = pr >= 0 ? (uint32_t)(pr * ldB) + q * 16 : nb_c;
        }
      } else {
        const int row = (j * NW + wave) * 16 + (lane >> 2);
        const bool isA = row < BM;  // uniform over the wave
        const int r = isA ? row : row - BM;
        const int q = swz(lane & 3, r);  // chunk that lands in this lane's slot (swz is its own inverse)
        int64_t pr = -1;
        if (row < BM + BN) pr = isA ? a_row_of(g, job, r) : b_row_of<GROUP, EPI, FN, BN>(g, job, nt_idx, r);
        c_off[j] = pr >= 0 ? (uint32_t)(pr * ldA) + q * 16 : (isA ? na_c : nb_c);
      }
    }
    uint32_t s_off[kScIters];
#pragma unroll
    for (int j = 0; j < (BF ? 0 : kScIters); ++j) {
      if constexpr (WF) {  // 64 A rows of 4 scale bytes
        const int r = (j * NW + wave) * 64 + lane;
        int64_t pr = -1;
        if (r < BM) pr = a_row_of(g, job, r);
        s_off[j] = pr >= 0 ? (uint32_t)(pr * ldAs) : na_s;
      } else {
        const int row = (j * NW + wave) * 32 + (lane >> 1);
        const bool isA = row < BM;
        const int r = isA ? row : row - BM;
        int64_t pr = -1;
        if (row < BM + BN) pr = isA ? a_row_of(g, job, r) : b_row_of<GROUP, EPI, FN, BN>(g, job, nt_idx, r);
        s_off[j] = pr >= 0 ? (uint32_t)(pr * ldAs) + (lane & 1) * 4 : (isA ? na_s : nb_s);
      }
    }

    // ---- K range in stages of BK (stage starts 128-aligned; blocks outside
    // [k_lo, k_hi) get scale 0 when read, so they contribute nothing)
    const int64_t kb0 = (job.k_lo / BK) * BK;
    const int nk = job.k_hi > job.k_lo ? (int)((job.k_hi - kb0 + BK - 1) / BK) : 0;

    auto issue = [&](int kt, uint8_t *dst) {
      // element (code) byte offset of the stage
      const uint32_t kc = (uint32_t)(BF ? (kb0 + (int64_t)kt * BK) * 2 : (kb0 + (int64_t)kt * BK) >> 1);
      const uint32_t kcb = WF ? (uint32_t)((kb0 + (int64_t)kt * BK) * 2) : kc;  // B element byte offset
      const uint32_t ks = (uint32_t)((kb0 + (int64_t)kt * BK) >> 4);  // scale byte offset of the stage
#pragma unroll
      for (int j = 0; j < kCodeIters; ++j) {
        const int blk = j * NW + wave;
        if (kCodeBlocks % NW != 0 && blk >= kCodeBlocks) break;
        const bool isA = WF ? blk < kCodeBlocksA : blk * 16 < BM;
        // a chunk past the row end reads the next row (finite codes); the scale
        // mask in compute() zeroes those blocks.  Past the operand's end the buffer
        // returns zeros.
        if (isA) dma16_to_lds(g.a_codes, na_c, dst + blk * 1024, c_off[j] + kc);
        else dma16_to_lds(b_elems, nb_c, dst + blk * 1024, c_off[j] + kcb);
      }
#pragma unroll
      for (int j = 0; j < (BF ? 0 : kScIters); ++j) {
        const int blk = j * NW + wave;
        if (kScBlocks % NW != 0 && blk >= kScBlocks) break;
        const bool isA = WF || blk * 32 < BM;
        if (isA) dma4_to_lds(g.a_scales, na_s, dst + kScBase + blk * 256, s_off[j] + ks);
        else dma4_to_lds(g.b_scales, nb_s, dst + kScBase + blk * 256, s_off[j] + ks);
      }
    };

    // B decode scales of this tile (the same for every column of a tile): per tensor;
    // per expert; gate and up of the expert (SwiGLU with 2E segments); or the two K
    // halves of the expert (KSPLIT, applied as a ratio at K/2 and b_gate at the end)
    float b_gate = 1.0f, b_up = 1.0f, k_ratio = 1.0f;
    if (!BF) {
      if (GROUP == NV4_GROUP_K || g.b_scale_mode == NV4_SCALE_TENSOR) {
        b_gate = b_up = g.b_tscale[0];
      } else if (KSPLIT) {
        const float g0 = g.b_tscale[2 * job.e], g1 = g.b_tscale[2 * job.e + 1];
        b_gate = b_up = g1;
        k_ratio = __fdiv_rn(g0, g1);
      } else if (EPI == NV4_EPI_SWIGLU && g.b_nseg == 2 * E) {
        b_gate = g.b_tscale[2 * job.e];
        b_up = g.b_tscale[2 * job.e + 1];
      } else {
        b_gate = b_up = g.b_tscale[job.e];
      }
    }

    // LDS stage layout: a row holds the stage's 128 codes in four XOR-swizzled
    // 16-byte chunks and its 8 scale bytes.  Lane half h takes stage elements
    // h*64 + [0, 64): slice `sub` is chunk 2h + sub (32 codes, one 16-byte read) and
    // scale bytes 4h + 2 sub + {0, 1}; MFMA step t = sub*4 + s consumes dword s of
    // the slice with the scale of block s/2.
    // FP16 B (WF): stages of 64; A as one slice (lane half h: elements h*32 + [0, 32), one
    // 16-byte read, scale bytes 2h and 2h + 1); MFMA step s takes elements h*32 + s*8 +
    // [0, 8) of both operands, for B one 16-byte read of chunk 4h + s of the fragment
    // row (chunks XOR-permuted by the row's low three bits).
    constexpr int kSubs = BF ? 1 : BK / 64, kSteps = BK / 16;  // (NVFP4 only)
    static_assert(BF || (WF ? kSubs == 1 : kSubs == 2), "NVFP4 stages of 128 codes (64 with FP16 B)");
    const uint8_t *lds_cur = lds0;  // the stage being computed (FP16 B is read step by step)
    uint4 ca[kSubs][FM], cb[kSubs][FN];
    f16x2 sa[kSubs][FM], sbv[kSubs][FN];
    // per-lane byte offsets inside a stage: the lane's fragment row (l32 of the
    // wave's first fragment), its chunk of each slice, its 4 scale bytes; fragment i
    // adds the constant i*32 rows.  The swizzle of row r depends on r & 12 only,
    // that is on l32.
    const int rowA = wm * FM * 32 + l32, rowB = BM + wn * FN * 32 + l32;
    const int ch0 = swz(2 * h, l32) * 16, ch1 = swz(2 * h + 1, l32) * 16;
    const int offA = rowA * RB, offB = rowB * RB;
    const int soffA = kScBase + rowA * SB + 4 * h, soffB = kScBase + rowB * SB + 4 * h;
    auto lds_read = [&](const uint8_t *base, int kt, auto full_c) {
      constexpr bool kFull = decltype(full_c)::value;
      if constexpr (WF) {  // full stages only (K % 64 == 0, GROUP_M)
        const int rA = wm * FM * 32 + l32;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          ca[0][i] = *reinterpret_cast<const uint4 *>(base + (rA + i * 32) * RB + h * 16);
          const uint32_t s4 = *reinterpret_cast<const uint32_t *>(base + kScBase + (rA + i * 32) * SB);
          sa[0][i] = e4m3x2_to_f16<false>(s4 >> (16 * h));
        }
      } else {
        // scale-byte mask of this lane's four blocks (k0 + h*64 + b*16, b = 0..3) when
        // the stage is partial: blocks outside [k_lo, k_hi) decode to zero
        uint32_t smask = 0xFFFFFFFFu;
        if (!kFull) {
          const int64_t kb = kb0 + (int64_t)kt * BK + h * 64;
          smask = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (kb + 16 * b >= job.k_lo && kb + 16 * b < job.k_hi) smask |= 0xFFu << (8 * b);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          ca[0][i] = *reinterpret_cast<const uint4 *>(base + offA + i * 32 * RB + ch0);
          ca[1][i] = *reinterpret_cast<const uint4 *>(base + offA + i * 32 * RB + ch1);
          uint32_t s4 = *reinterpret_cast<const uint32_t *>(base + soffA + i * 32 * SB);
          if (!kFull) s4 &= smask;
          sa[0][i] = e4m3x2_to_f16<false>(s4);
          sa[1][i] = e4m3x2_to_f16<true>(s4);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          cb[0][j] = *reinterpret_cast<const uint4 *>(base + offB + j * 32 * RB + ch0);
          cb[1][j] = *reinterpret_cast<const uint4 *>(base + offB + j * 32 * RB + ch1);
          uint32_t s4 = *reinterpret_cast<const uint32_t *>(base + soffB + j * 32 * SB);
          if (!kFull) s4 &= smask;
          sbv[0][j] = e4m3x2_to_f16<false>(s4);
          sbv[1][j] = e4m3x2_to_f16<true>(s4);
        }
      }
    };
    // FP16 B: A fragments of MFMA step st decoded, B fragments read as they are
    auto decode_a = [&](int st, f16x8 (&av)[FM]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t w = st == 0 ? ca[0][i].x : st == 1 ? ca[0][i].y : st == 2 ? ca[0][i].z : ca[0][i].w;
        const f16x2 sc = st < 2 ? __builtin_shufflevector(sa[0][i], sa[0][i], 0, 0)
                                : __builtin_shufflevector(sa[0][i], sa[0][i], 1, 1);
        av[i] = decode8_f16(w, sc);
      }
    };
    auto read_b = [&](int st, f16x8 (&bv)[FN]) {
      const uint8_t *bb = lds_cur + BM * RB;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * FN * 32 + j * 32 + l32;
        bv[j] = *reinterpret_cast<const f16x8 *>(bb + row * Cfg::kRowBytesB + (((4 * h + st) ^ (l32 & 7)) << 4));
      }
    };
    auto decode = [&](int t, f16x8 (&av)[FM], f16x8 (&bv)[FN]) {
      const int sub = t >> 2, st = t & 3;
      if constexpr (WF) {
        decode_a(st, av);
        read_b(st, bv);
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const uint32_t w = st == 0 ? ca[sub][i].x : st == 1 ? ca[sub][i].y : st == 2 ? ca[sub][i].z : ca[sub][i].w;
          const f16x2 sc = st < 2 ? __builtin_shufflevector(sa[sub][i], sa[sub][i], 0, 0)
                                  : __builtin_shufflevector(sa[sub][i], sa[sub][i], 1, 1);
          av[i] = decode8_f16(w, sc);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t w = st == 0 ? cb[sub][j].x : st == 1 ? cb[sub][j].y : st == 2 ? cb[sub][j].z : cb[sub][j].w;
          const f16x2 sc = st < 2 ? __builtin_shufflevector(sbv[sub][j], sbv[sub][j], 0, 0)
                                  : __builtin_shufflevector(sbv[sub][j], sbv[sub][j], 1, 1);
          bv[j] = decode8_f16(w, sc);
        }
      }
    };
    auto mfmas = [&](const f16x8 (&av)[FM], const f16x8 (&bv)[FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    };
    // BF16: MFMA step t of a stage takes 16 elements; lane half h supplies
    // elements t*16 + h*8 + [0, 8), 16-byte chunk 2t + h of the row.  An 8-element
    // group outside [k_lo, k_hi) is zeroed in both operands (ranges are 16-aligned,
    // so a group is either wholly inside or wholly outside).
    auto bf16_stage = [&](const uint8_t *base, int kt) {
      const int64_t k0 = kb0 + (int64_t)kt * BK;
      const bool full = k0 >= job.k_lo && k0 + BK <= job.k_hi;
      constexpr int kStepsBf = BK / 16;
#pragma unroll
      for (int t = 0; t < kStepsBf; ++t) {
        bf16x8 av[FM], bv[FN];
        const int q = 2 * t + h;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * FM * 32 + i * 32 + l32;
          av[i] = *reinterpret_cast<const bf16x8 *>(base + row * RB + swz(q, row) * 16);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * FN * 32 + j * 32 + l32;
          bv[j] = *reinterpret_cast<const bf16x8 *>(base + BM * RB + row * RB + swz(q, row) * 16);
        }
        if (!full) {
          const int64_t kb = k0 + t * 16 + h * 8;
          if (!(kb >= job.k_lo && kb < job.k_hi)) {
            const bf16x8 z = {};
#pragma unroll
            for (int i = 0; i < FM; ++i) av[i] = z;
#pragma unroll
            for (int j = 0; j < FN; ++j) bv[j] = z;
          }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    };
    // wait until this wave's LDS DMA of stage `need` is done, given that `after`
    // more stages were issued after it
    auto wait_stage = [&](int after) {
      if (after >= 2) wait_vmcnt<2 * kDmaMin>();
      else if (after == 1) wait_vmcnt<kDmaMin>();
      else wait_vmcnt<0>();
    };
    auto bufp = [&](int b) -> uint8_t * { return b == 0 ? lds0 : b == 1 ? lds1 : b == 2 ? lds2 : lds3; };

    // K loop over an LDS ring of S stages (stage kt+S-1 streams in by LDS DMA while
    // stage kt is computed); unrolled by S so that every buffer is a fixed LDS object.
    for (int s0 = 0; s0 < S - 1; ++s0)
      if (s0 < nk) issue(s0, bufp(s0));
    if constexpr (kLate) {
      // the previous tile's C stores follow this tile's first DMA in issue order
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (it > 0) epilogue(it - 1);
      if (!have) break;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    {
      auto stage = [&](const int B, int kt) {  // B = kt % S, a literal at every call
        // A wave's vector-memory operations retire in issue order (loads, LDS DMA and
        // stores alike, one vmcnt).  With kLate, stage 0 of a tile after the first was
        // issued before the previous tile's kEpiStores C stores: waiting until at most
        // that many operations are outstanding leaves the stores in flight.
        if (kLate && S == 2 && kt == 0 && it > 0) wait_vmcnt<kPostEpiWait>();
        else wait_stage(std::min(S - 2, nk - 1 - kt));
        block_barrier();
        if (kt + S - 1 < nk) issue(kt + S - 1, bufp((B + S - 1) % S));
        const uint8_t *base = bufp(B);
        lds_cur = base;
        if constexpr (BF) {
          bf16_stage(base, kt);
        } else {
          const int64_t k0 = kb0 + (int64_t)kt * BK;
          if (WF || (k0 >= job.k_lo && k0 + BK <= job.k_hi)) lds_read(base, kt, std::true_type{});
          else lds_read(base, kt, std::false_type{});
          if constexpr (WF) {
            // FP16 B: step t+1's B fragments are read into a second set of registers
            // before step t's MFMAs are issued
            f16x8 av[FM], bv[FN], bn[FN];
            decode(0, av, bv);
#pragma unroll
            for (int t = 0; t < kSteps; ++t) {
              if (t + 1 < kSteps) read_b(t + 1, bn);
              mfmas(av, bv);
              if (t + 1 < kSteps) {
                decode_a(t + 1, av);
#pragma unroll
                for (int j = 0; j < FN; ++j) bv[j] = bn[j];
              }
            }
          } else {
#pragma unroll
            for (int t = 0; t < kSteps; ++t) {
              f16x8 av[FM], bv[FN];
              decode(t, av, bv);
              mfmas(av, bv);
            }
          }
          // Instruction order of the stage: the first step's decode, then every MFMA
          // followed by an even share of the later steps' decode, so that a wave
          // decodes the next step while its own MFMAs run (the compiler otherwise
          // groups each step's MFMAs after its whole decode).
          constexpr int kMf = kSteps * FM * FN, kDec = (WF ? FM : FM + FN) * 8;  // decode VALU per step
          if constexpr (WF) {
            // FP16 B: the stage's A reads and step 0's B reads, step 0's decode; then per
            // step its MFMAs, the next step's B reads right after the first of them and
            // the next step's decode spread over the rest
            constexpr int kMs = FM * FN, kPerW = (kDec + kMs - 2) / (kMs - 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * FM + FN, 0);  // DS reads
            __builtin_amdgcn_sched_group_barrier(0x002, kDec, 0);         // VALU
#pragma unroll
            for (int t = 0; t < kSteps; ++t) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              if (t + 1 < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, FN, 0);
#pragma unroll
              for (int i = 1; i < kMs; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (t + 1 < kSteps) __builtin_amdgcn_sched_group_barrier(0x002, kPerW, 0);
              }
            }
          } else {
            constexpr int kPer = (kDec * (kSteps - 1) + kMf - 1) / kMf;
            __builtin_amdgcn_sched_group_barrier(0x002, kDec, 0);  // VALU
#pragma unroll
            for (int i = 0; i < kMf; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, kPer, 0);  // VALU
            }
          }
        }
      };
      // KSPLIT: the first K half's accumulators times G[2e] / G[2e+1]
      auto rescale = [&]() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] *= k_ratio;
      };
      if constexpr (S == 2) {
        // pairs of stages with no branch between them, then the odd stage: with a
        // conditional second stage the accumulators were copied between registers
        // on every iteration.  Stage kt is in buffer kt % 2.  KSPLIT rescales the
        // accumulators once, before the first stage of the second K half.
        const int nks = KSPLIT ? (int)((K >> 1) / BK) : -1;  // first stage of the second K half
        int kt = 0;
        if (KSPLIT && (nks & 1) == 0) {
          // the K halves meet between two pairs of stages: one loop over each half's
          // pairs, the rescale between them (1-2 % faster than a test in the loop)
          for (; kt < nks; kt += 2) {
            stage(0, kt);
            stage(1, kt + 1);
          }
          rescale();
          for (; kt + 1 < nk; kt += 2) {
            stage(0, kt);
            stage(1, kt + 1);
          }
        } else {
          for (; kt + 1 < nk; kt += 2) {
            if (KSPLIT && kt == nks) rescale();
            stage(0, kt);
            if (KSPLIT && kt + 1 == nks) rescale();
            stage(1, kt + 1);
          }
        }
        if (kt < nk) {
          if (KSPLIT && kt == nks) rescale();
          stage(0, kt);
        }
      } else {
        const int nks = KSPLIT ? (int)((K >> 1) / BK) : -1;  // first stage of the second K half
        for (int kt = 0; kt < nk; kt += S) {
          if (KSPLIT && kt == nks) rescale();
          stage(0, kt);
          if (KSPLIT && kt + 1 == nks) rescale();
          if (kt + 1 < nk) stage(1, kt + 1);
          if (KSPLIT && S > 2 && kt + 2 == nks) rescale();
          if (S > 2 && kt + 2 < nk) stage(2 % S, kt + 2);
          if (KSPLIT && S > 3 && kt + 3 == nks) rescale();
          if (S > 3 && kt + 3 < nk) stage(3 % S, kt + 3);
        }
      }
    }
    // every LDS read of this tile has been consumed; the next tile refills the ring
    if (dyn && tid == 0) scratch[(it + 1) & 1] = next_tile;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    block_barrier();

    ej = job;
    en = nt_idx;
    eg = b_gate;
    eu = b_up;
    if constexpr (!kLate) epilogue(it);
  }
  if (EPI == NV4_EPI_SWIGLU && g.amax_out) {
    // one atomic per workgroup: the waves' maxima meet in LDS first (same-address
    // atomics serialise in L2, and every workgroup ends at about the same time)
    __shared__ float wave_amax[NW];
    const float w = wave_max(amax_run);
    if (lane == 0) wave_amax[wave] = w;
    __syncthreads();
    if (tid == 0) {
      float m = wave_amax[0];
#pragma unroll
      for (int i = 1; i < NW; ++i) m = fmaxf(m, wave_amax[i]);
      atomic_max_nonneg(g.amax_out, m);
    }
  }
}

// NVFP4 tiles: every wave computes 128 x 64 with two waves per SIMD, so that one
// wave's FP16 decode overlaps the other's MFMAs; double-buffered LDS stages.
// Both group modes use 256 x 256 per workgroup, eight waves (one workgroup per
// CU): the larger tile halves the operand bytes each MFMA pulls through L2.
// (Measured on the learner batch against 128 x 256 with four waves: the GROUP_M
// GEMMs 3-5 % faster.  With the interleaved stage order, the weight gradients are
// 5-19 % faster than with 256 x 128 tiles of four waves, two workgroups per CU.)
using GemmTile = TileCfg<2, 4, 4, 2, 2, 2>;
using GemmTileK = GemmTile;
// Problems with few 256 x 256 tiles (a single dense GEMM of 8192 x 768 outputs has 96 of
// them for 256 compute units): 128 x 256 workgroup tiles of eight 64 x 64 wave tiles,
// twice the tiles at 8 instead of 6 decode instructions per MFMA.
using GemmTileSmall = TileCfg<2, 4, 2, 2, 2, 2>;
// NVFP4 A, exact FP16 B (decoded weights): 256 x 256 workgroup tiles of eight 64 x 128
// wave tiles (two A fragments decoded per eight MFMAs, B read from LDS as it is),
// stages of 64 (41 KB: 256 A rows of 32 code and 4 scale bytes, 256 B rows of 128
// bytes), double buffered.
using GemmTileWf16 = TileCfg<4, 2, 2, 4, 2, 2, false, true>;
// BF16 operands: 128 x 256 workgroup tiles of four 64 x 128 wave tiles, two
// workgroups per CU, double-buffered 24 KB stages.  (Measured on the learner
// batch: 15-25 % faster than 256 x 256 tiles with one workgroup per CU, whether
// of four 128 x 128 or eight 128 x 64 wave tiles.)
using GemmTileBf16 = TileCfg<2, 2, 2, 4, 2, 2, true>;

// clears the dynamic schedule's tile counter before a launch (a kernel, so that the
// step can be captured into a graph)
__global__ void k_zero_counter(int32_t *p) {
  const int i = threadIdx.x;
  if (i == 0) p[i] = 0;
}

template <int GROUP, int EPI, bool OUT_F32, bool ROWS, class Cfg = GemmTile, bool KSPLIT = false>
hipError_t launch_tile(const GemmArgs &g, hipStream_t stream) {
  if (GROUP == NV4_GROUP_K && g.tile_counter) k_zero_counter<<<1, 64, 0, stream>>>(g.tile_counter);
  const int cus = device_cu_count();
  // resident workgroups per CU: enough for kWavesPerSimd waves on every SIMD (one
  // eight-wave NVFP4 workgroup, two four-wave BF16 workgroups)
  int grid = cus * Cfg::kWavesPerSimd * 4 / (Cfg::kThreads / 64);
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  k_gemm<Cfg, GROUP, EPI, OUT_F32, ROWS, KSPLIT><<<grid, Cfg::kThreads, 0, stream>>>(g);
  return hipGetLastError();
}

}  // namespace
}  // namespace nv4
