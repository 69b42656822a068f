/*
 * nv4moe_bench.h -- measurement kernels of libnv4moe.so: the achievable HBM stream
 * rates and FP16 matrix-instruction rate of the device, against which the
 * expert path's memory-bound kernels (quantisers, combine) and its grouped GEMMs
 * are judged besides the published peaks.  [LBP] "Low-Bit Precision Training Is
 * Ready for Production ...", section "Throughput Gains and the Conditions That
 * Produce Them": whether a kernel gains from 4-bit data depends on whether it is
 * bound by arithmetic or by memory movement.
 *
 * These calls compute nothing of the method.  All pointers are device pointers
 * owned by the caller; `stream` is a hipStream_t; every call only enqueues one
 * kernel and returns NV4_EINVAL / NV4_EALIGN for bad arguments (nothing enqueued)
 * or NV4_EHIP when the launch fails.
 */
#ifndef NV4MOE_BENCH_H
#define NV4MOE_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "nv4moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Copy `bytes` (a positive multiple of 16) from src to dst with 16-byte
 * non-temporal loads and stores (src and dst 16-byte aligned, not overlapping):
 * 2 * bytes of HBM traffic. */
nv4_status nv4_bench_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Read `bytes` (a positive multiple of 16) of src with 16-byte non-temporal loads.
 * The XOR of all words is written to sink[0] only if it equals `never`, so a
 * caller that passes a value the data cannot produce gets a pure read stream. */
nv4_status nv4_bench_read(const void *src, size_t bytes, uint32_t never, uint32_t *sink, void *stream);

/* Write `bytes` (a positive multiple of 16) of dst with 16-byte ordinary stores, dst
 * 16-byte aligned: `bytes` of HBM write traffic. */
nv4_status nv4_bench_write(void *dst, size_t bytes, void *stream);

/* Read `bytes` (a positive multiple of 4096) of src and write bytes / 4 to dst, a
 * quantiser's 4:1 read:write mix (BF16 in, FP4 codes out), with 16-byte non-temporal
 * loads and stores: 1.25 * bytes of HBM traffic. */
nv4_status nv4_bench_mix(const void *src, size_t bytes, void *dst, void *stream);

/* A loop of `iters` x 8 independent v_mfma_f32_32x32x16_f16 per wave (32768 FLOP
 * each), with waves_per_simd (1 or 2) waves on every SIMD of every compute unit
 * and no memory traffic in the loop.  `out` receives one float per lane:
 * nv4_bench_mfma_out_floats(waves_per_simd) of them.  FLOPs of one call:
 * nv4_bench_mfma_out_floats(w) / 64 * iters * 8 * 32768. */
size_t nv4_bench_mfma_out_floats(int waves_per_simd);
nv4_status nv4_bench_mfma(float *out, int iters, int waves_per_simd, void *stream);

/* Two workgroups of 256 threads per compute unit, each filling a 64 KB LDS buffer and
 * then reading it `iters` x 8 times per lane with 16-byte reads (every wave reads
 * 1 KB of consecutive bytes per instruction, so no bank conflicts).  `out` receives
 * one word per thread: nv4_bench_lds_out_words() of them.  LDS bytes read per call:
 * nv4_bench_lds_out_words() * iters * 8 * 16. */
size_t nv4_bench_lds_out_words(void);
nv4_status nv4_bench_lds(uint32_t *out, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NV4MOE_BENCH_H */
