/* fp8bq probes: measurements of gfx950's FP8 matrix instruction that the
 * block-scaled GEMM's design rests on (libfp8bq_probe.so). Not part of the
 * GEMM path; the status codes and error conventions are those of fp8bq.h
 * (validation on the host before any HIP call, a status return,
 * fp8bq_probe_last_error() for the message). Every pointer is device memory
 * owned by the caller; calls enqueue on `stream` (a hipStream_t, NULL for the
 * default stream) and return after the launch.
 */
#ifndef FP8BQ_PROBE_H
#define FP8BQ_PROBE_H

#include <stdint.h>

#include "fp8bq.h"

#ifdef __cplusplus
extern "C" {
#endif

const char* fp8bq_probe_last_error(void);

/* Accumulation inside the matrix unit against promotion to FP32. The
 * DeepSeek-V3 report (Chinese translation), section 3.3.2 "increasing
 * accumulation precision", measures a maximum relative error near 2% when FP8
 * products of two random matrices with K = 4096 are accumulated inside the
 * H800 tensor cores, and promotes every N_C = 128 K-elements into FP32
 * registers; section 3.5.2 puts the accumulator at about 14 bits.
 *
 * a, b      E4M3 codes [16, k], row-major, k contiguous (16-byte aligned).
 * k         multiple of 128, at most 2^24.
 * chained   float [16, 16]: chained[i*16 + j] = sum_k a[i][k] b[j][k] computed
 *           by k/128 FP8 matrix instructions (16x16x128) each adding into the
 *           previous one's FP32 result (no promotion).
 * promoted  float [16, 16]: the same sum, each 128-K chunk a fresh instruction
 *           whose result is added in FP32 by the vector ALU (the GEMM's
 *           promotion with unit scales).
 * Errors: E_INVAL null pointer, E_SHAPE bad k, E_ALIGN, E_DEVICE, E_HIP. */
int fp8bq_probe_mfma_accum(const void* a, const void* b, int64_t k, float* chained, float* promoted,
                           void* stream);

/* One FP8 matrix instruction (v_mfma_f32_16x16x128_f8f6f4, E4M3 operands, no
 * block scales) on given inputs: d[i*16 + j] = c[i*16 + j] + sum_{k<128}
 * a[i][k] b[j][k] as the hardware evaluates it. a, b E4M3 [16, 128]
 * (16-byte aligned); c, d float [16, 16]. For crafted inputs that show how the
 * unit sums the 128 exact products. Errors as above. */
int fp8bq_probe_mfma_once(const void* a, const void* b, const float* c, float* d, void* stream);

/* Matrix-unit stream with or without the promotion FMAs: `workgroups`
 * workgroups of eight waves (two per SIMD), each wave issuing iters x 32
 * independent 16x16x128 FP8 instructions on register-resident fragments read
 * once from `codes`; with fold != 0 every result is also added into an FP32
 * accumulator with a per-row scale (four FMAs per instruction, three
 * instructions later), as the exact-scale GEMM promotes. The matrix unit is
 * kept busy in both cases, so the difference in time is the shader clock the
 * chip holds under each load.
 *
 * codes     4 MiB of E4M3 codes (at least 4194304 bytes, 16-byte aligned).
 * scales    64 floats.
 * sink      float [workgroups * 512]: keeps the results live.
 * ticks     uint64 [2 * workgroups]: per workgroup, s_memtime and
 *           s_memrealtime ticks between the loop's start and end.
 * Errors: E_INVAL null pointer, iters outside [1, 2^24], workgroups outside
 * [1, 4096]; E_ALIGN, E_DEVICE, E_HIP. */
int fp8bq_probe_mfma_stream(int fold, int64_t iters, int32_t workgroups, const void* codes, const float* scales,
                            float* sink, unsigned long long* ticks, void* stream);

/* Streaming ceiling of the quantisers' memory traffic: reads n bf16 (2n bytes)
 * from src and writes n bytes to dst (the high byte of each bf16), 32 bytes read
 * and 16 written per lane, nothing else. The quantisers move the same bytes per
 * element (plus 4 per 128-element tile), so its rate on a cold (MALL-evicted)
 * input is the ceiling their GB/s is compared with.
 * src, dst  device, 16-byte aligned, not overlapping; n a multiple of 16.
 * Errors: E_INVAL null pointer, E_SHAPE bad n, E_ALIGN, E_DEVICE, E_HIP. */
int fp8bq_probe_stream_2to1(const void* src, void* dst, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BQ_PROBE_H */
