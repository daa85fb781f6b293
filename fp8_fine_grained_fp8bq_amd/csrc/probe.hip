// Measurement probes of gfx950's FP8 matrix instruction (libfp8bq_probe.so),
// declared in include/fp8bq_probe.h. They are not part of the GEMM path: they
// measure the two hardware facts the GEMM's design rests on.
//
//  * Accumulation inside the matrix unit. The DeepSeek-V3 report (Chinese
//    translation), section 3.3.2 "increasing accumulation precision", finds
//    that FP8 products accumulated inside the H800 tensor cores keep about 14
//    bits, giving a maximum relative error near 2% for K = 4096, and promotes
//    every N_C = 128 elements to FP32 (section 3.5.2 restates the 14 bits).
//    fp8bq_probe_mfma_accum computes a 16 x 16 x K product both ways on gfx950:
//    chained inside the matrix unit (each 128-K instruction adds into the
//    previous result) and promoted (each 128-K chunk a fresh instruction,
//    added in FP32 on the vector ALU). fp8bq_probe_mfma_once runs a single
//    instruction on crafted inputs.
//  * Power. fp8bq_probe_mfma_stream keeps every SIMD's matrix unit busy from
//    register-resident operands, with or without the promotion FMAs (four per
//    instruction, as the exact-scale GEMM issues them), and reports the shader
//    clock the chip holds in each case.
//  * Memory. fp8bq_probe_stream_2to1 is the quantisers' traffic (2 bytes read,
//    1 written per element) with no arithmetic: their measured ceiling.
#include "../../include/fp8bq_probe.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

thread_local char g_err[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int check_gfx950() {
  int dev = -1;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(FP8BQ_E_DEVICE, "no HIP device available");
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(FP8BQ_E_DEVICE, "device is %s, the probes are built for gfx950", prop.gcnArchName);
  return FP8BQ_OK;
}

int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FP8BQ_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return FP8BQ_OK;
}

// Operand fragment of v_mfma_f32_16x16x128_f8f6f4: lane l holds row l % 16 of
// its operand and the 32 bytes k = 32 (l / 16) .. 32 (l / 16) + 31 of the
// 128-K chunk (both operands pair k the same way).
__device__ __forceinline__ v8i load_frag(const uint8_t* base, int64_t ld, int lane) {
  const uint4* p = reinterpret_cast<const uint4*>(base + (int64_t)(lane & 15) * ld + 32 * (lane >> 4));
  const uint4 x0 = p[0], x1 = p[1];
  return v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

__device__ __forceinline__ v4f mfma(const v8i& a, const v8i& b, const v4f& c) {
  // format 0 (E4M3) for both operands, no block scales: the plain FP8 instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Result layout: lane l, register r is row 4 (l / 16) + r of the first operand,
// row l % 16 of the second.
__device__ __forceinline__ void store_16x16(float* out, const v4f& d, int lane) {
#pragma unroll
  for (int r = 0; r < 4; ++r) out[(4 * (lane >> 4) + r) * 16 + (lane & 15)] = d[r];
}

__global__ __launch_bounds__(64) void accum_kernel(const uint8_t* a, const uint8_t* b, int64_t k, float* chained,
                                                   float* promoted) {
  const int lane = threadIdx.x;
  v4f acc_chain = {0.f, 0.f, 0.f, 0.f}, acc_prom = {0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = 0; c < k / 128; ++c) {
    const v8i fa = load_frag(a + 128 * c, k, lane), fb = load_frag(b + 128 * c, k, lane);
    acc_chain = mfma(fa, fb, acc_chain);
    const v4f p = mfma(fa, fb, zero);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc_prom[r] += p[r];
  }
  store_16x16(chained, acc_chain, lane);
  store_16x16(promoted, acc_prom, lane);
}

__global__ __launch_bounds__(64) void once_kernel(const uint8_t* a, const uint8_t* b, const float* c, float* d) {
  const int lane = threadIdx.x;
  v4f cin;
#pragma unroll
  for (int r = 0; r < 4; ++r) cin[r] = c[(4 * (lane >> 4) + r) * 16 + (lane & 15)];
  store_16x16(d, mfma(load_frag(a, 128, lane), load_frag(b, 128, lane), cin), lane);
}

// Eight waves per workgroup (two per SIMD), each with a 64 x 128 tile of 4 x 8
// MFMAs per iteration on register-resident fragments; FOLD adds each result to
// an FP32 accumulator with a per-row scale three instructions later (the
// promotion of the exact-scale GEMM).
template <bool FOLD>
__global__ __launch_bounds__(512) void stream_kernel(const uint8_t* codes, const float* scales, int64_t iters,
                                                     float* sink, unsigned long long* ticks) {
  constexpr int TM = 4, TN = 8, NT = TM * TN, LAG = 3;
  constexpr int64_t kFrags = (TM + TN) * 2048;   // a wave's fragments: 24 KiB
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // each wave's fragments start at a 2 KiB multiple below 4 MiB - 24 KiB, so every
  // read stays inside the 4 MiB codes buffer
  constexpr int64_t kSpan = ((int64_t)1 << 22) - kFrags;
  const uint8_t* base = codes + ((int64_t)blockIdx.x * 8 + wave) * kFrags % kSpan;
  v8i af[TM], bf[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[i] = load_frag(base + i * 2048, 128, lane);
#pragma unroll
  for (int j = 0; j < TN; ++j) bf[j] = load_frag(base + (TM + j) * 2048, 128, lane);
  float sc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) sc[i] = scales[(lane + 16 * i) & 63];
  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f pend[LAG + 1];
#pragma unroll
  for (int q = 0; q <= LAG; ++q) pend[q] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      pend[t % (LAG + 1)] = mfma(bf[t / TM], af[t % TM], zero);
      const int u = (t - LAG + NT) % NT;
      if constexpr (FOLD) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[u % TM][u / TM][r] = __builtin_fmaf(pend[u % (LAG + 1)][r], sc[u % TM], acc[u % TM][u / TM][r]);
        asm volatile("" : "+v"(acc[u % TM][u / TM]));
      } else {
        asm volatile("" ::"v"(pend[u % (LAG + 1)]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) s += acc[i][j][0];
#pragma unroll
  for (int q = 0; q <= LAG; ++q) s += pend[q][1];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = t1 - t0;
    ticks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Streaming ceiling of the quantisers' traffic: read 2 bytes, write 1 byte per
// element (lane i reads bytes [32 i, 32 i + 32) and writes the 16 high bytes of
// its 16 bf16 to bytes [16 i, 16 i + 16)), with no arithmetic beyond a byte
// permute: what the memory system delivers for the quantisers' read/write mix.
__global__ __launch_bounds__(256) void stream21_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                       int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 a = src[2 * i], b = src[2 * i + 1];
  auto hi = [](uint32_t u, uint32_t v) { return __builtin_amdgcn_perm(v, u, 0x07050301u); };
  dst[i] = make_uint4(hi(a.x, a.y), hi(a.z, a.w), hi(b.x, b.y), hi(b.z, b.w));
}

}  // namespace

extern "C" {

const char* fp8bq_probe_last_error(void) { return g_err; }

int fp8bq_probe_mfma_accum(const void* a, const void* b, int64_t k, float* chained, float* promoted, void* stream) {
  if (!a || !b || !chained || !promoted) return fail(FP8BQ_E_INVAL, "mfma_accum: null pointer");
  if (k <= 0 || k % 128 || k > ((int64_t)1 << 24)) return fail(FP8BQ_E_SHAPE, "mfma_accum: k must be a positive multiple of 128 up to 2^24");
  if (((uintptr_t)a | (uintptr_t)b) % 16) return fail(FP8BQ_E_ALIGN, "mfma_accum: a and b must be 16-byte aligned");
  if (int st = check_gfx950()) return st;
  hipLaunchKernelGGL(accum_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                     (const uint8_t*)b, k, chained, promoted);
  return launched("mfma_accum");
}

int fp8bq_probe_mfma_once(const void* a, const void* b, const float* c, float* d, void* stream) {
  if (!a || !b || !c || !d) return fail(FP8BQ_E_INVAL, "mfma_once: null pointer");
  if (((uintptr_t)a | (uintptr_t)b) % 16) return fail(FP8BQ_E_ALIGN, "mfma_once: a and b must be 16-byte aligned");
  if (int st = check_gfx950()) return st;
  hipLaunchKernelGGL(once_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a, (const uint8_t*)b,
                     c, d);
  return launched("mfma_once");
}

int fp8bq_probe_mfma_stream(int fold, int64_t iters, int32_t workgroups, const void* codes, const float* scales,
                            float* sink, unsigned long long* ticks, void* stream) {
  if (!codes || !scales || !sink || !ticks) return fail(FP8BQ_E_INVAL, "mfma_stream: null pointer");
  if (iters <= 0 || iters > ((int64_t)1 << 24)) return fail(FP8BQ_E_INVAL, "mfma_stream: iters must be in [1, 2^24]");
  if (workgroups <= 0 || workgroups > 4096) return fail(FP8BQ_E_INVAL, "mfma_stream: workgroups must be in [1, 4096]");
  if ((uintptr_t)codes % 16) return fail(FP8BQ_E_ALIGN, "mfma_stream: codes must be 16-byte aligned");
  if (int st = check_gfx950()) return st;
  const dim3 grid((unsigned)workgroups), block(512);
  if (fold)
    hipLaunchKernelGGL(stream_kernel<true>, grid, block, 0, (hipStream_t)stream, (const uint8_t*)codes, scales,
                       iters, sink, ticks);
  else
    hipLaunchKernelGGL(stream_kernel<false>, grid, block, 0, (hipStream_t)stream, (const uint8_t*)codes, scales,
                       iters, sink, ticks);
  return launched("mfma_stream");
}

}  // extern "C"

extern "C" int fp8bq_probe_stream_2to1(const void* src, void* dst, int64_t n, void* stream) {
  if (!src || !dst) return fail(FP8BQ_E_INVAL, "stream_2to1: null pointer");
  if (n <= 0 || n % 16 || n / 16 / 256 >= ((int64_t)1 << 31))
    return fail(FP8BQ_E_SHAPE, "stream_2to1: n must be a positive multiple of 16 (and below 2^43)");
  if (((uintptr_t)src | (uintptr_t)dst) % 16) return fail(FP8BQ_E_ALIGN, "stream_2to1: src and dst must be 16-byte aligned");
  if (int st = check_gfx950()) return st;
  const int64_t n16 = n / 16;
  hipLaunchKernelGGL(stream21_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, (uint4*)dst, n16);
  return launched("stream_2to1");
}
