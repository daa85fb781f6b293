// Grouped (per-expert) FP8 Fprop for decode-sized batches: every expert sees at
// most 256 tokens, so the GEMM is bound by streaming the experts' FP8 weights
// from HBM, not by the matrix unit (report section 3.4.2 / "inference and
// deployment", decoding stage: each expert processes a small batch, at most
// about 256 tokens, and the bottleneck is memory access).
//
// What it computes is the grouped Fprop of fp8bq_grouped_gemm (per-128-K-chunk
// promotion acc += P_c * s_a * s_b in FP32, bf16 out), without padding the
// experts' rows: expert e owns rows [row_off[e], row_off[e+1]) of any length
// up to 256.
//
// Design (MI355X / gfx950):
//  * One workgroup per (expert, 64 output columns), 8 waves (more waves issue
//    the loads: each load instruction keeps its wave for a while). The
//    expert's rows are T subtiles of 16 (T = 1, 2, 4, 8 or 16 for its count;
//    the LDS allocation follows the launch's largest expert); wave w computes
//    subtiles w, w + 8, ... against the slice's four weight subtiles, so
//    every activation fragment is read from LDS once. 64 columns lie inside
//    one 128 x 128 weight block, so a chunk has one weight scale per
//    workgroup.
//  * The weight slice streams through an LDS ring of kWStages chunks (8 KB
//    each) with global -> LDS DMA, issued kWStages - 1 chunks ahead: that is
//    the memory-level parallelism the HBM stream needs (≈ 40-64 KB in flight
//    per CU). The expert's activation rows (read by every column slice, so
//    mostly from L2) go through a shorter ring of kAStages chunks. Rows past
//    the expert's end read as zeros (buffer bound) and are never stored.
//  * One barrier per chunk; before it each wave waits only until its own DMA
//    for the chunk has landed (vmcnt counted from the fixed issue pattern, with
//    the final chunks re-issued so that the count stays exact). The loads are
//    split between waves by operand (activation waves, weight waves): a wave's
//    loads complete in issue order, so a wave that waited for the activations
//    of chunk c would also wait for every older weight load.
//  * Workgroups are expert-major in launch order, which the hardware deals
//    to the 8 XCDs in turn: each expert's column slices spread over all XCDs.
//    With skewed expert sizes this beats keeping an expert's slices on one
//    XCD (whose L2 would hold its activations): 61.5 -> 59.6 us on the
//    256-token decode mix; with 16 rows per expert it costs 3%.
#include "gemm_kernels.h"

namespace fp8bq {
namespace {

constexpr int kDN = 64;   // output columns per workgroup

// LDS DMA of one dword per lane through a raw buffer resource (see dma16_buf).
__device__ __forceinline__ void dma4_buf(const u32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// dma16_buf with the non-temporal hint, for the weight stream: each weight byte
// is read once per call, so it should not displace the activations (re-read by
// every column slice) from the caches. With a clean cache the two cost the
// same; after a kernel that leaves many dirty lines behind, plain loads have
// to evict them first (49 us against 28 us for the weight stream alone).
__device__ __forceinline__ void dma16_buf_nt(const u32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}

struct DecodeArgs {
  int64_t n, k;
  const uint8_t* a; int64_t lda;
  const float* sa; int64_t ldsa;
  const uint8_t* b; int64_t ldb;       // expert e's weight [n, k] at b + e * n * ldb
  const float* sb; int64_t ldsb;       // expert e's block grid at sb + e * (n / 128) * ldsb
  uint16_t* out; int64_t ldo;
  int groups, slices;                  // slices = n / 64
  int row_off[kMaxGroups + 1];
};

template <int T>
struct DecodeCfg {
  static constexpr int kAStages = T >= 16 ? 3 : 4;
  static constexpr int kWStages = T >= 16 ? 5 : 8;
  static constexpr int kARows = T * 16;
  static constexpr int kASlot = kARows * BK;
  static constexpr int kWSlot = kDN * BK;
  static constexpr int kAOff = 0;
  static constexpr int kWOff = kAStages * kASlot;
  static constexpr int kSaOff = kWOff + kWStages * kWSlot;
  static constexpr int kSaInstr = (kARows + 63) / 64;
  static constexpr int kSaSlot = kSaInstr * 256;           // activation scales of one chunk
  static constexpr int kSwOff = kSaOff + kAStages * kSaSlot;
  static constexpr int kBytes = kSwOff + kWStages * 16;
  // Loads are split by role, because a wave's loads complete in issue order
  // (one vmcnt per wave): waves 0-3 load the activations (8 rows per
  // instruction, group g by wave g % 4) and their scales (instruction j by
  // wave j), waves 4-7 the weight slice (16 rows each) and wave 7 the weight
  // scale. A wave then waits only for its own stream: the activation waves
  // for chunk c issued kAStages - 1 rounds back, the weight waves for chunk c
  // issued kWStages - 1 rounds back, so the weight stream keeps its depth.
  static constexpr int kAInstr = 2 * T;
  static constexpr int kAPerWave = (kAInstr + 3) / 4;
  static constexpr int ops(int w) {
    return w < 4 ? (kAInstr / 4 + (w < kAInstr % 4 ? 1 : 0)) + (w < kSaInstr ? 1 : 0) : 2 + (w == 7 ? 1 : 0);
  }
  // At the start of chunk c: after its loads of chunk c a wave has issued
  // kAStages - 2 (activation waves) or kWStages - 2 (weight waves) further
  // rounds; waiting until at most that many loads are outstanding leaves
  // chunk c's loads landed.
  static constexpr int wait(int w) { return (w < 4 ? kAStages - 2 : kWStages - 2) * ops(w); }
  static_assert(wait(0) <= 63 && wait(4) <= 63 && wait(7) <= 63, "vmcnt range");
  static_assert(kBytes <= 160 * 1024, "LDS");
  static_assert(kWStages >= kAStages, "weights are issued at least as far ahead as activations");
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// One workgroup's work with T row subtiles (the expert's rows rounded up):
// ring sizes, loads and MFMAs are those of DecodeCfg<T>, inside the LDS the
// kernel allocated for its largest T.
template <int T>
__device__ __forceinline__ void decode_slice(const DecodeArgs& p, uint8_t* smem, int e, int slice, int m0, int me) {
  using C = DecodeCfg<T>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int64_t n0 = (int64_t)slice * kDN;
  const int nc = (int)(p.k / BK);
  const uint32_t sbase = lds_addr(smem);

  const uint8_t* a_e = p.a + (int64_t)m0 * p.lda;
  const uint8_t* a_end = p.a + (int64_t)(m0 + me - 1) * p.lda + p.k;
  const uint8_t* b_e = p.b + (int64_t)e * p.n * p.ldb + n0 * p.ldb;
  const uint8_t* b_end = b_e + (int64_t)(kDN - 1) * p.ldb + p.k;
  const float* sb_e = p.sb + (int64_t)e * (p.n / 128) * p.ldsb + (n0 / 128) * p.ldsb;
  // per-lane DMA offsets (fixed for every chunk): lane ln of an 8-row group
  // loads row 8 g + ln / 8 at the logical slot that lands in physical slot ln % 8
  const int lr = lane >> 3, ls = lane & 7;
  uint32_t voff_a[C::kAPerWave];          // activation waves: groups 4 q + wave
#pragma unroll
  for (int q = 0; q < C::kAPerWave; ++q) {
    const int row = 8 * (4 * q + (wave & 3)) + lr;
    voff_a[q] = (uint32_t)row * (uint32_t)p.lda + (uint32_t)((ls ^ swz(row)) * 16);
  }
  uint32_t voff_w[2];                      // weight waves: rows 16 (wave - 4) + 8 h + lane / 8
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * (wave & 3) + 8 * h + lr;
    voff_w[h] = (uint32_t)row * (uint32_t)p.ldb + (uint32_t)((ls ^ swz(row)) * 16);
  }

  // One round of loads: activations (and their scales) of chunk ca into ring
  // slot ca % kAStages, the weight slice (and its scale) of chunk cw into
  // slot cw % kWStages. Chunks past the end load the last chunk again (into
  // slots no one reads any more), so every round issues the same loads.
  auto issue = [&](int ca, int cw) {
    const int as = ca % C::kAStages, ws = cw % C::kWStages;
    ca = min(ca, nc - 1);
    cw = min(cw, nc - 1);
    if (wave < 4) {
      const u32x4 ra = make_rsrc(a_e + (int64_t)ca * BK, a_end);
      const uint32_t abase = sbase + C::kAOff + as * C::kASlot;
#pragma unroll
      for (int q = 0; q < C::kAPerWave; ++q)
        if (4 * q + wave < C::kAInstr) dma16_buf(ra, voff_a[q], abase + (4 * q + wave) * 8 * BK);
      if (wave < C::kSaInstr) {
        const float* s0 = p.sa + (int64_t)ca * p.ldsa + m0;
        const u32x4 rs = make_rsrc(reinterpret_cast<const uint8_t*>(s0), reinterpret_cast<const uint8_t*>(s0 + me));
        dma4_buf(rs, (uint32_t)(64 * wave + lane) * 4u, sbase + C::kSaOff + as * C::kSaSlot + 64 * wave * 4);
      }
    } else {
      const u32x4 rw = make_rsrc(b_e + (int64_t)cw * BK, b_end);
      const uint32_t wbase = sbase + C::kWOff + ws * C::kWSlot;
#pragma unroll
      for (int h = 0; h < 2; ++h) dma16_buf_nt(rw, voff_w[h], wbase + (16 * (wave & 3) + 8 * h) * BK);
      if (wave == 7) {
        if (lane == 0) dma4(uniform_ptr(sb_e + cw), 0u, sbase + C::kSwOff + ws * 16);
      }
    }
  };

  // Prologue: kWStages - 1 rounds, weights of chunks 0 .. kWStages - 2 and
  // activations of chunks 0 .. kAStages - 2; the rounds beyond that load
  // activations into slot kAStages - 1, which the loop's first round fills
  // again (later, in issue order) before anyone reads it.
  for (int i = 0; i < C::kWStages - 1; ++i) issue(i < C::kAStages - 1 ? i : C::kAStages - 1, i);

  const int sw = swz(l16);
  const int off0 = l16 * BK + (((2 * lq) ^ sw) * 16);
  const int off1 = l16 * BK + (((2 * lq + 1) ^ sw) * 16);
  // wave w computes row subtiles 8 q + w (q < Q) against all four weight
  // subtiles of the slice: each activation fragment is read from LDS by one
  // wave only (with T < 8 the waves past T only load)
  constexpr int Q = (T + 7) / 8;
  const bool computes = T >= 8 || wave < T;          // uniform per wave
  v4f acc[Q][4];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[q][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

#pragma clang loop unroll(disable)
  for (int c = 0; c < nc; ++c) {
    switch (wave) {   // uniform
      case 0: wait_vmcnt<C::wait(0)>(); break;
      case 1: wait_vmcnt<C::wait(1)>(); break;
      case 2: wait_vmcnt<C::wait(2)>(); break;
      case 3: wait_vmcnt<C::wait(3)>(); break;
      case 7: wait_vmcnt<C::wait(7)>(); break;
      default: wait_vmcnt<C::wait(4)>(); break;
    }
    __syncthreads();
    issue(c + C::kAStages - 1, c + C::kWStages - 1);
    if (computes) {
      const uint8_t* as = smem + C::kAOff + (c % C::kAStages) * C::kASlot;
      const uint8_t* ws = smem + C::kWOff + (c % C::kWStages) * C::kWSlot;
      const float* sas = reinterpret_cast<const float*>(smem + C::kSaOff + (c % C::kAStages) * C::kSaSlot);
      const float swv = *reinterpret_cast<const float*>(smem + C::kSwOff + (c % C::kWStages) * 16);
      v8i wf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[j] = frag(ws + 16 * j * BK, off0, off1);
      // all MFMAs of the chunk, then their folds (no branch between them, so
      // the fragment reads and the MFMAs pipeline)
      v4f pc[Q][4];
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const v8i af = frag(as + 16 * (8 * q + wave) * BK, off0, off1);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pc[q][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], af, zero, 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float sc = sas[16 * (8 * q + wave) + l16] * swv;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[q][j][r] = __builtin_fmaf(pc[q][j][r], sc, acc[q][j][r]);
      }
    }
  }
  // the repeated loads after the last chunk must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!computes) return;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int r = 16 * (8 * q + wave) + l16;
    if (r < me) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x2 lo = __builtin_convertvector((f32x2){acc[q][j][0], acc[q][j][1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector((f32x2){acc[q][j][2], acc[q][j][3]}, bf16x2);
        uint2 packed;
        __builtin_memcpy(&packed.x, &lo, 4);
        __builtin_memcpy(&packed.y, &hi, 4);
        *reinterpret_cast<uint2*>(p.out + (int64_t)(m0 + r) * p.ldo + n0 + 16 * j + 4 * lq) = packed;
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(512) void gemm_decode_kernel(DecodeArgs p) {
  // DecodeCfg<T>::kBytes grows with T: the largest T sets the allocation
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeCfg<MT>::kBytes];

  // workgroup -> (expert, slice), expert-major: the hardware deals consecutive
  // workgroups to the 8 XCDs in turn, so each expert's slices spread over all
  // XCDs and a large expert does not load one XCD alone
  const int f = blockIdx.x;
  const int e = f / p.slices, slice = f % p.slices;
  const int m0 = p.row_off[e];
  const int me = p.row_off[e + 1] - m0;
  // uniform per workgroup: an empty expert has nothing to do; otherwise the
  // smallest T that covers its rows
  if (me <= 0) return;
  if (me <= 16) decode_slice<1>(p, smem, e, slice, m0, me);
  else if (me <= 32) { if constexpr (MT >= 2) decode_slice<2>(p, smem, e, slice, m0, me); }
  else if (me <= 64) { if constexpr (MT >= 4) decode_slice<4>(p, smem, e, slice, m0, me); }
  else if (me <= 128) { if constexpr (MT >= 8) decode_slice<8>(p, smem, e, slice, m0, me); }
  else { if constexpr (MT >= 16) decode_slice<16>(p, smem, e, slice, m0, me); }
}

}  // namespace

hipError_t launch_grouped_gemm_decode(int groups, const int64_t* row_off, int64_t n, int64_t k,
                                      const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                      const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                                      uint16_t* out, int64_t ldo, hipStream_t st) {
  DecodeArgs p;
  p.n = n; p.k = k;
  p.a = a; p.lda = lda; p.sa = sa; p.ldsa = ldsa;
  p.b = b; p.ldb = ldb; p.sb = sb; p.ldsb = ldsb;
  p.out = out; p.ldo = ldo;
  p.groups = groups;
  p.slices = (int)(n / kDN);
  int64_t most = 0;
  for (int e = 0; e <= groups; ++e) p.row_off[e] = (int)row_off[e];
  for (int e = 0; e < groups; ++e) most = row_off[e + 1] - row_off[e] > most ? row_off[e + 1] - row_off[e] : most;
  if (most == 0) return hipSuccess;
  const dim3 grid((unsigned)(groups * p.slices)), block(512);
  if (most <= 16)       hipLaunchKernelGGL(gemm_decode_kernel<1>, grid, block, 0, st, p);
  else if (most <= 32)  hipLaunchKernelGGL(gemm_decode_kernel<2>, grid, block, 0, st, p);
  else if (most <= 64)  hipLaunchKernelGGL(gemm_decode_kernel<4>, grid, block, 0, st, p);
  else if (most <= 128) hipLaunchKernelGGL(gemm_decode_kernel<8>, grid, block, 0, st, p);
  else                  hipLaunchKernelGGL(gemm_decode_kernel<16>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace fp8bq
