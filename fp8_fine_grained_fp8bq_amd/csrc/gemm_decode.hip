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
//  * Two workgroup shapes, each streaming 64 x K weight bytes: an expert of at
//    most 32 rows gets one workgroup per 64 output columns over all of K; a
//    larger expert (when the caller gives a workspace) one per 128 output
//    columns and half of K. A workgroup moves its weight slice once and its
//    expert's rows once per K range, so the 128-column shape reads half the
//    activation bytes per output column. Per CU the bytes moved, not the
//    matrix unit, set a workgroup's time: a 64-column workgroup of a 217-row
//    expert moves 0.46 MB of weights and 1.6 MB of activations; its 128-column
//    half-K pair 0.46 + 0.8 MB each. The two halves add their FP32 sums: each
//    stores its partial sums with device-coherent stores and bumps a counter;
//    the second to finish adds the other's partial (two-term sums are the
//    same in either order) and writes the bf16 output. Nobody waits.
//  * 8 waves with fixed roles: waves 0-3 compute, waves 4-5 stream the weight
//    slice, waves 6-7 the expert's rows. The expert's rows are T subtiles of
//    16, T the next available count at or above rows / 16 (1, 2, 3, 4, 6, 8,
//    10, 12, 14 or 16; rows past the expert's end read as zeros through the
//    buffer bound and are never stored). 64-column shape: compute wave w takes
//    the slice's four weight subtiles against row subtiles w, w + 4, ...;
//    128-column shape: the four weight subtiles of column half w % 2 against
//    row subtiles w / 2, w / 2 + 2, ... Either way a 64 or 128 column slice
//    lies inside one 128 x 128 weight block: a chunk has one weight scale.
//    With every wave both loading and computing, a wave stalled on a full
//    memory queue could not compute and the memory pipeline idled while the
//    waves computed: the 256-token decode mix took 51.2 us, 42.8 us with the
//    roles separated.
//  * The weight slice streams through an LDS ring of kWStages chunks with
//    global -> LDS DMA (non-temporal: each weight byte is read once), issued
//    kWStages - 1 chunks ahead; the activation rows (mostly L2 hits: every
//    column slice of the expert reads them) through a ring of kAStages chunks.
//  * One barrier per chunk; before it each loader waits only until its own DMA
//    for the chunk has landed (vmcnt counted from the fixed issue pattern, with
//    the final chunks re-issued so that the count stays exact). Each loader
//    carries one stream: a wave's loads complete in issue order, so a wave
//    that waited for the activations of chunk c would also wait for every
//    older weight load.
//  * Workgroups are expert-major in launch order, which the hardware deals
//    to the 8 XCDs in turn: each expert's column slices spread over all XCDs.
//    With skewed expert sizes this beats keeping an expert's slices on one
//    XCD (whose L2 would hold its activations, but whose 32 CUs would then
//    ask the same L2 channels for the same lines at once): with the split
//    workgroups 52.0 against 53.4 us on the 256-token decode mix, 50.5
//    against 53.9 us for one 217-row expert among 1-row ones.
#include "gemm_kernels.h"

#include <mutex>

// Scratch of fp8bq_grouped_gemm_decode_noalloc, the split form for callers
// that cannot allocate: its workspace (the counters, then the partial sums)
// lives here, kNoAllocScratchBytes per device, held until the process ends.
// Every call on a device shares that device's copy. The counters start at zero
// (the array is zero when the code object is loaded on a device) and every
// call leaves them at zero; the partial sums need no clearing (a K half reads
// only what its partner stored in the same call). Calls that overlap on one
// device race. Host code never passes this name to a kernel: it is a host-side
// stand-in; the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[fp8bq::kNoAllocScratchBytes];

namespace fp8bq {
namespace {

constexpr int kDN = 64;    // output columns of a full-K workgroup
constexpr int kDN2 = 128;  // output columns of a half-K workgroup

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
  int64_t n, k, m;
  const uint8_t* a; int64_t lda;
  const float* sa; int64_t ldsa;
  const uint8_t* b; int64_t ldb;       // expert e's weight [n, k] at b + e * n * ldb
  const float* sb; int64_t ldsb;       // expert e's block grid at sb + e * (n / 128) * ldsb
  uint16_t* out; int64_t ldo;
  float* part;                         // split experts' partial sums (layout at decode_slice's epilogue)
  uint32_t* cnt;                       // counter of (expert e, 128-column slice s) at cnt[e * 256 + s]; zero between calls
  int groups, slices;                  // slices = n / 64 workgroups per expert
  int part_subtiles;                   // 16-row subtiles of all split experts (one K half's share of part)
  int row_off[kMaxGroups + 1];
  int part_off[kMaxGroups];            // split expert e's first subtile in part
  uint8_t split[kMaxGroups];           // 1: the expert runs as 128-column, half-K workgroups
};

template <int T, int CW>
struct DecodeCfg {
  static_assert(CW == kDN || CW == kDN2, "workgroup width");
  static constexpr bool kWide = CW == kDN2;
  static constexpr int kAStages = T > 8 ? 3 : 4;
  static constexpr int kWStages = kWide ? (T >= 15 ? 3 : T >= 13 ? 4 : 5) : (T >= 16 ? 5 : 8);
  static constexpr int kARows = T * 16;
  static constexpr int kASlot = kARows * BK;
  static constexpr int kWSlot = CW * BK;
  static constexpr int kAOff = 0;
  static constexpr int kWOff = kAStages * kASlot;
  static constexpr int kSaOff = kWOff + kWStages * kWSlot;
  static constexpr int kSaInstr = (kARows + 63) / 64;
  static constexpr int kSaSlot = kSaInstr * 256;           // activation scales of one chunk
  static constexpr int kSwOff = kSaOff + kAStages * kSaSlot;
  static constexpr int kBytes = kSwOff + kWStages * 16 + 16;   // + one word to broadcast the split state
  // Waves 0-3 only compute; waves 4-7 only load, one stream per wave, because a
  // wave's loads complete in issue order (one vmcnt per wave): waves 4 and 5 the
  // weight slice (8-row instruction i by wave 4 + i % 2) and wave 5 its scale,
  // waves 6 and 7 the activation rows (instruction i by wave 6 + i % 2) and
  // their scales (instruction j by wave 6 + j % 2). A loader stalled on a full
  // memory queue delays no arithmetic, and the compute waves hold no loads, so
  // nothing makes them wait on memory but the barrier (with every wave both
  // loading and computing, switching the arithmetic off made the kernel
  // 18-20% faster: the two were serialised).
  static constexpr int kAInstr = 2 * T;
  static constexpr int kWInstr = CW / 8;
  static constexpr int ops(int w) {   // loads per round of loader wave w
    return w < 6 ? kWInstr / 2 + (w == 5 ? 1 : 0) : kAInstr / 2 + kSaInstr / 2 + (w == 6 ? kSaInstr % 2 : 0);
  }
  // At the start of chunk c: after its loads of chunk c a wave has issued
  // kAStages - 2 (activation waves) or kWStages - 2 (weight waves) further
  // rounds; waiting until at most that many loads are outstanding leaves
  // chunk c's loads landed.
  static constexpr int wait(int w) { return (w < 6 ? kWStages - 2 : kAStages - 2) * ops(w); }
  static_assert((kWStages - 1) * ops(5) <= 63 && (kAStages - 1) * ops(6) <= 63, "vmcnt range");
  static_assert(kBytes <= 160 * 1024, "LDS");
  static_assert(kWStages >= kAStages, "weights are issued at least as far ahead as activations");
  static_assert(kWStages >= 3 && kAStages >= 3, "ring depth");
};

// LDS of the largest configuration a launch can run (cmax from gemm_kernels.h).
constexpr int kSmallBytes = cmax(DecodeCfg<1, kDN>::kBytes, DecodeCfg<2, kDN>::kBytes);
constexpr int kNarrowBytes = cmax(cmax(cmax(DecodeCfg<3, kDN>::kBytes, DecodeCfg<4, kDN>::kBytes),
                                       cmax(DecodeCfg<6, kDN>::kBytes, DecodeCfg<8, kDN>::kBytes)),
                                  cmax(cmax(DecodeCfg<10, kDN>::kBytes, DecodeCfg<12, kDN>::kBytes),
                                       cmax(DecodeCfg<14, kDN>::kBytes, DecodeCfg<16, kDN>::kBytes)));
constexpr int kWideBytes = cmax(cmax(cmax(DecodeCfg<3, kDN2>::kBytes, DecodeCfg<4, kDN2>::kBytes),
                                     cmax(DecodeCfg<6, kDN2>::kBytes, DecodeCfg<8, kDN2>::kBytes)),
                                cmax(cmax(DecodeCfg<10, kDN2>::kBytes, DecodeCfg<12, kDN2>::kBytes),
                                     cmax(DecodeCfg<14, kDN2>::kBytes, DecodeCfg<16, kDN2>::kBytes)));
constexpr int kBigBytes = cmax(kSmallBytes, cmax(kNarrowBytes, kWideBytes));

// Cache policy of the workspace's buffer accesses: sc1, device-coherent.
constexpr int kSc1 = 16;

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint2 bf16x4(const v4f& v) {
  const bf16x2 lo = __builtin_convertvector((f32x2){v[0], v[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2){v[2], v[3]}, bf16x2);
  uint2 packed;
  __builtin_memcpy(&packed.x, &lo, 4);
  __builtin_memcpy(&packed.y, &hi, 4);
  return packed;
}

// One workgroup's work: T row subtiles (the expert's rows rounded up), CW
// output columns from n0, K chunks [kc0, kc1); h = which K half (wide shape).
// Ring sizes, loads and MFMAs are those of DecodeCfg<T, CW>, inside the LDS
// the kernel allocated for its largest configuration.
template <int T, int CW>
__device__ __forceinline__ void decode_slice(const DecodeArgs& p, uint8_t* smem, int e, int64_t n0, int kc0,
                                             int kc1, int h, int m0, int me) {
  using C = DecodeCfg<T, CW>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int nc = kc1 - kc0;
  const uint32_t sbase = lds_addr(smem);

  const uint8_t* a_e = p.a + (int64_t)m0 * p.lda + (int64_t)kc0 * BK;
  const uint8_t* a_end = p.a + (int64_t)(m0 + me - 1) * p.lda + p.k;
  const uint8_t* b_e = p.b + (int64_t)e * p.n * p.ldb + n0 * p.ldb + (int64_t)kc0 * BK;
  const uint8_t* b_end = p.b + (int64_t)e * p.n * p.ldb + (n0 + CW - 1) * p.ldb + p.k;
  const float* sb_e = p.sb + (int64_t)e * (p.n / 128) * p.ldsb + (n0 / 128) * p.ldsb + kc0;
  const float* sa_e = p.sa + (int64_t)kc0 * p.ldsa + m0;
  // per-lane DMA offsets of a loader wave (fixed for every chunk): lane ln of an
  // 8-row group loads row 8 g + ln / 8 at the logical slot that lands in
  // physical slot ln % 8; instruction i of wave 4 + h (weights) or 6 + h
  // (activations) is group g = 2 i + h
  const int lr = lane >> 3, ls = lane & 7, h2 = wave & 1;
  const bool wload = wave == 4 || wave == 5, aload = wave >= 6;
  constexpr int kAPer = C::kAInstr / 2, kWPer = C::kWInstr / 2;
  constexpr int kPer = kAPer > kWPer ? kAPer : kWPer;
  uint32_t voff[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int row = 8 * (2 * i + h2) + lr;
    voff[i] = (uint32_t)row * (uint32_t)(aload ? p.lda : p.ldb) + (uint32_t)((ls ^ swz(row)) * 16);
  }

  // One round of loads: activations (and their scales) of chunk ca into ring
  // slot ca % kAStages, the weight slice (and its scale) of chunk cw into
  // slot cw % kWStages. Chunks past the end load the last chunk again (into
  // slots no one reads any more), so every round issues the same loads.
  auto issue = [&](int ca, int cw) {
    if (wload) {
      const int ws = cw % C::kWStages;
      cw = min(cw, nc - 1);
      const u32x4 rw = make_rsrc(b_e + (int64_t)cw * BK, b_end);
      const uint32_t wbase = sbase + C::kWOff + ws * C::kWSlot;
#pragma unroll
      for (int i = 0; i < kWPer; ++i) dma16_buf_nt(rw, voff[i], wbase + (2 * i + h2) * 8 * BK);
      if (wave == 5) {
        if (lane == 0) dma4(uniform_ptr(sb_e + cw), 0u, sbase + C::kSwOff + ws * 16);
      }
    } else if (aload) {
      const int as = ca % C::kAStages;
      ca = min(ca, nc - 1);
      const u32x4 ra = make_rsrc(a_e + (int64_t)ca * BK, a_end);
      const uint32_t abase = sbase + C::kAOff + as * C::kASlot;
#pragma unroll
      for (int i = 0; i < kAPer; ++i) dma16_buf(ra, voff[i], abase + (2 * i + h2) * 8 * BK);
      const float* s0 = sa_e + (int64_t)ca * p.ldsa;
      const u32x4 rs = make_rsrc(reinterpret_cast<const uint8_t*>(s0), reinterpret_cast<const uint8_t*>(s0 + me));
#pragma unroll
      for (int jj = 0; jj < C::kSaInstr; jj += 2) {
        const int j = jj + h2;
        if (j < C::kSaInstr)
          dma4_buf(rs, (uint32_t)(64 * j + lane) * 4u, sbase + C::kSaOff + as * C::kSaSlot + 64 * j * 4);
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
  // Compute wave w (0-3). 128-column shape: the four weight subtiles of column
  // half w % 2 against row subtiles rs(q) = w / 2 + 2 q; 64-column shape: all
  // four weight subtiles against rs(q) = w + 4 q. Subtiles at or past T are
  // skipped (uniform per wave; never the case for an even T in the 128-column
  // shape or a T divisible by 4 in the 64-column one).
  constexpr int kRowStep = C::kWide ? 2 : 4;
  constexpr int Q = (T + kRowStep - 1) / kRowStep;
  constexpr bool kAllValid = T % kRowStep == 0;
  const bool computes = wave < 4;
  const int rs0 = C::kWide ? (wave >> 1) : wave;
  const int cs0 = C::kWide ? 4 * (wave & 1) : 0;
  auto valid = [&](int q) { return kAllValid || kRowStep * q + rs0 < T; };
  v4f acc[Q][4];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[q][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

#pragma clang loop unroll(disable)
  for (int c = 0; c < nc; ++c) {
    switch (wave) {   // uniform
      case 4: wait_vmcnt<C::wait(4)>(); break;
      case 5: wait_vmcnt<C::wait(5)>(); break;
      case 6: wait_vmcnt<C::wait(6)>(); break;
      case 7: wait_vmcnt<C::wait(7)>(); break;
      default: break;   // compute waves hold no loads
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
      for (int j = 0; j < 4; ++j) wf[j] = frag(ws + 16 * (cs0 + j) * BK, off0, off1);
      // two row subtiles at a time: their MFMAs, then their folds, so that no
      // fold waits for the matrix unit and at most 8 results are live
#pragma unroll
      for (int q0 = 0; q0 < Q; q0 += 2) {
        v4f pc[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = q0 + u;
          if (q < Q && valid(q)) {
            const v8i af = frag(as + 16 * (kRowStep * q + rs0) * BK, off0, off1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              pc[u][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], af, zero, 0, 0, 0, 0, 0, 0);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int q = q0 + u;
          if (q < Q && valid(q)) {
            const float sc = sas[16 * (kRowStep * q + rs0) + l16] * swv;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[q][j][r] = __builtin_fmaf(pc[u][j][r], sc, acc[q][j][r]);
          }
        }
      }
    }
  }
  // the repeated loads after the last chunk must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if constexpr (!C::kWide) {
    if (!computes) return;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int r = 16 * (kRowStep * q + rs0) + l16;
      if (valid(q) && r < me) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<uint2*>(p.out + (int64_t)(m0 + r) * p.ldo + n0 + 16 * j + 4 * lq) = bf16x4(acc[q][j]);
      }
    }
  } else {
    // The two K halves of this slice meet through the workspace. Partial sums
    // and the counter are device-coherent accesses (sc1: written through to,
    // and read from, the level all XCDs share): a half's stores are complete
    // (vmcnt(0)) before its counter increment, and the other half reads them
    // only after it has seen that increment.
    // Layout: each 16 x 16 accumulator subtile (row subtile rs, column
    // subtile cs of the slice) is one 1 KB block, lane L's four values at
    // 16 L bytes, so a store or load instruction moves one whole block; the
    // slice's blocks (rs, cs) lie at (8 rs + cs) KB, t16 x 8 KB per slice, the
    // expert's n / 128 slices in a row, the split experts one after the other,
    // each K half's share of the workspace after the other's.
    const int t16 = (me + 15) / 16;
    uint32_t* cnt = p.cnt + e * kDecodeSlices + (int)(n0 / kDN2);
    int* flag = reinterpret_cast<int*>(smem + C::kSwOff + C::kWStages * 16);
    const int64_t col = n0 + 16 * cs0 + 4 * lq;       // + 16 j: this lane's output columns
    auto region = [&](int half) {
      const float* base = p.part + ((int64_t)half * p.part_subtiles + p.part_off[e]) * 16 * p.n;
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)(t16 * 16 * p.n * 4), 0x00020000);
    };
    const uint32_t lane_off = (uint32_t)(n0 / kDN2) * (uint32_t)t16 * 8192u + (uint32_t)lane * 16u;
    __syncthreads();                                   // every wave is past its last LDS read
    if (tid == 0) *flag = (int)__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    bool last = *flag == 1;                            // the other half has finished: add its sums
    if (!last) {
      const auto rm = region(h);
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int rs = kRowStep * q + rs0;
        if (computes && rs < t16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[q][j]), rm,
                                                   lane_off + (uint32_t)(8 * rs + cs0 + j) * 1024u, 0, kSc1);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();                                 // every wave's partial sums are stored
      if (tid == 0)
        *flag = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      last = *flag == 1;
    }
    if (!last) return;                                 // uniform: the other half finishes the slice
    if (computes) {
      const auto ro = region(1 - h);
      // four row subtiles at a time: all their loads, then their sums and stores
#pragma unroll
      for (int q0 = 0; q0 < Q; q0 += 4) {
        v4f oth[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rs = kRowStep * (q0 + u) + rs0;
          if (q0 + u < Q && rs < t16) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              oth[u][j] = __builtin_bit_cast(
                  v4f, __builtin_amdgcn_raw_buffer_load_b128(ro, lane_off + (uint32_t)(8 * rs + cs0 + j) * 1024u, 0, kSc1));
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q0 + u;
          const int r = 16 * (kRowStep * q + rs0) + l16;
          if (q < Q && kRowStep * q + rs0 < t16 && r < me) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              *reinterpret_cast<uint2*>(p.out + (int64_t)(m0 + r) * p.ldo + col + 16 * j) = bf16x4(acc[q][j] + oth[u][j]);
          }
        }
      }
    }
    if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
  }
}

// Row subtile counts with a compiled configuration: the next one at or above t16.
template <int CW>
__device__ __forceinline__ void dispatch_rows(const DecodeArgs& p, uint8_t* smem, int e, int64_t n0, int kc0,
                                              int kc1, int h, int m0, int me, int t16) {
  if constexpr (CW == kDN) {
    if (t16 <= 1) { decode_slice<1, CW>(p, smem, e, n0, kc0, kc1, h, m0, me); return; }
    if (t16 <= 2) { decode_slice<2, CW>(p, smem, e, n0, kc0, kc1, h, m0, me); return; }
  }
  if (t16 <= 3) decode_slice<3, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else if (t16 <= 4) decode_slice<4, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else if (t16 <= 6) decode_slice<6, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else if (t16 <= 8) decode_slice<8, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else if (t16 <= 10) decode_slice<10, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else if (t16 <= 12) decode_slice<12, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else if (t16 <= 14) decode_slice<14, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
  else decode_slice<16, CW>(p, smem, e, n0, kc0, kc1, h, m0, me);
}

// BIG: the launch holds an expert of more than 32 rows (all configurations,
// the largest LDS); otherwise only the 1- and 2-subtile configurations.
template <bool BIG>
__global__ __launch_bounds__(512) void gemm_decode_kernel(DecodeArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[BIG ? kBigBytes : kSmallBytes];

  // workgroup -> (expert, slice), expert-major: the hardware deals consecutive
  // workgroups to the 8 XCDs in turn, so each expert's slices spread over all
  // XCDs and a large expert does not load one XCD alone. A split expert's
  // workgroups 2 s and 2 s + 1 are the two K halves of its 128-column slice s.
  const int f = blockIdx.x;
  const int e = f / p.slices, local = f % p.slices;
  const int m0 = p.row_off[e];
  const int me = p.row_off[e + 1] - m0;
  // uniform per workgroup: an empty expert has nothing to do
  if (me <= 0) return;
  const int t16 = (me + 15) / 16;
  const int nc = (int)(p.k / BK);
  if (p.split[e]) {
    if constexpr (BIG) {
      const int h = local & 1, half = nc / 2;
      dispatch_rows<kDN2>(p, smem, e, (int64_t)(local >> 1) * kDN2, h ? half : 0, h ? nc : half, h, m0, me, t16);
    }
  } else if (t16 <= 2) {
    dispatch_rows<kDN>(p, smem, e, (int64_t)local * kDN, 0, nc, 0, m0, me, t16);
  } else {
    if constexpr (BIG) dispatch_rows<kDN>(p, smem, e, (int64_t)local * kDN, 0, nc, 0, m0, me, t16);
  }
}

}  // namespace

// 16-row subtiles of the experts that run split (more than 32 rows).
static int64_t split_subtiles(int groups, const int64_t* row_off) {
  int64_t t = 0;
  for (int e = 0; e < groups; ++e) {
    const int64_t rows = row_off[e + 1] - row_off[e];
    if (rows > 32) t += (rows + 15) / 16;
  }
  return t;
}

int64_t grouped_gemm_decode_workspace(int groups, const int64_t* row_off, int64_t n, int64_t k) {
  if (k / BK < 2 || n / kDN2 > kDecodeSlices) return 0;
  const int64_t t = split_subtiles(groups, row_off);
  if (t == 0) return 0;
  // the counters first, at the same place for every call (kMaxGroups x
  // kDecodeSlices words), then each K half's partial sums of the split
  // experts' 16-row subtiles
  return kDecodeCounterBytes + 2 * t * 16 * n * 4;
}

hipError_t launch_grouped_gemm_decode(int groups, const int64_t* row_off, int64_t n, int64_t k,
                                      const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                      const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                                      uint16_t* out, int64_t ldo, void* workspace, hipStream_t st) {
  DecodeArgs p;
  p.n = n; p.k = k; p.m = row_off[groups];
  p.a = a; p.lda = lda; p.sa = sa; p.ldsa = ldsa;
  p.b = b; p.ldb = ldb; p.sb = sb; p.ldsb = ldsb;
  p.out = out; p.ldo = ldo;
  p.groups = groups;
  p.slices = (int)(n / kDN);
  const bool can_split = workspace != nullptr && k / BK >= 2 && n / kDN2 <= kDecodeSlices;
  p.cnt = static_cast<uint32_t*>(workspace);
  p.part = can_split ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kDecodeCounterBytes) : nullptr;
  int64_t most = 0;
  for (int e = 0; e <= groups; ++e) p.row_off[e] = (int)row_off[e];
  int subtiles = 0;
  for (int e = 0; e < groups; ++e) {
    const int64_t rows = row_off[e + 1] - row_off[e];
    most = rows > most ? rows : most;
    p.split[e] = (uint8_t)(can_split && rows > 32 ? 1 : 0);
    p.part_off[e] = subtiles;
    if (p.split[e]) subtiles += (int)((rows + 15) / 16);
  }
  p.part_subtiles = subtiles;
  for (int e = groups; e < kMaxGroups; ++e) { p.split[e] = 0; p.part_off[e] = subtiles; }
  if (most == 0) return hipSuccess;
  const dim3 grid((unsigned)(groups * p.slices)), block(512);
  if (most <= 32) hipLaunchKernelGGL(gemm_decode_kernel<false>, grid, block, 0, st, p);
  else            hipLaunchKernelGGL(gemm_decode_kernel<true>, grid, block, 0, st, p);
  return hipGetLastError();
}


namespace {
constexpr int kScratchDevices = 64;
std::once_flag g_scratch_once[kScratchDevices];
void* g_scratch_ptr[kScratchDevices];
hipError_t g_scratch_err[kScratchDevices];
}  // namespace

hipError_t launch_grouped_gemm_decode_noalloc(int groups, const int64_t* row_off, int64_t n, int64_t k,
                                              const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                                              const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                                              uint16_t* out, int64_t ldo, hipStream_t st) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  // once per device, with that device current: the address of its copy
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  return launch_grouped_gemm_decode(groups, row_off, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, ldo,
                                    g_scratch_ptr[dev], st);
}

}  // namespace fp8bq
