/*
 * fp8bq -- fine-grained FP8 (E4M3) quantisation and block-scaled FP8 GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the FP8 mixed-precision Linear of the DeepSeek-V3 report
 * (Chinese translation, chapter 3 "Infrastructure"):
 *   - section 3.3.2 "fine-grained quantization" and Figure 7a: activations are
 *     scaled per 1x128 tile (one token, 128 channels), weights per 128x128
 *     block; the scales run along the GEMM's inner dimension K;
 *   - section 3.3.2 "online quantization": the max-abs of every tile / block is
 *     taken on the fly, the scale is derived from it and the data is cast to
 *     FP8 at once (the tech note "DeepSeek-V3 FP8 dynamic quantisation" gives
 *     s = absmax / F_max and q = round(x / s));
 *   - section 3.3.2 "mantissa over exponents": E4M3 for every tensor;
 *   - section 3.3.2 "increasing accumulation precision" and Figure 7b: the
 *     partial sum of every N_C = 128 K-elements is promoted to an FP32
 *     accumulator, where it is multiplied by both operands' scales;
 *   - section 3.3.1 and Figure 6: Fprop, Dgrad and Wgrad all run in FP8 and
 *     produce BF16 or FP32;
 *   - section 3.3.3 "low-precision activations" / 3.5.2 "transposed GEMM":
 *     the weight-gradient GEMM needs the tiles along the token dimension
 *     (128x1);
 *   - section 3.3.3 "low-precision communication": the MoE up-projection runs
 *     an FP8 Fprop per expert.
 *
 * Numerics (the same on every entry point):
 *   FP8 is OCP E4M3FN (largest finite 448, no infinities, 0x7F/0xFF NaN).
 *   s = fl32(absmax / 448) (IEEE binary32 quotient, round-to-nearest-even);
 *   q = E4M3 round-to-nearest-even of fl32(x / s), saturating to +-448, sign
 *   kept for zeros; a tile whose absmax is 0 gets s = 0 and codes +0 / -0.
 *   With FP8BQ_SCALE_POW2 (section 3.3.3 "low-precision storage and
 *   communication": scaling factors that are integral powers of 2) the scale
 *   is instead s = 2^k, k the smallest integer with absmax <= 448 * 2^k,
 *   clamped to [-127, 127] (an E8M0 exponent byte); an all-zero tile gets
 *   s = 2^-127; q = E4M3 round-to-nearest-even of the exact x * 2^-k.
 *   Inputs must be finite (NaN / Inf give unspecified codes and outputs).
 *
 * Conventions:
 *   - All matrices are row-major with an explicit leading dimension (ld, in
 *     elements). bf16 data is passed as raw 16-bit patterns.
 *   - Every pointer except `row_off` of fp8bq_grouped_gemm is a DEVICE pointer
 *     owned by the caller. The library never allocates or frees memory and
 *     keeps no device state; outputs must not alias inputs.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work and return; results are ready when the stream has run it.
 *   - Arguments are validated on the host before any GPU call. The return
 *     value is an fp8bq_status; on any status other than FP8BQ_OK nothing was
 *     enqueued and fp8bq_last_error() (thread-local) describes the problem.
 *   - Alignment: data pointers 16-byte aligned; bf16 leading dimensions
 *     multiples of 8, FP8 leading dimensions multiples of 16, float scale
 *     pointers 4-byte aligned.
 */
#ifndef FP8BQ_H
#define FP8BQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8BQ_OK = 0,
  FP8BQ_E_INVAL = 1,   /* null pointer, non-positive size, ld too small, bad enum */
  FP8BQ_E_SHAPE = 2,   /* a dimension is not a multiple of 128 where required, bad group offsets */
  FP8BQ_E_ALIGN = 3,   /* pointer or leading dimension misaligned */
  FP8BQ_E_DEVICE = 4,  /* no HIP device, or the current device is not gfx950 */
  FP8BQ_E_HIP = 5      /* the HIP runtime reported an error when launching */
} fp8bq_status;

typedef enum {
  FP8BQ_FPROP = 0,     /* Y = X W^T : B block-scaled [N/128][K/128], bf16 out   */
  FP8BQ_DGRAD = 1,     /* dX = dY W : B = W^T, scales = W's grid,   bf16 out    */
  FP8BQ_WGRAD = 2      /* dW = dY^T X : B row-scaled [K/128][N],    fp32 out    */
} fp8bq_op;

enum { FP8BQ_ACT_ROWWISE = 0, FP8BQ_ACT_COLWISE = 1 };

/* Flag: power-of-two scales. OR-ed into the mode of fp8bq_quant_act_1x128,
   passed as `flags` to fp8bq_quant_w_128x128, OR-ed into the op of
   fp8bq_gemm (which then applies the scales inside the matrix instruction). */
enum { FP8BQ_SCALE_POW2 = 0x10 };

/*
 * Online activation quantisation (report section 3.3.2, Figure 7a; for the
 * column-wise mode section 3.3.3 "low-precision activations" and 3.5.2).
 *
 * x      bf16 [rows, cols], leading dimension ldx >= cols.
 * mode   FP8BQ_ACT_ROWWISE: 1x128 tiles along each row (cols % 128 == 0).
 *          q  E4M3 [rows, cols], ldq >= cols.
 *          s  float, tile (r, c) -- row r, columns [128c, 128c+128) -- at
 *             s[c * lds + r], lds >= rows ("chunk-major").
 *        FP8BQ_ACT_COLWISE: 128x1 tiles along each column (rows % 128 == 0,
 *          cols % 128 == 0); the result is written transposed so that the
 *          grouped (token) dimension is contiguous:
 *          q  E4M3 [cols, rows], ldq >= rows; q[j * ldq + r] encodes x[r][j].
 *          s  tile (rows [128c, 128c+128), column j) at s[c * lds + j],
 *             lds >= cols.
 *        Either mode may be OR-ed with FP8BQ_SCALE_POW2 (power-of-two scales).
 * Errors: E_INVAL (null, rows/cols <= 0, ld too small, bad mode), E_SHAPE,
 *         E_ALIGN, E_DEVICE, E_HIP.
 */
int fp8bq_quant_act_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx, int mode,
                          void* q, int64_t ldq, float* s, int64_t lds, void* stream);

/*
 * E5M6 activation cache, 1x128 tiles (report section 3.3.3 "low-precision
 * storage and communication", low-precision activations, item 1: the inputs of
 * the Linear after the attention operator are cached in a custom 12-bit E5M6
 * format, with power-of-two scaling factors so that turning the 1x128 tiles
 * into 128x1 tiles in the backward pass adds no error).
 *
 * Format: 1 sign, 5 exponent (bias 15), 6 mantissa bits, the layout of IEEE
 * binary16 without its four lowest mantissa bits; exponent field 0 holds
 * subnormals m * 2^-20; largest finite value 65024; field 31 is never written.
 * Tile scale s = 2^k, k the smallest integer with the tile's absmax <= 65024 *
 * 2^k, within [-127, 127] (2^-127 for an all-zero tile); codes
 * E5M6(x * 2^-k), the product exact, rounded to nearest even once, sign kept.
 *
 * x     bf16 [rows, cols], ldx >= cols (elements, multiple of 8).
 * q     packed codes: row r at q + r * ldq (bytes), 1.5 * cols bytes per row;
 *       elements 2i and 2i+1 of a row share bytes 3i .. 3i+2 (element 2i in
 *       bits 0..11 of the little-endian 24-bit group). ldq >= 1.5 * cols, a
 *       multiple of 16.
 * s     float, tile (r, c) at s[c * lds + r], lds >= rows.
 * cols must be a multiple of 128. The caller owns all buffers.
 * Errors: E_INVAL (null, sizes <= 0, ld too small), E_SHAPE, E_ALIGN (x and q
 *         16-byte aligned, s 4-byte aligned), E_DEVICE, E_HIP.
 */
int fp8bq_cache_e5m6_1x128(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                           void* q, int64_t ldq, float* s, int64_t lds, void* stream);

/*
 * The inverse of fp8bq_cache_e5m6_1x128: y = bf16 round-to-nearest-even of
 * E5M6(code) * s (the product is exact; it is the cached value itself whenever
 * that lies in bf16's normal range). q, ldq, s, lds as written by the cache
 * call; y bf16 [rows, cols], ldy >= cols (elements, multiple of 8), 16-byte
 * aligned. Errors as fp8bq_cache_e5m6_1x128.
 */
int fp8bq_uncache_e5m6_1x128(const void* q, int64_t rows, int64_t cols, int64_t ldq,
                             const float* s, int64_t lds, void* y, int64_t ldy, void* stream);

/*
 * The backward use of the E5M6 cache (report section 3.3.3, low-precision
 * activations, item 1: the cached 1x128 tiles are turned into 128x1 tiles for
 * the backward pass, and with power-of-two scales the conversion itself adds
 * no quantisation error): the cached values x_hat = E5M6(code) * s, exact, are
 * re-quantised to E4M3 in 128x1 tiles (128 consecutive rows of one column) and
 * written transposed, ready to be the activation operand of the Wgrad GEMM.
 *
 * q, ldq, s, lds  as written by fp8bq_cache_e5m6_1x128: s must hold powers of
 *       two 2^kc with -127 <= kc <= 113 (the range the cache writes for finite
 *       bf16 input; only the exponent is read) and codes must be finite
 *       (exponent field below 31). The values are then formed exactly in fp32
 *       as E5M6(code) * 2^(kc - 2), which stays within [2^-149, 2^127).
 * qt    E4M3 [cols, rows], ldqt >= rows: qt[j * ldqt + r] encodes column j,
 *       row r (the layout fp8bq_quant_act_1x128 writes in COLWISE mode).
 * st    float, scale of tile (rows [128c, 128c+128), column j) at
 *       st[c * ldst + j], ldst >= cols: 2^k with k the smallest integer such
 *       that the tile's absmax <= 448 * 2^k, within [-127, 127] (2^-127 for
 *       an all-zero tile); codes E4M3(fl32(x_hat * 2^-k)), nearest even, sign
 *       kept. With x_hat in bf16's normal range this is bit for bit
 *       fp8bq_quant_act_1x128 (COLWISE | FP8BQ_SCALE_POW2) of the bf16 values
 *       that fp8bq_uncache_e5m6_1x128 returns.
 * rows and cols must be multiples of 128. The caller owns all buffers; the
 * inputs must not overlap the outputs.
 * Errors: E_INVAL (null, sizes <= 0, ld too small), E_SHAPE, E_ALIGN (q, qt
 *         16-byte aligned; ldq, ldqt multiples of 16; scales 4-byte aligned),
 *         E_DEVICE, E_HIP.
 */
int fp8bq_requant_e5m6_t_128x1(const void* q, int64_t rows, int64_t cols, int64_t ldq, const float* s,
                               int64_t lds, void* qt, int64_t ldqt, float* st, int64_t ldst, void* stream);

/*
 * Transposing re-quantisation of an FP8 activation cache, 1x128 -> 128x1
 * (report section 3.5.2 "support for transposed GEMM": the forward pass keeps
 * activations as 1x128 FP8 tiles, the backward pass reads them, dequantises,
 * transposes and quantises them again as 128x1 tiles; section 3.3.3 gives
 * these activations power-of-two scales so the conversion adds no error of
 * its own).
 *
 * q     E4M3 [rows, cols], ldq >= cols, as written by fp8bq_quant_act_1x128
 *       in ROWWISE mode (any scales: the dequantised value dec(q) * s is
 *       formed exactly).
 * s     float, tile (r, c) at s[c * lds + r], lds >= rows.
 * qt    E4M3 [cols, rows], ldqt >= rows: qt[j * ldqt + r] encodes column j,
 *       row r (the layout of COLWISE mode, ready to be a Wgrad operand).
 * st    float, power-of-two scale of tile (rows [128c, 128c+128), column j)
 *       at st[c * ldst + j], ldst >= cols: 2^k with k the smallest integer
 *       such that the tile's absmax <= 448 * 2^k, within [-127, 127] (2^-127
 *       for an all-zero tile); codes are E4M3(fl32(x_hat * 2^-k)).
 * flags 0, or FP8BQ_SCALE_POW2 when the scales in s are powers of two (as
 *       fp8bq_quant_act_1x128 writes them with that flag): a kernel specialised
 *       for that case, which forms x_hat in binary32 wherever that is exact.
 *       The outputs are the same for either value (each 128-row block checks
 *       its own scales), so the flag is only a hint.
 * rows and cols must be multiples of 128.
 * The caller owns all buffers; q/s and qt/st must not overlap.
 * Errors: E_INVAL (null, sizes <= 0, ld too small, unknown flags), E_SHAPE,
 *         E_ALIGN (q, qt 16-byte aligned; ldq, ldqt multiples of 16; scales
 *         4-byte aligned), E_DEVICE, E_HIP.
 */
int fp8bq_requant_t_128x1(const void* q, int64_t rows, int64_t cols, int64_t ldq, const float* s, int64_t lds,
                          void* qt, int64_t ldqt, float* st, int64_t ldst, int flags, void* stream);

/*
 * Online weight quantisation with 128x128 blocks (report section 3.3.2,
 * Figure 7a: per 128 input channels x 128 output channels).
 *
 * w      bf16 [n, k], ldw >= k; n % 128 == 0 and k % 128 == 0.
 * q      E4M3 [n, k], ldq >= k.
 * s      float block grid: block (nb, kb) at s[nb * lds + kb], lds >= k/128.
 * qt     optional (may be NULL): the transposed FP8 copy [k, n], ldqt >= n,
 *        qt[j * ldqt + i] == q[i * ldq + j]. It is the B operand of the Dgrad
 *        GEMM (block quantisation commutes with transposition).
 * flags  0 (s = absmax / 448) or FP8BQ_SCALE_POW2 (power-of-two scales).
 * Errors: as above; E_INVAL for unknown flags.
 */
int fp8bq_quant_w_128x128(const void* w, int64_t n, int64_t k, int64_t ldw,
                          void* q, int64_t ldq, float* s, int64_t lds,
                          void* qt, int64_t ldqt, int flags, void* stream);

/*
 * Block-scaled FP8 GEMM with per-128-K-chunk promotion (report section 3.3.2
 * "increasing accumulation precision", Figure 7b; section 3.3.1, Figure 6):
 *
 *   out[i][j] = sum_c ( sum_{k in chunk c} dec(a[i][k]) * dec(b[j][k]) ) * sa(i,c) * sb(j,c)
 *
 * accumulated in FP32; each chunk is 128 consecutive k. Both operands are
 * stored with k contiguous ("TN"): a E4M3 [m, k] (lda >= k), b E4M3 [n, k]
 * (ldb >= k). k % 128 == 0 and n % 128 == 0; m >= 1 is free.
 *
 * sa     row scales of a, chunk-major: sa(i, c) = sa[c * ldsa + i], ldsa >= m
 *        (the layout fp8bq_quant_act_1x128 writes).
 * sb     op FPROP: block grid of the weight b: sb(j, c) = sb[(j/128) * ldsb + c],
 *                  ldsb >= k/128 (the layout fp8bq_quant_w_128x128 writes).
 *        op DGRAD: b is the transposed copy qt of a weight W [k, n] and sb is
 *                  W's own block grid: sb(j, c) = sb[c * ldsb + j/128],
 *                  ldsb >= n/128.
 *        op WGRAD: row scales of b, chunk-major: sb(j, c) = sb[c * ldsb + j],
 *                  ldsb >= n (column-wise activation quantisation output).
 * out    FPROP / DGRAD: bf16 [m, n] (round-to-nearest-even), ldo >= n.
 *        WGRAD: float [m, n], ldo >= n.
 * Scale range (general scales): each chunk's partial sum is multiplied by the
 *        binary32 product fl32(sa(i,c) * sb(j,c)) and added with one FMA. A
 *        product below 2^-126 is an fp32 subnormal with fewer significant
 *        bits; its rounding adds at most |P_c| * 2^-150, so the accuracy bound
 *        |out - exact| <= 2e-3 * sum_k |a_hat_k||b_hat_k| holds for products
 *        down to 2^-140 (tested at 2^-135). Smaller products (operand tiles
 *        whose absmax values multiply to less than about 2^-122) lose accuracy
 *        gradually; the result is then still finite.
 * op | FP8BQ_SCALE_POW2: every scale of sa and sb is a power of two in
 *        [2^-127, 2^127], as the quantisers write with FP8BQ_SCALE_POW2 (only
 *        the exponent field is read; other scales give wrong results). The
 *        scales are applied inside the matrix instruction (E8M0 block scales)
 *        and each chunk's scaled sum is accumulated in FP32 by the matrix unit
 *        itself, which adds it in blocks of 8 products rather than in one
 *        rounding (report section 3.3.2 asks hardware for exactly this
 *        "MMA with group scaling"; error measured against the oracle).
 * Errors: as above.
 */
int fp8bq_gemm(int op, int64_t m, int64_t n, int64_t k,
               const void* a, int64_t lda, const float* sa, int64_t ldsa,
               const void* b, int64_t ldb, const float* sb, int64_t ldsb,
               void* out, int64_t ldo, void* stream);

/*
 * fp8bq_gemm (FPROP or DGRAD) whose epilogue also quantises the bf16 output as
 * the activation operand of the next GEMM: producer fusion of the 1x128
 * quantisation (report section 3.5.2 "online quantization support": without
 * it the output is written to HBM, read back, quantised, written again and
 * read once more by the next matrix multiply).
 *
 * op, m, n, k, a, lda, sa, ldsa, b, ldb, sb, ldsb: as fp8bq_gemm; op is
 *        FP8BQ_FPROP or FP8BQ_DGRAD, optionally | FP8BQ_SCALE_POW2 (input
 *        scales applied by the matrix instruction).
 * out    bf16 [m, n] (ldo >= n) as fp8bq_gemm writes it, or NULL when only
 *        the quantised copy is wanted.
 * q, s   E4M3 [m, n] (ldq >= n) and chunk-major scales s[c * lds + row]
 *        (lds >= m): bit for bit what fp8bq_quant_act_1x128 in ROWWISE mode
 *        (| qflags) writes for the bf16 output.
 * qflags 0 (s = absmax / 448) or FP8BQ_SCALE_POW2 (power-of-two scales).
 * Errors: as fp8bq_gemm (out may be NULL); E_INVAL for a WGRAD op, unknown
 *         qflags, null q or s, ldq < n or lds < m; E_ALIGN unless q is
 *         16-byte aligned with ldq a multiple of 16 and s 4-byte aligned.
 */
int fp8bq_gemm_quant(int op, int64_t m, int64_t n, int64_t k,
                     const void* a, int64_t lda, const float* sa, int64_t ldsa,
                     const void* b, int64_t ldb, const float* sb, int64_t ldsb,
                     void* out, int64_t ldo, void* q, int64_t ldq, float* s, int64_t lds,
                     int qflags, void* stream);

/*
 * Grouped (per-expert) Fprop for the MoE up-projection (report section 3.3.3
 * "low-precision communication": FP8 Fprop of the dispatched activations).
 *
 * groups   G >= 1 experts, G <= 256.
 * row_off  HOST array of G + 1 int64: expert e owns rows [row_off[e],
 *          row_off[e+1]) of a and out; row_off[0] == 0, non-decreasing, every
 *          entry a multiple of 128 (pad each expert's rows, e.g. with zeros).
 *          m = row_off[G].
 * a, sa    E4M3 [m, k] with chunk-major row scales (as fp8bq_gemm), ldsa >= m.
 * b        G weights of [n, k] each, row stride ldb, expert e's at b + e*n*ldb.
 * sb       G block grids [n/128][k/128], row stride ldsb, expert e's at
 *          sb + e*(n/128)*ldsb.
 * out      bf16 [m, n], ldo >= n.
 * flags    0, or FP8BQ_SCALE_POW2 for power-of-two scales applied by the matrix
 *          instruction (as fp8bq_gemm with op | FP8BQ_SCALE_POW2).
 * Errors: as above; E_SHAPE for bad offsets, E_INVAL for unknown flags.
 */
int fp8bq_grouped_gemm(int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                       const void* a, int64_t lda, const float* sa, int64_t ldsa,
                       const void* b, int64_t ldb, const float* sb, int64_t ldsb,
                       void* out, int64_t ldo, int flags, void* stream);

/*
 * Grouped Fprop for decode-sized expert batches (report section 3.4.2
 * "decoding stage": each expert then sees a small batch, at most about 256
 * tokens, and the step is bound by memory access, chiefly the experts' FP8
 * weights). Same operation, operands and scales as fp8bq_grouped_gemm, but the
 * experts' rows are not padded: row_off may hold any non-decreasing offsets
 * with row_off[0] == 0 and at most 256 rows per expert (an expert may be
 * empty). The kernel streams each expert's weight once; it is the memory-bound
 * counterpart of fp8bq_grouped_gemm.
 *
 * flags  must be 0 (scales are applied as floats by the FP32 promotion, which
 *        power-of-two scales satisfy too).
 * Errors: as fp8bq_grouped_gemm; E_SHAPE for a group of more than 256 rows.
 */
int fp8bq_grouped_gemm_decode(int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                              const void* a, int64_t lda, const float* sa, int64_t ldsa,
                              const void* b, int64_t ldb, const float* sb, int64_t ldsb,
                              void* out, int64_t ldo, int flags, void* stream);

/*
 * Bytes of workspace fp8bq_grouped_gemm_decode_ws needs for these experts and
 * shapes: 256 KiB of counters (one per expert and 128-column slice, at the
 * same place in every call) and 8 * m * n bytes of partial sums; 0 when no
 * expert has more than 32 rows, k < 256 or n > 32768 (nothing is split then). Arguments as fp8bq_grouped_gemm_decode; *bytes receives the size.
 * Errors: E_INVAL (null bytes or row_off, groups out of range), E_SHAPE (bad
 * offsets, as fp8bq_grouped_gemm_decode).
 */
int fp8bq_grouped_gemm_decode_workspace_size(int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                                             int64_t* bytes);

/*
 * fp8bq_grouped_gemm_decode with a workspace. Experts of more than 32 rows
 * then run as pairs of workgroups over the two halves of K, each for 128
 * output columns (half the activation bytes per output column of the
 * 64-column, full-K workgroups, which bound the larger experts): each half
 * stores its FP32 partial sums in the workspace and the second to finish adds
 * the other's and writes the bf16 output. The result is deterministic (a sum
 * of two terms does not depend on their order) and differs from
 * fp8bq_grouped_gemm_decode's only in the order the FP32 chunk sums are added.
 *
 * workspace        device memory of at least workspace_bytes >= the size
 *                  fp8bq_grouped_gemm_decode_workspace_size gives (NULL allowed
 *                  when that size is 0), 16-byte aligned, owned by the caller.
 *                  It must be zero-filled before its first use; every call
 *                  leaves its counters zero again, so a workspace is reused
 *                  without clearing. Calls that share a workspace must not run
 *                  concurrently (they would share counters).
 * Other arguments and errors as fp8bq_grouped_gemm_decode; E_INVAL for a
 * missing or too small workspace, E_ALIGN for a misaligned one.
 */
int fp8bq_grouped_gemm_decode_ws(int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                                 const void* a, int64_t lda, const float* sa, int64_t ldsa,
                                 const void* b, int64_t ldb, const float* sb, int64_t ldsb,
                                 void* out, int64_t ldo, void* workspace, int64_t workspace_bytes,
                                 int flags, void* stream);

/*
 * fp8bq_grouped_gemm_decode_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the workspace is the library's own scratch, a static device
 * array of 32 MiB (FP8BQ_DECODE_NOALLOC_SCRATCH_BYTES) on each device the
 * library runs on, held until the process ends. The call allocates nothing.
 * Results are bit for bit those of fp8bq_grouped_gemm_decode_ws.
 *
 * Every call on a device shares that device's scratch: calls that overlap on
 * one device (e.g. on two streams) race. The scratch's counters start at zero
 * and every call leaves them at zero.
 * Arguments as fp8bq_grouped_gemm_decode. Errors as fp8bq_grouped_gemm_decode;
 * E_SHAPE when the workspace these experts need
 * (fp8bq_grouped_gemm_decode_workspace_size) exceeds the scratch.
 */
enum { FP8BQ_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20 };
int fp8bq_grouped_gemm_decode_noalloc(int32_t groups, const int64_t* row_off, int64_t n, int64_t k,
                                      const void* a, int64_t lda, const float* sa, int64_t ldsa,
                                      const void* b, int64_t ldb, const float* sb, int64_t ldsb,
                                      void* out, int64_t ldo, int flags, void* stream);

/* Thread-local description of the last non-OK status on this thread. */
const char* fp8bq_last_error(void);

/* Library version string. */
const char* fp8bq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BQ_H */
