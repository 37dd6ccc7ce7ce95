/*
 * hr.h -- C ABI of libhr.so: randomized Hadamard rotation, fused int4 (and
 * int8) quantization, HARP-style butterfly, int4 dequant and the W4A4 (and
 * W4A8) GEMM on AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array argument is a DEVICE pointer owned by the caller; the library
 *   allocates no memory and keeps no state between calls.
 * - Every call is asynchronous: it enqueues kernels on `stream` (a
 *   hipStream_t; NULL means the null stream) and returns.  Buffers must stay
 *   valid until the stream has executed the work.
 * - Arguments are validated on the host before anything is enqueued.  A call
 *   that returns an error has enqueued nothing and made no HIP call:
 *     HR_EINVAL        null pointer where one is required, negative size,
 *                      pointer not 16-byte aligned, unknown dtype code;
 *     HR_EUNSUPPORTED  a size or mode outside what the kernels implement;
 *     HR_EDEVICE       the kernel launch itself failed (hipGetLastError).
 *   hr_last_error() returns a message describing the most recent failure of
 *   the calling thread.
 * - rows == 0 (or M == 0 or N == 0) is a valid no-op that returns HR_OK once
 *   the scalar arguments are valid; the arrays sized by it may then be NULL.
 * - Calls are thread-safe; concurrent calls on different streams are fine.
 * - Rows are contiguous and row-major: row r of an [rows][n] array starts at
 *   element r*n.
 * - int4 codes are packed two per byte, two's complement, element 2j in the
 *   low nibble and element 2j+1 in the high nibble; the quantizer produces
 *   codes in [-7, 7] only.
 *
 * Notation: x a row of length n; d a +-1 sign diagonal; H_p the Sylvester-
 * Hadamard matrix of order p = 2^k in natural order, H[i][j] =
 * (-1)^popcount(i & j); O an m x m orthogonal block; G the group size.
 */
#ifndef HR_H
#define HR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HR_OK = 0,
  HR_EINVAL = 1,
  HR_EUNSUPPORTED = 2,
  HR_EDEVICE = 3
} hr_status;

typedef enum {
  HR_F32 = 0,   /* IEEE binary32 */
  HR_BF16 = 1,  /* bfloat16 */
  HR_F16 = 2    /* IEEE binary16 */
} hr_dtype;

/* ABI version of this header (bumped on any signature change). */
#define HR_ABI_VERSION 5
int32_t hr_abi_version(void);

/* Identifier of the sources the library was built from (a hash of every
 * source file), for bindings that check they load a current build. */
const char* hr_build_id(void);

/* Static description of a status code. */
const char* hr_status_string(int32_t status);

/* Message of the calling thread's most recent failed call ("" if none). */
const char* hr_last_error(void);

/*
 * hr_rotate -- randomized (mixed-radix) Hadamard rotation, fp32 output.
 *
 * Defines: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy",
 * Hypothesis and Method (Q = H / sqrt(K) applied by a fast Walsh-Hadamard
 * transform then x 1/sqrt(K)); HARP abstract (the fixed randomized Hadamard
 * transform of incoherence processing; mixed-radix schedules for dimensions
 * that are not powers of two); HARP technical summary, section 2.1 (a radix
 * that is not a power of two uses a fixed orthogonal block).
 *
 * For every row r:   y[r] = (O kron H_p) (d * x[r]) / sqrt(p),   n = m * p,
 * with (O kron H)[i*p+a][j*p+b] = O[i][j] H[a][b] (chunk i of a row is elements
 * [i*p, (i+1)*p)).  m == 1 is the plain randomized Hadamard transform
 * y = H_n (d * x) / sqrt(n).
 *
 *   x       [rows][n] of x_dtype (HR_BF16 or HR_F32).
 *   y       [rows][n] fp32.  y == x is allowed when x_dtype == HR_F32
 *           (in place); any other overlap is undefined.
 *   n       row length, n = m * p with p a power of two, 64 <= p <= 16384,
 *           and n <= 16384.
 *   m       number of chunks, 1 <= m <= 16.
 *   signs   [n] int8, each +1 or -1 (other values are undefined behaviour);
 *           NULL means all +1.
 *   block   [m][m] fp32 row-major orthogonal block O; must be NULL when
 *           m == 1 and non-NULL when m > 1.  It is used as given (it is not
 *           re-orthogonalised).
 */
int32_t hr_rotate(const void* x, int32_t x_dtype, float* y, int64_t rows,
                  int32_t n, int32_t m, const int8_t* signs, const float* block,
                  void* stream);

/*
 * hr_rotate_quant_int4 -- hr_rotate fused with per-group symmetric absmax int4
 * quantization and nibble packing.  The rotated values never leave the chip.
 *
 * Defines: as hr_rotate, plus "Experiment -- Hadamard rotation for int4 (W4A4)
 * accuracy", Method (per-group symmetric integer quantize/dequantize) and
 * Verdict (per-group work belongs inside one kernel).
 *
 * For every row and every group of G consecutive rotated values y (aligned at
 * multiples of G):
 *   a   = max |y| over the group           (fp32)
 *   s32 = a / 7                             (fp32)
 *   s   = s32 rounded to fp16 (scale_dtype HR_F16) or s32 (HR_F32); stored
 *   q   = y / s rounded to nearest, clamped to [-7, 7]; 0 when s == 0.
 * Rounding ties of y / s are resolved to even; results within 1e-4 of a tie
 * may differ from a round-half-away reference.
 *
 *   codes   [rows][n/2] uint8, packed int4 (see conventions).
 *   scales  [rows][n/G] of scale_dtype (HR_F16 or HR_F32).
 *   group   G in {32, 64, 128, 256}; G must divide p.
 *   other arguments as hr_rotate.
 */
int32_t hr_rotate_quant_int4(const void* x, int32_t x_dtype, int64_t rows,
                             int32_t n, int32_t m, const int8_t* signs,
                             const float* block, int32_t group, uint8_t* codes,
                             void* scales, int32_t scale_dtype, void* stream);

/*
 * hr_rotate_quant_int8 -- hr_rotate fused with per-group symmetric absmax int8
 * quantization: the activation operand of the W4A8 GEMM.
 *
 * Defines: as hr_rotate_quant_int4, with the 8-bit case of the experiment
 * page's quantizer (Method: per-group symmetric quantization at any bit
 * width) that its W4A8 (act8/wt4) rows of Results use for the activations.
 *
 * For every row and every group of G consecutive rotated values y:
 *   a   = max |y| over the group           (fp32)
 *   s32 = a / 127                           (fp32, correctly rounded)
 *   s   = s32 rounded to fp16 (scale_dtype HR_F16) or s32 (HR_F32); stored
 *   q   = y / s rounded to nearest, clamped to [-127, 127]; 0 when s == 0.
 * Ties are resolved as in hr_rotate_quant_int4.
 *
 *   codes   [rows][n] int8, one code per element.
 *   scales  [rows][n/G] of scale_dtype (HR_F16 or HR_F32).
 *   other arguments and errors as hr_rotate_quant_int4.
 */
int32_t hr_rotate_quant_int8(const void* x, int32_t x_dtype, int64_t rows,
                             int32_t n, int32_t m, const int8_t* signs,
                             const float* block, int32_t group, int8_t* codes,
                             void* scales, int32_t scale_dtype, void* stream);

/*
 * hr_quant_int4 -- per-group symmetric absmax int4 quantization of rows that
 * are NOT rotated (the plain operand of the experiment page's comparison).
 *
 * Defines: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Method
 * (per-group symmetric integer quantize/dequantize) and Results (its table
 * quantizes each operand both plain and after the Hadamard rotation).
 *
 * For every group of G consecutive values y of a row the rule of
 * hr_rotate_quant_int4 applies: s32 = max|y| / 7, s = fp16(s32) or s32,
 * q = y / s rounded to nearest (ties to even), clamped to [-7, 7], 0 when
 * s == 0.
 *
 *   x       [rows][n] of x_dtype (HR_BF16 or HR_F32).
 *   n       a positive multiple of G, n <= 2^30.
 *   group   G in {32, 64, 128, 256}.
 *   codes   [rows][n/2] uint8 packed int4; scales [rows][n/G] of scale_dtype.
 */
int32_t hr_quant_int4(const void* x, int32_t x_dtype, int64_t rows, int32_t n, int32_t group,
                      uint8_t* codes, void* scales, int32_t scale_dtype, void* stream);

/*
 * hr_quant_int8 -- as hr_quant_int4 with qmax = 127 and one int8 code per
 * element (codes [rows][n] int8): the plain 8-bit operands of the same page's
 * W8A8 and W4A8 rows.
 */
int32_t hr_quant_int8(const void* x, int32_t x_dtype, int64_t rows, int32_t n, int32_t group,
                      int8_t* codes, void* scales, int32_t scale_dtype, void* stream);

/*
 * hr_butterfly_coeffs -- build the per-pair 2x2 coefficient table of a
 * HARP-style butterfly from its angles (run once per set of angles).
 *
 * Defines: HARP technical summary, section 2.2: block kernel
 * B(theta) = Q(theta) G_b with Q a Givens rotation for b = 2 and G_2 the
 * normalised Sylvester-Hadamard mixer; theta = 0 gives B = G_2.
 *
 * Stage s (0 <= s < log2 n) pairs elements (i, i + 2^s) for every i with bit s
 * clear; the pair's index is ((i >> (s+1)) << s) | (i & (2^s - 1)).  For pair
 * index j of stage s, with c = cos(angles[s][j]), t = sin(angles[s][j])
 * evaluated in double precision:
 *   precondition == 0:  block [[c, -t], [t, c]]          -> stores (c, t)
 *   precondition == 1:  block [[c, -t], [t, c]] G_2
 *                       = [[u, v], [v, -u]], u = (c - t)/sqrt2,
 *                         v = (c + t)/sqrt2                -> stores (u, v)
 *   angles  [log2 n][n/2] fp32.
 *   coeffs  [log2 n][n/2][2] fp32 (output; pass it to hr_butterfly_apply with
 *           the same precondition value).
 *   n       power of two, 64 <= n <= 8192.
 */
int32_t hr_butterfly_coeffs(const float* angles, int32_t n, int32_t precondition,
                            float* coeffs, void* stream);

/*
 * hr_butterfly_apply -- apply the butterfly (or its transpose) to every row,
 * optionally fused with int4 quantization of the result.
 *
 * Defines: HARP abstract (a rotation as a product of sparse butterfly-like
 * block-orthogonal stages); HARP technical summary, sections 2.1 (stages of
 * block-diagonal orthogonal matrices separated by stride permutations; here the
 * permutations are folded into the pair indexing), 2.2 (the block kernel) and
 * 2.4 (O(d log d) application without materialised permutations).
 *
 * Forward (inverse == 0): stages s = 0 .. log2(n)-1 in ascending order, each
 * block applied to (x_i, x_{i+2^s}) as a column vector, then the gather
 * y[i] = z[perm[i]].  Inverse (inverse == 1): the transpose: scatter
 * z[perm[i]] = x[i], then the transposed blocks in descending stage order.
 *
 *   x       [rows][n] fp32.
 *   y       [rows][n] fp32 output, or NULL to skip the fp32 output.  y == x is
 *           allowed (in place).
 *   coeffs  table from hr_butterfly_coeffs for the same n and precondition.
 *   precondition  0 or 1, as given to hr_butterfly_coeffs.
 *   perm    [n] int32 permutation of 0..n-1; NULL means identity.
 *   codes, scales, group, scale_dtype: as hr_rotate_quant_int4, quantizing
 *           the butterfly output; codes == NULL skips quantization (then
 *           scales must be NULL too).  At least one of y and codes must be
 *           non-NULL.  Quantization is only available with inverse == 0.
 */
int32_t hr_butterfly_apply(const float* x, float* y, int64_t rows, int32_t n,
                           const float* coeffs, int32_t precondition,
                           const int32_t* perm, int32_t inverse, int32_t group,
                           uint8_t* codes, void* scales, int32_t scale_dtype,
                           void* stream);

/*
 * hr_harp_blocks -- the dense blocks B_{t,c} = Q_{t,c}(theta) G_{b_t} of a HARP
 * processor with a general mixed-radix schedule (run once per set of
 * parameters).
 *
 * Defines: HARP technical summary, section 2.1 (a mixed-radix schedule
 * b = (b_0 .. b_{m-1}) with prod b_t = d, e.g. 5120 = (8, 8, 8, 5, 2); radices
 * that are not powers of two use a fixed orthogonal fallback from the QR
 * factorisation of a Gaussian matrix) and section 2.2 (B = Q(theta) G_b, Q a
 * Givens rotation for b = 2 and the Cayley map for b > 2, G_b the normalised
 * Sylvester-Hadamard matrix for powers of two; theta = 0 gives B = G_b).
 *
 * Stage t has d / b_t blocks.  Its parameters are [d/b_t][P_t] floats,
 * P_t = 1 for b_t = 2 (the angle th: Q = [[cos th, -sin th], [sin th, cos th]])
 * and b_t (b_t - 1) / 2 otherwise (the upper triangle A[i][j], i < j, row-major,
 * of a skew-symmetric A; Q = (I - A)^(-1) (I + A)).  Q and the product are
 * formed in double precision and stored as fp32.
 *
 *   radices    HOST array [nstages] int32, each in [2, 8]; their product d is a
 *              multiple of 4 and at most 16384; 1 <= nstages <= 16.
 *   theta      [sum_t (d / b_t) P_t] fp32, stages concatenated in order.
 *   fallbacks  [b][b] fp32 orthogonal matrices (row-major), one per stage whose
 *              radix is not a power of two, concatenated in stage order; may be
 *              NULL when every radix is a power of two.  Used as given.
 *   blocks     output [sum_t 4 K_t (d / b_t)] fp32, K_t = ceil(b_t^2 / 4), stages
 *              concatenated in order; stage t is quad-major, [K_t][d/b_t][4]:
 *              entry k = r * b_t + q of block c at ((k / 4) * (d / b_t) + c) * 4
 *              + k % 4; the K_t * 4 - b_t^2 padding entries of each block are 0.
 */
int32_t hr_harp_blocks(const int32_t* radices, int32_t nstages, const float* theta,
                       const float* fallbacks, float* blocks, void* stream);

/*
 * hr_harp_apply -- apply a HARP processor (or its transpose) to every row,
 * optionally fused with int4 quantization of the result.
 *
 * Defines: as hr_harp_blocks, plus section 2.4 of the same summary (stages
 * applied in O(d log d) work without materialised permutations).
 *
 * Write a coordinate as i = sum_t i_t S_t, S_t = b_0 ... b_{t-1}.  Forward
 * (inverse == 0): stages t = 0 .. m-1; block c = lo + S_t hi (lo < S_t) of
 * stage t maps the coordinates i_r = lo + S_t (r + b_t hi), r < b_t, by
 * y_{i_r} = sum_q B_{t,c}[r][q] x_{i_q}.  Inverse (inverse == 1): the
 * transpose, stages t = m-1 .. 0 with B^T.  With all radices 2 this is
 * hr_butterfly_apply with precondition = 1 and no permutation.
 *
 *   x       [rows][d] fp32.
 *   y       [rows][d] fp32 output, or NULL to skip it; y == x is allowed.
 *   radices, nstages  the schedule, as for hr_harp_blocks (HOST array).
 *   blocks  the table from hr_harp_blocks for the same schedule.
 *   codes, scales, group, scale_dtype: as hr_rotate_quant_int4, quantizing the
 *           processor's output; codes == NULL skips quantization (scales must
 *           then be NULL).  At least one of y and codes must be non-NULL.
 */
int32_t hr_harp_apply(const float* x, float* y, int64_t rows, const int32_t* radices,
                      int32_t nstages, const float* blocks, int32_t inverse, int32_t group,
                      uint8_t* codes, void* scales, int32_t scale_dtype, void* stream);

/*
 * hr_dequant_int4 -- x_hat = q * s per element (one fp32 product, so the result
 * is bit-exact).
 *
 * Defines: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy", Method
 * (quantize -> dequantize).
 *
 *   codes   [rows][n/2] uint8 packed int4.
 *   scales  [rows][n/G] of scale_dtype (HR_F16 or HR_F32).
 *   n       even, a multiple of G, n <= 2^30.
 *   group   G in {32, 64, 128, 256}.
 *   out     [rows][n] fp32.
 */
int32_t hr_dequant_int4(const uint8_t* codes, const void* scales,
                        int32_t scale_dtype, int64_t rows, int32_t n,
                        int32_t group, float* out, void* stream);

/*
 * hr_w4a4_gemm -- C = A W^T on packed int4 operands with per-group scales.
 *
 * Defines: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy",
 * Hypothesis (W4A4: both operands int4 on a same-precision integer MAC) and
 * Verdict (the per-group scaling must stay inside one GEMM).
 *
 *   acc[m][n][g] = sum_{k = gG}^{gG+G-1} A[m][k] W[n][k]      (exact int32)
 *   C[m][n]      = sum_g sA[m][g] sW[n][g] acc[m][n][g]       (fp32)
 *
 *   a_codes   [M][K/2] uint8 packed int4 (activations, K contiguous).
 *   a_scales  [M][K/G] of scale_dtype.
 *   w_codes   [N][K/2] uint8 packed int4 (weights, K contiguous).
 *   w_scales  [N][K/G] of scale_dtype.
 *   scale_dtype  HR_F16 or HR_F32.
 *   M >= 0; N a multiple of 64; K a multiple of 256 and of G, K <= 65536.
 *   group     G in {32, 64, 128, 256}.
 *   c         [M][N] fp32 output.
 *   group_acc optional [M][N][K/G] int32 output of the exact per-group sums
 *             (a debugging aid; NULL to skip).
 * Codes equal to -8 are accepted and multiply exactly.
 */
int32_t hr_w4a4_gemm(const uint8_t* a_codes, const void* a_scales,
                     const uint8_t* w_codes, const void* w_scales,
                     int32_t scale_dtype, int64_t M, int64_t N, int64_t K,
                     int32_t group, float* c, int32_t* group_acc, void* stream);

/*
 * hr_w4a8_gemm -- C = A W^T with int8 activation codes and packed int4
 * weights, per-group scales on both.
 *
 * Defines: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy",
 * Results (the W4A8 act8/wt4 rows: int8 activations against int4 weights)
 * and the third of its conclusions (W4A8 is far more accurate than W4A4; an
 * int8 MAC runs it directly); the sums and the scale fusion are those of
 * hr_w4a4_gemm.
 *
 *   acc[m][n][g] = sum_{k = gG}^{gG+G-1} A[m][k] W[n][k]      (exact int32)
 *   C[m][n]      = sum_g sA[m][g] sW[n][g] acc[m][n][g]       (fp32)
 *
 *   a_codes   [M][K] int8 (activations, K contiguous; hr_rotate_quant_int8
 *             output).  Every int8 value is accepted.
 *   w_codes   [N][K/2] uint8 packed int4 (weights).
 *   other arguments, sizes and errors as hr_w4a4_gemm.
 */
int32_t hr_w4a8_gemm(const int8_t* a_codes, const void* a_scales,
                     const uint8_t* w_codes, const void* w_scales,
                     int32_t scale_dtype, int64_t M, int64_t N, int64_t K,
                     int32_t group, float* c, int32_t* group_acc, void* stream);

/*
 * hr_w8a8_gemm -- C = A W^T with both operands held one int8 code per
 * element, per-group scales on both.
 *
 * Defines: "Experiment -- Hadamard rotation for int4 (W4A4) accuracy",
 * Results (the W8A8 rows: int8 activations and weights); with codes in
 * -8..7 it is the W4A4 GEMM of hr_w4a4_gemm with its codes held in int8, the
 * form an int8 MAC consumes directly (no nibble unpacking in the kernel).
 * The sums and the scale fusion are those of hr_w4a4_gemm.
 *
 *   acc[m][n][g] = sum_{k = gG}^{gG+G-1} A[m][k] W[n][k]      (exact int32)
 *   C[m][n]      = sum_g sA[m][g] sW[n][g] acc[m][n][g]       (fp32)
 *
 *   a_codes   [M][K] int8 (activations, K contiguous).
 *   w_codes   [N][K] int8 (weights, K contiguous).
 *   Every int8 value is accepted.
 *   other arguments, sizes and errors as hr_w4a4_gemm.
 */
int32_t hr_w8a8_gemm(const int8_t* a_codes, const void* a_scales,
                     const int8_t* w_codes, const void* w_scales,
                     int32_t scale_dtype, int64_t M, int64_t N, int64_t K,
                     int32_t group, float* c, int32_t* group_acc, void* stream);

/*
 * hr_w4a4_to_fp6 -- packed int4 codes (and their scales) to the tiled fp6
 * operand format that hr_w4a4_gemm_fp6 reads: the same codes and scales, held
 * where the fp6 matrix cores and the GEMM's copies take them.
 *
 * Defines: the operands of "Experiment -- Hadamard rotation for int4 (W4A4)
 * accuracy", Hypothesis (int4 codes on a same-precision MAC).
 *
 * A code q in [-8, 7] becomes the fp6 e2m3 field (q < 0) << 5 | |q| (the value
 * q / 8; exact).  A slot is 32 consecutive codes of a row in 24 bytes, code
 * 32 j + e (e < 32) of the slot in bits 6 e .. 6 e + 5 of its 192-bit
 * little-endian value.  Rows go in panels of 128, the last panel padded with
 * zero rows (P = ceil(rows / 128) * 128 rows in all); K goes in blocks of 128
 * codes (slots 0-3 of the block).  Panel p, block b is a 12288-byte tile at
 * ((p * K / 128) + b) * 12288; in it, slots h and h + 2 (h = 0, 1) of the
 * panel's row r are the 48 bytes at h * 6144 + r * 48.
 *
 *   codes       [rows][K/2] uint8 packed int4 (see conventions).
 *   out         P * K * 3 / 4 bytes.
 *   scales      [rows][K/G] of scale_dtype (HR_F16 or HR_F32), or NULL.
 *   out_scales  [K/G][P] of scale_dtype: scales transposed, zeros for the
 *               padding rows; NULL exactly when scales is.
 *   K           a multiple of 128; group G in {128, 256} dividing K (only read
 *               with scales); rows <= 128 * 65535.
 * All pointers 16-byte aligned.
 */
int32_t hr_w4a4_to_fp6(const uint8_t* codes, const void* scales, int32_t scale_dtype, int64_t rows, int64_t K,
                       int32_t group, uint8_t* out, void* out_scales, void* stream);

/*
 * hr_rotate_quant_fp6 -- hr_rotate_quant_int4 (m = 1) with its codes written
 * straight into the tiled fp6 format of hr_w4a4_to_fp6 and its scales
 * transposed, for activations headed to hr_w4a4_gemm_fp6.
 *
 * Defines: as hr_rotate_quant_int4 ("Experiment -- Hadamard rotation for int4
 * (W4A4) accuracy", Hypothesis and Method), the same codes and scales.
 *
 *   x        [rows][n] bf16 (x_dtype must be HR_BF16); n = 2048 or 4096.
 *   signs    [n] int8 +-1 or NULL.
 *   group    G in {128, 256}.
 *   tiles    P * n * 3 / 4 bytes, P = ceil(rows / 128) * 128, as
 *            hr_w4a4_to_fp6 writes them, except that the padding rows of the
 *            last panel are not written (hr_w4a4_gemm_fp6 stores no output
 *            from them, so their contents do not matter).
 *   scales   [n / G][P] of scale_dtype (HR_F16 or HR_F32), transposed; the
 *            padding rows' entries are not written either.
 * All pointers 16-byte aligned.
 */
int32_t hr_rotate_quant_fp6(const void* x, int32_t x_dtype, const int8_t* signs, int64_t rows, int32_t n,
                            int32_t group, int32_t scale_dtype, uint8_t* tiles, void* scales, void* stream);

/*
 * hr_w4a4_gemm_fp6 -- the W4A4 GEMM of hr_w4a4_gemm on operands in the tiled
 * fp6 format of hr_w4a4_to_fp6, on v_mfma_f32_32x32x64_f8f6f4.
 *
 * Defines: as hr_w4a4_gemm ("Experiment -- Hadamard rotation for int4 (W4A4)
 * accuracy", Hypothesis and Verdict).  The same sums and scale fusion: every
 * fp6 product of two codes is exact and so is the fp32 sum of a group, so
 * acc[m][n][g] is the exact integer group sum and C matches hr_w4a4_gemm.
 *
 *   a_f6, a_scales  activation codes of M rows and their transposed scales,
 *                   as hr_w4a4_to_fp6 or hr_rotate_quant_fp6 write them
 *                   (ceil(M / 128) panels; padding rows may hold anything).
 *   w_f6, w_scales  weight codes of N rows and scales, the same way.
 *   scale_dtype, c, group_acc: as hr_w4a4_gemm.
 *   M >= 0; N a multiple of 128; K a multiple of G, K <= 65536.
 *   group     G in {128, 256}.
 */
int32_t hr_w4a4_gemm_fp6(const uint8_t* a_f6, const void* a_scales, const uint8_t* w_f6, const void* w_scales,
                         int32_t scale_dtype, int64_t M, int64_t N, int64_t K, int32_t group, float* c,
                         int32_t* group_acc, void* stream);

/*
 * hr_rotate_quant_w4a4_gemm -- online rotation in the decode GEMM: the
 * activation rows are rotated and int4-quantized (hr_rotate_quant_int4 with
 * m = 1) and multiplied with the weights (hr_w4a4_gemm) in one kernel; the
 * activation codes never go to memory in between.
 *
 * Defines: as hr_rotate_quant_int4 followed by hr_w4a4_gemm; HARP technical
 * summary (gist.science), section 4 (the decode cost of an online rotation:
 * 0.0078 s against 0.0070 s per token) and section 2.4 (fused GPU kernels).
 *
 *   x         [M][K] bf16 activations (x_dtype must be HR_BF16).
 *   signs     [K] int8 +-1 or NULL (all +1).
 *   group     G in {32, 64, 128, 256}; the activations and the weights use it.
 *   w_codes   [N][K/2] uint8 packed int4; w_scales [N][K/G] of scale_dtype.
 *   M <= 16 (decode); K = 2048 or 4096; N a multiple of 64.
 *   c         [M][N] fp32:  C = sum_g sA sW acc_g on the activation codes.
 *   a_codes, a_scales  optional outputs ([M][K/2] uint8, [M][K/G] of
 *             scale_dtype): the activation codes and scales the GEMM used,
 *             as hr_rotate_quant_int4 would store them.  Both or neither.
 * Sizes outside these return HR_EUNSUPPORTED.
 */
int32_t hr_rotate_quant_w4a4_gemm(const void* x, int32_t x_dtype, const int8_t* signs, int32_t group,
                                  const uint8_t* w_codes, const void* w_scales, int32_t scale_dtype,
                                  int64_t M, int64_t N, int64_t K, float* c, uint8_t* a_codes,
                                  void* a_scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HR_H */
