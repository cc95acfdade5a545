/* libpingala: Pingala-8 trellis-coded 2-bit weights on AMD Instinct MI355X
 * (gfx950).  C ABI; every call returns an int status.
 *
 * What the method is (the pages describe it in words only):
 *   - "Pingala-8" landing page, section "How it works": an Ungerboeck 8-state
 *     trellis code encodes groups of 4 weights in order; a small state carried
 *     from one group to the next picks the value set the next group can use;
 *     before coding, a random Hadamard rotation spreads out the few very large
 *     weights; LDLQ rounding is used by the compressor.
 *   - same page, section "Where the name comes from": 8 states over short
 *     three-symbol patterns, trellis labels after Ungerboeck.
 *   - same page, section "Paper": the paper title calls it small-state coset
 *     trellis coding.
 *   - article "8 open models, 77-85% smaller: what 2-bit quantization costs
 *     and what it keeps", section "What 2-bit keeps": files keep per-block
 *     scales; one-user generation is mostly reading every weight once per
 *     token.
 *
 * Format P8F v1 (the pages give no bit layout; these are the plainest
 * choices they support):
 *   codes   u8 [n][k/4], row-major, one byte per group of 4 weights.
 *   scales  u16 [n][k/128], row-major, IEEE binary16 bits, one per block of
 *           128 weights (32 code bytes) of a row.  k % 128 == 0.
 *   state   s in 0..7 = the last three branch bits; s = 0 at every block
 *           start; after byte c: s = ((s << 1) | (c & 1)) & 7.
 *   decode  of byte c read in state s:
 *             z0 = (s >> 1) & 1                  value set A0 = {-7,-3,1,5},
 *                                                 A1 = {-5,-1,3,7}
 *             z1 = (c & 1) ^ (s & 1) ^ (s >> 2)   parity coset
 *             b_j = bit (1+j) of c for j < 3;  b_3 = z1 ^ b_0 ^ b_1 ^ b_2
 *             e_j = bit (4+j) of c
 *             level_j = 4 * (2 e_j + b_j) + 2 z0 - 7      (odd, -7..7)
 *             weight_j = scale * level_j   (rotated domain; exact in fp32)
 *   rotation per 128-block b of the input dimension:
 *             (R v)_i = 2^-3.5 * sum_j (-1)^popcount(i & j) sigma_j v_j
 *           sigma = the input site's random signs, sign_bits u8 [k/8], bit
 *           (k & 7) of byte (k >> 3), 1 meaning -1.  Rows of W are stored
 *           rotated (w~ = R w); activations are rotated at run time (x~ = R x)
 *           so that W~ x~ = W x.
 *   footprint: n*k/4 + 2*n*k/128 bytes = 2.125 bits per weight.
 *
 * Conventions.
 *   - Device pointers are device memory (e.g. torch tensors' data_ptr());
 *     host pointers are ordinary host memory.  All buffers are caller-owned;
 *     no call allocates, keeps or frees a caller buffer.
 *   - Device calls are asynchronous on the caller's hipStream_t (0 = the null
 *     stream) and validate all arguments on the host before any launch; on an
 *     invalid argument nothing is launched.  pg_encode_ref is synchronous.
 *   - codes, x, y, w and workspace pointers must be 16-byte aligned;
 *     scales and sign_bits at least 2-byte and 1-byte aligned (a call that
 *     needs more says so in its comment).
 *   - Errors: PG_OK = 0; negative codes below.  pg_last_error() returns a
 *     per-thread message for the last failing call of that thread.
 *   - Results of pg_decode are bit-exact; products accumulate in fp32.
 */
#ifndef PINGALA_H
#define PINGALA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pg_stream_t; /* a hipStream_t */

enum {
    PG_OK = 0,
    PG_ERR_INVALID_ARG = -1,  /* bad size, null or misaligned pointer, bad dtype */
    PG_ERR_UNSUPPORTED = -2,  /* valid request the library does not implement */
    PG_ERR_HIP = -3           /* a HIP runtime call or launch failed */
};

enum { PG_F32 = 0, PG_F16 = 1, PG_BF16 = 2,     /* element types of x / y */
       PG_Q16 = 3 };                               /* rotated activations, 16-bit fixed point */

enum { PG_FLAG_RMSNORM = 1u,                    /* pg_fwht_rotate / pg_rot_qgemv flags */
       PG_FLAG_CARRY_STATE = 2u,                 /* codes of the carried-state variant (below) */
       PG_FLAG_KERNEL_VDOT = 4u,                 /* kernel choice, for tests and tuning (below) */
       PG_FLAG_KERNEL_MMA = 8u,
       PG_FLAG_RATE23 = 16u };                   /* rate-2/3 trellis, through a codebook table (below) */

/* Kernel choice.  Each product has kernels that compute the same values
 * (within the stated tolerances): products on the v_dot4 vector
 * instructions and products on the int8 matrix cores.  Without a choice
 * flag the library picks by batch and shape; PG_FLAG_KERNEL_VDOT or
 * PG_FLAG_KERNEL_MMA (at most one) selects a kernel, so that tests can check
 * each against the oracle and a tuning sweep can time each.  Where the
 * selected kernel does not take the shape, the call falls back to the
 * library's own choice.  The library reads no environment variable. */

/* Carried-state variant of the format (the small-state coset-trellis design
 * space of the landing page, section "Paper"): the same bytes, scales and
 * per-group rule, but the trellis state runs on from one 128-block to the
 * next along a row instead of restarting at 0; a zero-scale block is 32
 * zero bytes.  Calls that take PG_FLAG_CARRY_STATE read (or write) codes of
 * this variant: pg_decode_ex, pg_encode_ex and pg_rot_qgemv. */

/* Rate-2/3 trellis (landing page, section "Where the name comes from": 8
 * states over short patterns, Ungerboeck-style labels): two branch bits per
 * group (byte bits 0, 1) and the state step s' = ((s << 2) | u) & 7, so the
 * state of a group is the previous byte's two branch bits (bits 0, 1) and
 * bit 0 of the byte before it (bit 2).  Its codebook is given as a table:
 * pg_codebook_table_ex(PG_FLAG_RATE23) writes the variant's own (the 512
 * points of P8F v1 in 8 cosets of 64: z0 = bit 0 of s picks the value set,
 * z1 = u0 ^ bit 1 of s the D4 parity, z2 = u1 ^ bit 2 of s the split
 * b0 ^ b1; bits 2, 3 are b0, b2, b1 = b0 ^ z2, b3 = b2 ^ z1 ^ z2, bits 4..7
 * are e0..e3).  pg_decode_table and pg_rot_qgemv_table take the flag. */

#define PG_FORMAT_VERSION 1
#define PG_LIB_VERSION 1

/* (format_version << 16) | lib_version. */
int pg_version(void);

/* Bytes of codes + scales for an n x k matrix: n*k/4 + n*(k/128)*2.
 * Returns 0 if n < 1 or k is not a positive multiple of 128. */
size_t pg_footprint_bytes(int64_t n, int64_t k);

/* PG_Q16: the library's own format for rotated activations, written by
 * pg_fwht_rotate and read by pg_qgemv.  Per row of k values (k % 128 == 0),
 * pg_q16_row_bytes(k) bytes:
 *   [0, 2k)          int8 digits; chunk c (values 16c..16c+15) holds 32 bytes:
 *                    byte 4j+g = hi digit of value 16c+4g+j, byte 16+4j+g = lo
 *                    digit, for group g = 0..3 and position j = 0..3;
 *   [2k, 2k+k/32)    f32 sx per 128-block;
 *   [2k+k/32, 2k+3k/32) int32 sum of the 16-bit values per 64-value half-block;
 *   then zero padding to a multiple of 64 bytes.
 * A value v of block b is q * sx[b], q = round(v / sx[b]) with |q| <= 32512,
 * sx[b] = max|v| / 32512 over the block (0 for an all-zero block), and
 * q = 256 * hi + lo with lo in [-128, 127].  Relative error <= 2^-16 of the
 * block's largest value. */
size_t pg_q16_row_bytes(int64_t k);

/* Message of the calling thread's last failed call ("" if none). */
const char* pg_last_error(void);

/* P8F v1's codebook written out as a table: out[s][c][j] = level_j of
 * byte c read in state s (int8 [8][256][4], host memory).  Given to
 * pg_decode_table / pg_rot_qgemv_table it reproduces P8F v1 (the other
 * entry points compute the same levels from the byte's bits). */
int pg_codebook_table(int8_t* out);

/* A format's codebook as a table, [8][256][4] int8, host memory: flags 0
 * is pg_codebook_table; PG_FLAG_RATE23 the rate-2/3 variant's (with
 * PG_FLAG_RATE23 on the table calls it reproduces that variant). */
int pg_codebook_table_ex(uint32_t flags, int8_t* out);

/* Host (CPU) reference encoder, synchronous.  Follows the "How it works"
 * description (rotation, then sequential trellis coding; the LDLQ Hessian is
 * the identity, i.e. plain minimum squared error):
 *   w          host fp32 [n][k], original (unrotated) weights
 *   sign_bits  host u8 [k/8], the input site's random signs
 *   codes      host u8 [n][k/4] out
 *   scales     host u16 [n][k/128] out (fp16 bits)
 *   n_threads  worker threads (<= 0: the hardware concurrency, at most 16)
 * Per row: rotate each 128-block in fp64; scale = fp16_RNE(min(0.29 * rms,
 * 65504)) with the squares summed in index order (0 if the block is zero);
 * Viterbi over the 32 groups from state 0 with a free end state, the branch
 * metric being the nearest of the 128 points of the branch's coset
 * (distortion ((d0^2 + d1^2) + d2^2) + d3^2); ties go to the predecessor
 * s'>>1, then the smaller byte, then the smaller end state; a zero scale
 * codes every group as byte 0. */
int pg_encode_ref(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits,
                  uint8_t* codes, uint16_t* scales, int n_threads);

/* The same encoder on the GPU, asynchronous on `stream`: codes and scales
 * are bit-identical to pg_encode_ref's for the same input (every step runs in
 * fp64 in the same operation order, without fused multiply-add).  One
 * workgroup per 128-block: rotation, scale rule, the nearest point of each
 * coset per group, then the 8-state add-compare-select and traceback.
 *   w          device fp32 [n][k], original (unrotated) weights
 *   sign_bits  device u8 [k/8]
 *   codes      device u8 [n][k/4] out (16-byte aligned)
 *   scales     device u16 [n][k/128] out (fp16 bits)
 * Buffers are the caller's; nothing is allocated.  n * k / 128 < 2^31. */
int pg_encode(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint8_t* codes,
              uint16_t* scales, pg_stream_t stream);

/* LDLQ encoding with a proxy Hessian (landing page, "How it works": the
 * compressor rounds with LDLQ, passing each coded unit's error through the
 * Hessian on to the units not yet coded).  The unit is the 128-block:
 *   H~ = R H R^T (the site's block rotation on both sides) = U D U^T, U unit
 *   upper block-triangular, D block-diagonal (blocks of 128), factored on
 *   the host in fp64;
 *   block b of each row is coded (scale rule and Viterbi as pg_encode_ref)
 *   against t = v + sum_{c < 128 b} e_c * (U - I)[c][128 b + i], summed in
 *   increasing c with one rounding per product and per sum, where v are the
 *   block's rotated weights and e = W~ - What of the blocks already coded.
 * H = I (or any H without terms across blocks after rotation) gives
 * pg_encode_ref's codes.
 *   hessian  host fp64 [k][k], symmetric positive definite, in the original
 *            (unrotated) input basis, e.g. the mean of x x^T over calibration
 *            inputs; PG_ERR_INVALID_ARG if not finite, not symmetric (to
 *            1e-12 of its largest entry) or not positive definite
 * k <= 16384 (PG_ERR_UNSUPPORTED beyond): the feedback matrix is held as
 * k x k fp64.  Other arguments as pg_encode_ref.  Synchronous. */
int pg_encode_ref_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* hessian,
                       uint8_t* codes, uint16_t* scales, int n_threads);

/* The LDLQ encoder on the GPU: codes and scales bit-identical to
 * pg_encode_ref_ldlq's.  The factorisation runs on the host (shared with
 * pg_encode_ref_ldlq); the library then allocates k x k + n x k fp64 device
 * buffers for the feedback matrix and the coded blocks' errors, launches one
 * kernel per 128-block on `stream` (one workgroup per row: rotation, the
 * feedback sum in the stated order, the block encoder of pg_encode, the
 * block's errors), and frees them before returning.  Synchronous.
 *   w, sign_bits, codes, scales: device, as pg_encode
 *   hessian  host fp64 [k][k], as pg_encode_ref_ldlq */
int pg_encode_ldlq(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const double* hessian,
                   uint8_t* codes, uint16_t* scales, pg_stream_t stream);

/* Encoders through a codebook table (the table-driven variant, landing
 * page section "Paper"; codes are then read back with pg_decode_table /
 * pg_rot_qgemv_table and the same table and flags).  Rotation and scale rule
 * as pg_encode_ref; per 128-block a Viterbi search over the table: for every
 * group, state p and byte c the distortion ((d0^2 + d1^2) + d2^2) + d3^2,
 * d_j = w_j - s * table[p][c][j] (fp64, no fused multiply-add); per state
 * and branch the first byte of least distortion (the branch is byte bit 0,
 * or bits 0..1 with PG_FLAG_RATE23); add-compare-select from state 0, each
 * next state's predecessors in increasing order with strict improvement,
 * the first best end state; a zero scale codes every group as byte 0.  On
 * P8F v1's own table the codes are pg_encode_ref's.
 *   table  int8 [8][256][4]: host memory for pg_encode_ref_table, device
 *          memory (16-byte aligned) for pg_encode_table
 *   flags  0 or PG_FLAG_RATE23
 * pg_encode_table is the same search on the GPU, bit-identical, one
 * workgroup per 128-block, asynchronous on `stream`.  Other arguments as
 * pg_encode_ref / pg_encode. */
int pg_encode_ref_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                        uint32_t flags, uint8_t* codes, uint16_t* scales, int n_threads);
int pg_encode_table(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, const int8_t* table,
                    uint32_t flags, uint8_t* codes, uint16_t* scales, pg_stream_t stream);

/* pg_encode with format flags: 0 is pg_encode (format P8F v1);
 * PG_FLAG_CARRY_STATE codes the carried-state variant with one Viterbi
 * search per row over all of its blocks (state carried on, per-block scales
 * and branch metrics, free end state, the same tie-breaks; in a zero-scale
 * block the only branch is byte 0).  One workgroup per row; k <= 16384 for
 * the variant (PG_ERR_UNSUPPORTED beyond).  Other arguments as pg_encode. */
int pg_encode_ex(const float* w, int64_t n, int64_t k, const uint8_t* sign_bits, uint32_t flags,
                 uint8_t* codes, uint16_t* scales, pg_stream_t stream);

/* Decode to rotated-domain fp32 weights (bit-exact: scale * level in fp32).
 *   codes device u8 [n][k/4], scales device u16 [n][k/128],
 *   w_rot device f32 [n][k] out. */
int pg_decode(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
              float* w_rot, pg_stream_t stream);

/* pg_decode with format flags: 0 is pg_decode; PG_FLAG_CARRY_STATE decodes
 * codes of the carried-state variant.  Bit-exact. */
int pg_decode_ex(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, uint32_t flags,
                 float* w_rot, pg_stream_t stream);

/* Table-driven codebook variant (landing page, section "Paper": the format
 * is a small-state coset trellis; the trellis and the codebook separate).
 * The trellis is P8F v1's (branch bit u = bit 0 of the byte, state = the
 * last three branch bits, 0 at each 128-block start, or run on along the
 * row with PG_FLAG_CARRY_STATE); the codebook is a caller-supplied table:
 *   table    device int8 [8][256][4], 16-byte aligned: table[s][c][j] is
 *            level j (units of the block scale) of the group read in state s
 *            as byte c.  Any int8 values: a non-uniform or learned value set,
 *            or P8F v1's own (pg_codebook_table).  Read only; the caller owns
 *            it and may change it between calls.
 * Decode to rotated-domain fp32 weights, w = fp32(scale) * level (exact).
 * flags: PG_FLAG_CARRY_STATE (state run on along the row), PG_FLAG_RATE23
 * (the states of the rate-2/3 trellis instead of P8F v1's).  Other
 * arguments as pg_decode. */
int pg_decode_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const int8_t* table,
                    uint32_t flags, float* w_rot, pg_stream_t stream);

/* Run-time activation rotation ("How it works": the random Hadamard
 * rotation; the activations take the same rotation as the weight rows):
 *   x        device [rows][k] of in_dtype (PG_F32 / PG_F16 / PG_BF16)
 *   y        device [rows][k] of out_dtype (PG_F32 / PG_F16 / PG_BF16), or
 *            rows * pg_q16_row_bytes(k) bytes for PG_Q16
 *   sign_bits device u8 [k/8]
 *   flags    PG_FLAG_RMSNORM: first replace each row v by n(v), the
 *            normalisation between the layers of a linear stack:
 *              S = sum of v^2 over the row (fp32, order unspecified),
 *              inv = rsq(fma(S, rk, 1e-6)), rk = 1/k rounded to fp32,
 *              rsq the hardware reciprocal square root (<= 1 ulp),
 *              n(v) = fp16_RNE(v * inv)   (every kernel computes this;
 *              some round the product to fp32 first, some convert the
 *              exact product as one mixed-precision fma: the two differ
 *              by one fp16 unit in rare ties)
 * x and y may not overlap.  fp32 arithmetic; fp16/bf16 outputs round to
 * nearest even. */
int pg_fwht_rotate(const void* x, int in_dtype, void* y, int out_dtype,
                   const uint8_t* sign_bits, int64_t rows, int64_t k, uint32_t flags,
                   pg_stream_t stream);

/* pg_fwht_rotate over rows of x that are ldx >= k elements apart (the first
 * k columns of each row are rotated, as when a stage reads part of the
 * previous stage's output); y as in pg_fwht_rotate.  pg_fwht_rotate is this
 * call with ldx = k. */
int pg_fwht_rotate_ex(const void* x, int in_dtype, int64_t ldx, void* y, int out_dtype,
                      const uint8_t* sign_bits, int64_t rows, int64_t k, uint32_t flags,
                      pg_stream_t stream);

/* Batch-1..8 product over the compressed weights (the generation path,
 * article "8 open models...", section "What 2-bit keeps": one pass over all
 * weights per token):
 *   y[b][i] = sum_blk scale[i][blk] * sum_{k in blk} level[i][k] * x_rot[b][k]
 *   codes device u8 [n][k/4], scales device u16 [n][k/128]
 *   x_rot device [batch][k] PG_F32 or PG_F16, or batch * pg_q16_row_bytes(k)
 *         bytes of PG_Q16 (the fast path: exact integer dot products of the
 *         levels with the 16-bit activations, one fp32 scale per half-block),
 *         already rotated
 *   batch 1..8, y device f32 [batch][n] out.
 * fp32 accumulation; summation order is fixed, so repeated calls are
 * bitwise identical.  With PG_Q16 and batch >= 2 the products run on the
 * int8 matrix cores (the level planes of a code dword serve up to 16 batch
 * rows at once); the results agree with the batch-1 kernel's within fp32
 * rounding, not bit for bit. */
int pg_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
             const void* x_rot, int x_dtype, int batch, float* y, pg_stream_t stream);

/* pg_qgemv with kernel-choice flags (PG_Q16 input only; 0 is pg_qgemv):
 * PG_FLAG_KERNEL_VDOT keeps the v_dot4 kernel at every batch,
 * PG_FLAG_KERNEL_MMA takes the matrix cores at every batch. */
int pg_qgemv_ex(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                const void* x_rot, int x_dtype, int batch, uint32_t flags, float* y, pg_stream_t stream);

/* One stage of a linear stack in a single launch: the RMS normalisation and
 * the run-time rotation of the activations (landing page, section "How it
 * works": a random Hadamard rotation is applied before coding, so the
 * activations take the same rotation) are the product's prologue:
 *   y[b] = W~ . R . n(x[b][0:k])
 * with n(v) the normalisation of pg_fwht_rotate under PG_FLAG_RMSNORM
 * (fp16_RNE(v * rsq(fma(S, 1/k, 1e-6))), S the row's sum of squares;
 * within rounding of fp16_RNE(v / sqrt(mean(v^2) + 1e-6))), n(v) = v
 * otherwise, R the input
 * site's rotation (as pg_fwht_rotate), and the rotated activations carried
 * at 16-bit precision (error <= 2^-16 of the largest value of each 32
 * consecutive rotated values).
 *   codes, scales  as for pg_qgemv (scales 4-byte aligned)
 *   x        device [batch][ldx] of x_dtype (PG_F32 / PG_F16); the first k
 *            values of each row are the input (e.g. the q part of a merged
 *            q/k/v output); ldx >= k; x and every row start 16-byte
 *            aligned (ldx a multiple of 4 for PG_F32, of 8 for PG_F16);
 *            ldx < 2^31 (PG_ERR_UNSUPPORTED beyond)
 *   sign_bits device u8 [k/8], 4-byte aligned
 *   y        device f32 [batch][n] out
 *   batch    1..8
 * k <= 16384 (PG_ERR_UNSUPPORTED beyond).  PG_F32 input needs
 * PG_FLAG_RMSNORM (the rotation runs on fp16 values, exact after the
 * normalisation's fp16 rounding or for fp16 input; PG_ERR_UNSUPPORTED
 * otherwise).  The rotated values are quantised to 16-bit digits with one
 * scale per 32 values at batch 1 and per 128-block at batch 2..8 (there the
 * product runs on the matrix cores, for k <= 4096; larger k stays on the
 * batch-1 kernels).  PG_FLAG_CARRY_STATE: the codes are of the carried-state
 * variant (v_dot4 kernel at every batch).  PG_FLAG_KERNEL_VDOT: the v_dot4
 * products with the rotation on the matrix cores at every batch;
 * PG_FLAG_KERNEL_MMA: the int8 matrix-core products at every batch where
 * k <= 4096.  x and y may not overlap.  The
 * summation order is fixed: repeated calls are bitwise identical. */
int pg_rot_qgemv(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                 const void* x, int x_dtype, int64_t ldx, const uint8_t* sign_bits,
                 uint32_t flags, int batch, float* y, pg_stream_t stream);

/* The fused stage of pg_rot_qgemv at batch 1 through a codebook table (as
 * pg_decode_table): y = W~ . R . n(x) with W~'s levels read from table.
 *   codes, scales, sign_bits, x (first k values), y, x_dtype: as pg_rot_qgemv
 *   at batch 1; table as pg_decode_table
 *   flags    PG_FLAG_RMSNORM, PG_FLAG_CARRY_STATE (state run on along rows),
 *            PG_FLAG_RATE23 (the rate-2/3 trellis's states)
 * The rotated activations are quantised to 16-bit digits per 32 values as
 * pg_rot_qgemv at batch 1; each 32-value partial sum of level * digit is
 * exact in int32 and rounded once to fp32.  With P8F v1's table the output
 * is bitwise that of pg_rot_qgemv at batch 1 (k <= 4096, where that takes
 * the same stage).  k <= 16384 (PG_ERR_UNSUPPORTED beyond); PG_F32 input
 * needs PG_FLAG_RMSNORM.  x and y may not overlap.  Fixed summation order. */
int pg_rot_qgemv_table(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k, const void* x,
                       int x_dtype, const uint8_t* sign_bits, const int8_t* table, uint32_t flags, float* y,
                       pg_stream_t stream);

/* Prompt-processing product for m activation rows (landing page, section
 * "Results": prompt reading is the mat-mat path):
 *   Y[r][i] = sum_blk scale[i][blk] * sum_{k in blk} level[i][k] * X[r][k]
 *   x_rot_bf16 device u16 [m][k] (bf16 bits, already rotated), y device f32
 *   [m][n] out.  Levels enter the matrix cores as exact bf16 values and
 *   the block scales are applied in fp32 by carrying the running sum from
 *   block to block (acc = acc * s_prev / s_new at each block start, times
 *   the last scale at the end: one rounding per later block, within
 *   nbk * 2^-24 relative of per-block partial sums).  For a given shape,
 *   device and workspace size the result is the same on every call. */
int pg_qgemm(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
             const uint16_t* x_rot_bf16, int64_t m, float* y, pg_stream_t stream);

/* pg_qgemm with a caller-owned device workspace, which lets the product
 * split K when the output tiles alone would leave compute units idle
 * (small m, few weight rows against a long k, or a last round of tiles that
 * fills only part of the chip): the tiles of the split (all of them, or
 * those of the last round) are each summed over ranges of whole 128-blocks,
 * split 0 into y and the others into the workspace, and a second launch adds
 * the parts to y in split order.
 *   workspace        device, 16-byte aligned, or NULL (then workspace_bytes
 *                    must be 0 and the call is pg_qgemm); it may not overlap
 *                    codes, scales, x_rot_bf16 or y.  Its contents on entry
 *                    do not matter; on return they are unspecified.
 *   workspace_bytes  its size; pg_qgemm_workspace_bytes(n, k, m) bytes allow
 *                    the split the library picks for the shape, fewer bytes
 *                    a smaller split or none (each further part takes 128 KiB
 *                    per split tile of 256 x 128 outputs).
 * Results may differ from pg_qgemm's in the last bits (another summation
 * order), but for a given shape, workspace size and device the order is
 * fixed: repeated calls are bitwise identical. */
int pg_qgemm_ex(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                const uint16_t* x_rot_bf16, int64_t m, float* y, void* workspace,
                size_t workspace_bytes, pg_stream_t stream);

/* pg_qgemm_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the split workspace is the library's own scratch, a device
 * array of 32 MiB that each GPU the library runs on holds until the
 * process ends.  Same arguments as pg_qgemm; same result as pg_qgemm_ex with
 * a workspace of pg_qgemm_workspace_bytes(n, k, m) bytes (bitwise).
 * PG_ERR_UNSUPPORTED (nothing launched) when the shape needs more than the
 * scratch holds.  Calls no allocating routine.  Every call on a GPU shares
 * that GPU's scratch: calls that may overlap on one GPU (other streams,
 * other host threads) race and must be serialised by the caller. */
int pg_qgemm_noalloc(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                     const uint16_t* x_rot_bf16, int64_t m, float* y, pg_stream_t stream);

/* pg_qgemm_ex with its kernel and split plan given, for tests and tuning:
 *   kernel  0: the library's choice (what pg_qgemm and pg_qgemm_ex run),
 *              at present kernel 8;
 *           1: the one-buffer 128 x 128-tile kernel (never splits);
 *           2: the pipelined tile with separate producer waves (copies and
 *              decode) and consumer waves (matrix cores);
 *           3: as 2 in 1024 threads, the block scales carried in the
 *              running sums (no per-block partial sums: each later block
 *              rescales the sum by a ratio of scales, one fp32 rounding
 *              each, within nbk * 2^-24 relative of kernel 4's sums);
 *           4: the pipelined 256 x 128-tile kernel, per-block partial sums
 *              scaled in fp32 (levels enter the matrix cores exactly);
 *           5: 256 x 256 tiles over the whole of K, the block scales
 *              carried as in kernel 3 (results equal to kernel 3's); never
 *              splits, so splits, first_split and the workspace are unused;
 *           6: as 5 with each wave decoding its weight rows straight into
 *              the matrix cores' operands (only X passes through the LDS);
 *              the products take K in another order within each 64-wide
 *              step, so results differ from kernel 5's in the last bits;
 *           7: as 6 with 256 x 32 wave tiles (each weight row decoded by
 *              one wave; results equal to kernel 6's);
 *           8: 256 x 128 tiles of four waves with 256 x 32 wave tiles and
 *              register-decoded operands, two workgroups per compute unit,
 *              the split plans of kernel 4
 *   splits  0: the library's plan; S >= 1: tiles first_split .. split S ways
 *           (tiles before it whole), S capped by the 128-blocks of k, by 8
 *           and by the workspace
 * Other arguments as pg_qgemm_ex. */
int pg_qgemm_tune(const uint8_t* codes, const uint16_t* scales, int64_t n, int64_t k,
                  const uint16_t* x_rot_bf16, int64_t m, float* y, void* workspace, size_t workspace_bytes,
                  int kernel, int splits, int64_t first_split, pg_stream_t stream);

/* Workspace bytes that give pg_qgemm_ex its full split of K for this shape on
 * the current device (0: it would not split; 0 as well for invalid sizes). */
size_t pg_qgemm_workspace_bytes(int64_t n, int64_t k, int64_t m);

/* Measurement helper, not part of the method: the HBM bandwidth a plain
 * streaming kernel reaches on this device, as the practical ceiling next to
 * the vendor peak (the batch-1 product is meant to stream its compressed
 * bytes at HBM speed: article "8 open models...", section "What 2-bit
 * keeps", one pass over all weights per token).
 *   p        device, 16-byte aligned, `bytes` readable bytes
 *   bytes    a positive multiple of 16
 *   xor_out  device u32, 4-byte aligned, not inside [p, p + bytes): the XOR of
 *            all 32-bit words of the range is XOR-ed into *xor_out (so a
 *            caller that zeroes it first gets exactly that XOR; the value
 *            checks that every byte was read).
 * Asynchronous on `stream`. */
int pg_hbm_read(const void* p, size_t bytes, uint32_t* xor_out, pg_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PINGALA_H */
