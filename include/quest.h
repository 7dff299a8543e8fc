/*
 * libquest - the QuEST quantiser hot path on AMD Instinct MI355X (gfx950).
 *
 * QuEST (arXiv 2502.05003) quantises weights and activations for
 * quantisation-aware training.  Forward: each row is cut into blocks of n
 * entries, every block is multiplied by the orthonormal Hadamard matrix, the
 * row is RMS-normalised and projected onto a b-bit symmetric uniform grid
 * whose clip scale alpha_b * RMS minimises the expected squared error for a
 * standard Gaussian; entries whose quantisation error is at most half a grid
 * step are marked as trusted.  Backward: the Hadamard-domain gradient is
 * multiplied by that trust mask and transformed back.
 * Sources: the QuEST abstract (codewithpapers.app record of arXiv
 * 2502.05003: Hadamard normalisation, MSE-optimal fitting, trust gradient
 * estimator); atlas.scime.ai summary of QuEST, "Approach"; pith.science
 * review of QuEST, "What carries the argument", "Assumptions & free
 * parameters" and the Figure 2 caption.
 *
 * Conventions shared by every call
 *   - Tensors are row-major and contiguous: element (r, c) of a rows x cols
 *     tensor is at index r * cols + c.
 *   - Every buffer is allocated, owned and freed by the caller.  Device
 *     buffers are HIP device memory on the current device; the library never
 *     allocates, frees or synchronises.
 *   - Device calls enqueue their kernels on `stream` (a hipStream_t; NULL is
 *     the null stream) and return without waiting.  A status other than
 *     QUEST_EHIP means nothing was enqueued.  They enqueue nothing but
 *     kernels (no copy, fill or wait), so a sequence of calls on a stream
 *     under HIP graph capture records into the graph and replays as called.
 *   - Arguments are checked before anything is launched.  On any error the
 *     call writes nothing and returns a status code; no C++ exception crosses
 *     this interface.
 *   - rows == 0 is a valid empty call: it returns QUEST_OK, touches no
 *     buffer and may be given NULL pointers.
 *   - Calls are thread-safe.  The only global state is the table of clip
 *     scales alpha_b, filled once on first use.
 *   - Inputs must be finite, and every row's RMS must lie in [2^-60, 2^50]
 *     (about 8.7e-19 to 1.1e15) or the row must be exactly zero: the sum of
 *     squares is accumulated in fp32 and must neither overflow nor underflow.
 *
 * Data layouts
 *   codes : per row, an LSB-first stream of b-bit unsigned codes: element c
 *           occupies bits [c*b, (c+1)*b) of the row's cols*b/8 bytes, and
 *           bit i of byte j is stream bit 8j+i (at b=4 element 2i is the low
 *           nibble of byte i).  Codes are offset binary u in [0, 2^b - 1];
 *           the grid value of code u is (2u - L + 1) * s / (L - 1), L = 2^b.
 *           XOR with 2^(b-1) gives the two's-complement form.
 *   mask  : per row, an LSB-first stream of cols bits; 1 = trusted (the
 *           gradient passes), 0 = masked.
 *   scale : one fp32 per row, the clip scale s_r = alpha_b * RMS_r (the
 *           outermost grid level), not the RMS and not the step.
 */
#ifndef QUEST_H
#define QUEST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QUEST_OK = 0,
  QUEST_EINVAL = 1,       /* bad pointer, size, dtype or forbidden aliasing */
  QUEST_EUNSUPPORTED = 2, /* block, bit width or row width outside what is built */
  QUEST_EALIGN = 3,       /* a buffer is not 16-byte aligned */
  QUEST_EHIP = 4,         /* the HIP runtime reported an error at launch */
  QUEST_STATUS_INT_RANGE_ = 0x7FFFFFFF /* not a status: gives the type int's range of values */
} quest_status;

/* Element types.  The last enumerator is not a type: it gives quest_dtype the
   whole range of int, so that any value a caller passes can be received and
   rejected with QUEST_EINVAL (in C++ a value outside an enumeration's range
   could not even be loaded). */
typedef enum { QUEST_F32 = 0, QUEST_BF16 = 1, QUEST_DTYPE_INT_RANGE_ = 0x7FFFFFFF } quest_dtype;

/* Largest row width handled in one pass (a row is reduced by one workgroup). */
#define QUEST_MAX_COLS 32768

/*
 * Clip scale alpha_b of the b-bit grid: the alpha minimising
 * E[(Q_{alpha,b}(X) - X)^2] for X ~ N(0, 1), where Q_{alpha,b} rounds to the
 * nearest of the L = 2^b levels (2k - L + 1) alpha / (L - 1), k = 0..L-1.
 * pith.science review of QuEST, "What carries the argument" (the grid scale
 * minimises the L2 error against a standard Gaussian) and "Assumptions &
 * free parameters" (alpha* is derived from a fixed N(0,1) target).
 * Host only, float64; computed once per b and cached.  b in [1, 8];
 * returns NaN for any other b.  alpha_1 = sqrt(2/pi).
 */
double quest_fit_alpha(int b);

/*
 * Forward QuEST quantisation of x (rows x cols):
 *   y     = blockwise Hadamard transform of each row, blocks of `block`
 *           entries, orthonormal Sylvester matrix (natural order);
 *   s_r   = alpha_b * sqrt(mean_c y[r,c]^2),  Delta_r = 2 s_r / (2^b - 1);
 *   u     = clamp(floor(y / Delta_r) + 2^(b-1), 0, 2^b - 1);
 *   mask  = [ |grid(u) - y| <= Delta_r / 2 ]  (equivalently |y| <= s_r L/(L-1)).
 * A row of zeros gives s_r = 0, u = 2^(b-1) everywhere and an all-ones mask.
 * atlas.scime.ai summary of QuEST, "Approach"; pith.science review of
 * QuEST, "What carries the argument" and the Figure 7 caption (mask M_alpha*).
 *
 *   x       device, rows*cols elements of x_dtype (QUEST_F32 or QUEST_BF16)
 *   rows    >= 0
 *   cols    > 0, a multiple of `block`, at most QUEST_MAX_COLS
 *   block   Hadamard block size: 64, 128 or 256
 *   b       bits per code: 1 .. 8
 *   codes   device output, quest_codes_bytes(rows, cols, b) bytes
 *   scale   device output, rows floats (s_r)
 *   mask    device output, quest_mask_bytes(rows, cols) bytes
 * Pointers must be 16-byte aligned.  No output may overlap x or another
 * output (QUEST_EINVAL).  rows * cols must stay below 2^36
 * (QUEST_EUNSUPPORTED).  The transform and the reduction run in fp32; an
 * entry within about 1e-6 * s_r of a decision or trust threshold may round
 * to the neighbouring outcome of the exact (fp64) definition.
 * bf16 rows of 512, 1024 or 2048 columns take the 32-point transforms on the
 * matrix cores; setting the environment variable QUEST_FWD_KERNEL=valu
 * before the first call keeps them on the vector ALUs (timing comparisons).
 */
quest_status quest_quantize_fwd(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                int b, uint8_t* codes, float* scale, uint8_t* mask, void* stream);

/*
 * The forward of quest_quantize_fwd on several tensors in one call: the
 * outputs are those of calling quest_quantize_fwd on each tensor in turn
 * (same block, bit width and input dtype), bit for bit.  A quantisation-aware
 * training step quantises every weight of a model (pith.science review of
 * QuEST, "What carries the argument": the quantiser is applied to weights and
 * activations in every forward pass); with b <= 4 the library launches the
 * bf16 tensors whose rows have 512, 1024 or 2048 entries together (one
 * launch per width for up to eight tensors) and adds those whose rows have
 * 2560 to 8192 entries (a multiple of 512; up to four per launch) to the
 * first of these launches, and launches the others one by one.
 *
 *   tensors  host array of `count` descriptors, read during the call only;
 *            each names x, rows, cols, codes, scale and mask as the
 *            arguments of quest_quantize_fwd (a tensor with rows == 0 is
 *            skipped and its pointers are not read)
 *   count    >= 0 (0: nothing is done)
 *   x_dtype, block, b, stream: as for quest_quantize_fwd, for every tensor
 * Errors: everything quest_quantize_fwd rejects for any tensor, with the
 * same status; count < 0 or tensors NULL with count > 0 is QUEST_EINVAL; an
 * output of one tensor overlapping an input or output of another is
 * QUEST_EINVAL (inputs may overlap each other).  Validation covers every
 * tensor before the first launch, so on error nothing is written.
 */
typedef struct {
  const void* x;
  int64_t rows;
  int64_t cols;
  uint8_t* codes;
  float* scale;
  uint8_t* mask;
} quest_fwd_tensor;

quest_status quest_quantize_fwd_group(const quest_fwd_tensor* tensors, int count, quest_dtype x_dtype, int block,
                                      int b, void* stream);

/*
 * Forward quantisation that also writes the dequantised ("fake-quantised")
 * tensor, in one pass over x: everything quest_quantize_fwd computes, plus
 *   dq[r, c] = (2 u[r, c] - L + 1) * s_r / (L - 1)   (Hadamard domain),
 * the grid value of each entry's code, rounded to dq_dtype (bf16: round to
 * nearest even).  The values are those quest_dequantize returns for the
 * same codes and scale, bit for bit.  This is the tensor a quantisation-
 * aware training step multiplies with: both operands of a product are
 * transformed and quantised, and their product in the Hadamard domain equals
 * the product of the originals' reconstructions (pith.science review of
 * QuEST, "Assumptions & free parameters"; "What carries the argument").
 *
 *   x, x_dtype, rows, cols, block, b, scale, mask, stream: as for
 *           quest_quantize_fwd
 *   codes   device output as for quest_quantize_fwd, or NULL: codes are then
 *           not written (a training step that keeps only dq, scale and mask)
 *   dq      device output, rows*cols elements of dq_dtype (QUEST_BF16 or
 *           QUEST_F32), 16-byte aligned, overlapping no other argument
 * Errors as for quest_quantize_fwd; a NULL dq with rows > 0 or an unknown
 * dq_dtype is QUEST_EINVAL.
 */
quest_status quest_quantize_fwd_dq(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                   int b, uint8_t* codes, float* scale, uint8_t* mask, void* dq,
                                   quest_dtype dq_dtype, void* stream);

/*
 * The general forward: quest_quantize_fwd_dq with an outer trust factor t.
 * The trust mask keeps every entry inside the grid's range and, beyond the
 * outermost levels, those within t half-steps of them:
 *   mask = [ |q - y| <= Delta_r / 2 ]       for |y| <= s_r,
 *          [ |q - y| <= t * Delta_r / 2 ]   for |y| >  s_r,
 * i.e. trusted iff |y| <= s_r (1 + t / (L - 1)).  t = 1 is the plain rule of
 * quest_quantize_fwd; the 1-bit runs of the pages use t = 1.30 (pith.science
 * review of QuEST, "Assumptions & free parameters": the outer trust scaling
 * factor s*; atlas.scime.ai summary, "Limitations").
 *
 *   trust   t, finite and >= 0 (QUEST_EINVAL otherwise)
 *   codes   device output or NULL (not written)
 *   dq      device output of dq_dtype or NULL (not written); dq_dtype is
 *           checked only when dq is given
 * Everything else as for quest_quantize_fwd_dq.
 */
quest_status quest_quantize_fwd_ex(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                   int b, double trust, uint8_t* codes, float* scale, uint8_t* mask, void* dq,
                                   quest_dtype dq_dtype, void* stream);

/*
 * Dequantise codes to their grid values, in the Hadamard domain:
 *   out[r, c] = (2 u[r, c] - L + 1) * s_r / (L - 1),  L = 2^b,
 * rounded to out_dtype (bf16: round to nearest even).  The Hadamard domain
 * is where the quantised operands of a product live, since the orthogonal
 * transform is applied to both operands (pith.science review of QuEST,
 * "Assumptions & free parameters"); the official repository names the same
 * step `dequantize_dense` (codewithpapers.app record).
 *   codes   device, quest_codes_bytes(rows, cols, b) bytes (layout above)
 *   scale   device, rows floats
 *   rows    >= 0;  cols > 0, a multiple of 64, at most QUEST_MAX_COLS
 *   b       1 .. 8
 *   out     device output, rows*cols elements of out_dtype; must not
 *           overlap codes or scale (QUEST_EINVAL)
 */
quest_status quest_dequantize(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, int b,
                              void* out, quest_dtype out_dtype, void* stream);

/*
 * Trust-gradient backward:  grad_out[r, block k] = H_n (M * G)[r, block k],
 * H_n the orthonormal Hadamard matrix (its own inverse), M the stored mask.
 * The scale is treated as a constant (no gradient through the RMS).
 * pith.science review of QuEST, "What carries the argument" (the gradient in
 * the Hadamard domain is multiplied by the binary mask) and the Figure 2
 * caption (inverse Hadamard transforms on the backward pass).
 *   grad     device, rows*cols elements of g_dtype: the gradient with respect
 *            to the Hadamard-domain (quantised) tensor
 *   mask     device, quest_mask_bytes(rows, cols) bytes from quest_quantize_fwd
 *   rows     >= 0;  cols > 0, a multiple of `block`, at most QUEST_MAX_COLS
 *   block    64, 128 or 256 (the block used in the forward pass)
 *   grad_out device output, rows*cols elements of g_dtype (bf16 rounded to
 *            nearest even).  grad_out == grad runs in place; any other
 *            overlap with grad, or any overlap with mask, is QUEST_EINVAL.
 */
quest_status quest_trust_bwd(const void* grad, quest_dtype g_dtype, const uint8_t* mask, int64_t rows, int64_t cols,
                             int block, void* grad_out, void* stream);

/*
 * The matrix-core operand of a quantised tensor, for products of two of them
 * (quest_gemm).  The pages time QuEST's 4-bit matrix products against BF16
 * ones, quantisation, dequantisation and Hadamard costs included
 * (pith.science review of QuEST, Figure 5 caption; atlas.scime.ai summary,
 * "Key results").  Every level of the midrise grid is a half-integer
 * multiple of the row's step Delta_r = 2 s_r / (L - 1):
 *   q = (u - (L - 1)/2) * Delta_r,
 * and for b <= 4 the half-integer h = u - (L - 1)/2 (|h| <= 7.5) is held
 * exactly by the FP6 E2M3 element type of the OCP Microscaling Formats
 * specification v1.0 (sign bit 5, exponent bits 4..3 with bias 1, mantissa
 * bits 2..0; subnormals at exponent 0), the operand type of gfx950's
 * 6-bit matrix instructions.
 *
 * Operand layout (tiled for the matrix cores; cols a multiple of 128):
 *   rows form blocks of 32 (the last block padded), each row block is
 *   cols / 128 consecutive 3072-byte blocks of 128 columns, and a block is
 *   two 1536-byte halves of 64 columns, each 64 slots of 24 bytes.  Slot l
 *   of half e of block c of row block R holds row 32 R + l % 32, columns
 *   128 c + 64 e + 32 (l / 32) + (0 .. 31) as 6-bit fields, LSB-first
 *   (field i in bits [6 i, 6 i + 6) of the slot, bit j of byte t is bit
 *   8 t + j).  Run j (columns 32 j .. 32 j + 31) of row r therefore starts at
 *     (r / 32) * (cols / 128) * 3072 + (j / 4) * 3072 + (j / 2 % 2) * 1536
 *       + (32 (j % 2) + r % 32) * 24.
 *   The padding rows of the last row block may be written by
 *   quest_quantize_fwd_op (their contents are unspecified) and are left alone
 *   by quest_codes_to_operand; a product only uses them for outputs it does
 *   not store.
 */

/* Bytes of the operand: ceil(rows / 32) * 32 * cols * 3 / 4 (0 unless cols is a
   positive multiple of 128 and rows >= 0). */
size_t quest_operand_bytes(int64_t rows, int64_t cols);

/*
 * The operand of stored codes: the tiled FP6 operand that
 * quest_quantize_fwd_op writes for the same codes, built from packed b-bit
 * codes (quest_quantize_fwd's layout), so that codes kept at b bits per
 * entry (a frozen layer's weight, for instance) can feed quest_gemm.  The
 * pages time QuEST's 4-bit layer products (pith.science review of QuEST,
 * Figure 5 caption); gfx950 multiplies them as FP6 (see the operand above),
 * and this is the step from the stored codes to that type.
 *   codes    device, quest_codes_bytes(rows, cols, b) bytes
 *   rows     >= 0;  cols a positive multiple of 128 (QUEST_EINVAL
 *            otherwise), at most QUEST_MAX_COLS
 *   b        1 .. 4 (QUEST_EUNSUPPORTED otherwise)
 *   operand  device output, quest_operand_bytes(rows, cols) bytes; the
 *            padding rows of the last 32-row block are not written
 * 16-byte aligned pointers (QUEST_EALIGN); the operand may not overlap the
 * codes (QUEST_EINVAL).  Asynchronous on `stream`.
 */
quest_status quest_codes_to_operand(const uint8_t* codes, int64_t rows, int64_t cols, int b, uint8_t* operand,
                                    void* stream);

/*
 * Forward writing the matrix-core operand: the quantiser of
 * quest_quantize_fwd_ex, whose levels go to `operand` instead of a
 * dequantised tensor.  Codes and mask are optional (an inference forward
 * needs neither).
 *   b        1 .. 4 (QUEST_EUNSUPPORTED otherwise)
 *   cols     a multiple of 128 as well as of `block` (QUEST_EUNSUPPORTED)
 *   codes    device output or NULL (not written)
 *   scale    device output, rows floats (required)
 *   mask     device output or NULL (not written)
 *   operand  device output, quest_operand_bytes(rows, cols) bytes, 16-byte
 *            aligned, overlapping no other argument (required when rows > 0)
 * Everything else as for quest_quantize_fwd_ex.  The operand's levels are
 * those of the codes: h = u - (L - 1)/2 for the code u the call stores.
 */
quest_status quest_quantize_fwd_op(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                   int b, double trust, uint8_t* codes, float* scale, uint8_t* mask,
                                   uint8_t* operand, void* stream);

/*
 * The forward of quest_quantize_fwd_op on several tensors in one call: the
 * outputs are those of calling quest_quantize_fwd_op on each tensor in turn
 * (same block, bit width, trust factor and input dtype), bit for bit.  A
 * quantisation-aware layer quantises its activations and its weights before
 * every product (pith.science review of QuEST, "What carries the argument";
 * Figure 2 caption); with bf16 inputs the library launches the tensors whose
 * rows have 512, 1024 or 2048 entries together (one launch per width for up
 * to four tensors) and launches the others one by one.
 *
 *   tensors  host array of `count` descriptors, read during the call only;
 *            each names x, rows, cols, codes, scale, mask and operand as the
 *            arguments of quest_quantize_fwd_op (codes and mask may be NULL;
 *            a tensor with rows == 0 is skipped and its pointers are not
 *            read)
 *   count    >= 0 (0: nothing is done)
 *   x_dtype, block, b, trust, stream: as for quest_quantize_fwd_op, for
 *            every tensor
 * Errors: everything quest_quantize_fwd_op rejects for any tensor, with the
 * same status; count < 0 or tensors NULL with count > 0 is QUEST_EINVAL; an
 * output of one tensor overlapping an input or output of another is
 * QUEST_EINVAL (inputs may overlap each other).  Validation covers every
 * tensor before the first launch, so on error nothing is written.
 */
typedef struct {
  const void* x;
  int64_t rows;
  int64_t cols;
  uint8_t* codes;
  float* scale;
  uint8_t* mask;
  uint8_t* operand;
} quest_fwd_op_tensor;

quest_status quest_quantize_fwd_op_group(const quest_fwd_op_tensor* tensors, int count, quest_dtype x_dtype,
                                         int block, int b, double trust, void* stream);

/*
 * Product of two quantised operands along their quantised axis:
 *   out[i, j] = Delta_a[i] Delta_b[j] * sum_c h_a[i, c] h_b[j, c],
 *   Delta = 2 s / (L - 1) from each operand's clip scale and bit width,
 * which is Q(A) Q(B)^T for the grid values Q of both (in the Hadamard
 * domain, where the product of two transformed operands equals the product
 * of their original-domain reconstructions: pith.science review of QuEST,
 * "Assumptions & free parameters").  Both operands come from
 * quest_quantize_fwd_op with the same cols = k.  The sum of half-integer
 * products is accumulated exactly in fp32; the result is rounded three
 * times (Delta_a Delta_b, the product, and the output type).
 *   a, a_scale  device, quest_operand_bytes(m, k) bytes and m floats (s_r)
 *   b, b_scale  device, quest_operand_bytes(n, k) bytes and n floats
 *   m, n        >= 0 (0: nothing is done); m <= 2^30, n <= 2^20, and at
 *               most 2^23 - 1 output tiles of 256 x 256, ceil(m / 256) *
 *               ceil(n / 256) (QUEST_EUNSUPPORTED)
 *   a_bits, b_bits  1 .. 4: the bit widths the operands were quantised to
 *   k           the common number of columns: a positive multiple of 128,
 *               at most 65536 (QUEST_EUNSUPPORTED; above that the fp32 sum
 *               would no longer be exact)
 *   out         device output, m x n row-major elements of out_dtype
 *               (QUEST_F32 or QUEST_BF16, round to nearest even), 16-byte
 *               aligned, overlapping no input (QUEST_EINVAL)
 * All pointers 16-byte aligned (QUEST_EALIGN).
 */
quest_status quest_gemm(const uint8_t* a, const float* a_scale, int64_t m, int a_bits, const uint8_t* b,
                        const float* b_scale, int64_t n, int b_bits, int64_t k, void* out, quest_dtype out_dtype,
                        void* stream);

/*
 * Other grids of the pages: FP4 levels and 2:4-sparse codes.  The pages
 * extend the method to an FP4 format and to 2:4-sparse INT4 (pith.science
 * review of QuEST, the list of contributions and the captions of Figures 3
 * and 4; atlas.scime.ai summary, "Key results": FP4 fits a slightly worse
 * scaling law, which the authors put down to a higher Gaussian MSE when
 * clipping is allowed; the ablation table: 2:4 sparsity added to INT4).
 * Both run the same Hadamard transform, RMS scale and trust rule; the trust
 * backward (quest_trust_bwd) takes their masks unchanged.
 */

/* alpha of the FP4 grid (largest level at alpha * RMS), minimising the
   expected squared error for a standard Gaussian; host, cached. */
double quest_fit_alpha_fp4(void);

/*
 * Forward onto the FP4 grid: levels e2m1(code) * s / 6 with the E2M1
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP MX v1.0) and
 * s = quest_fit_alpha_fp4() * RMS.  The code is the E2M1 bit pattern (sign
 * bit 3) of the level nearest to 6 y / s (ties to the code with mantissa bit
 * 0, saturating at +-6; the zero level is code 0), packed 4 bits per element
 * LSB-first (quest_codes_bytes(rows, cols, 4)).  Trusted iff
 * |y| <= s (1 + t / 6): beyond the grid, t times half the outermost interval.
 *   codes  device output or NULL;  mask  device output (required)
 *   dq     device output of dq_dtype or NULL: e2m1(code) * (s / 6)
 * Everything else as for quest_quantize_fwd_ex.
 */
quest_status quest_quantize_fwd_fp4(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                    double trust, uint8_t* codes, float* scale, uint8_t* mask, void* dq,
                                    quest_dtype dq_dtype, void* stream);

/*
 * Forward onto the 2:4-sparse b-bit grid (b = 1..4, QUEST_EUNSUPPORTED
 * otherwise).  In every group of 4 consecutive Hadamard-domain entries of a
 * row (columns 4g .. 4g + 3) the 2 of largest |y| are kept (on equal
 * magnitudes the lower index); s = alpha_b * RMS of the kept entries; kept
 * entries take the code and level of the dense quantiser with that s; pruned
 * entries reconstruct as 0.  Mask: kept entries as in quest_quantize_fwd_ex;
 * pruned entries trusted iff |y| <= Delta / 2 (the trust rule with q = 0).
 *   codes  device output or NULL: per row the cols / 2 kept codes, b bits
 *          each, LSB-first in column order (quest_sparse24_codes_bytes)
 *   index  device output or NULL: per row the kept entries' positions inside
 *          their group, 2 bits each, LSB-first in the same order
 *          (quest_sparse24_index_bytes)
 *   dq     device output or NULL: the dense reconstruction (zeros pruned)
 * Everything else as for quest_quantize_fwd_ex.
 */
quest_status quest_quantize_fwd_sparse24(const void* x, quest_dtype x_dtype, int64_t rows, int64_t cols, int block,
                                         int b, double trust, uint8_t* codes, uint8_t* index, float* scale,
                                         uint8_t* mask, void* dq, quest_dtype dq_dtype, void* stream);

/* FP4 codes back to e2m1(code) * (s / 6), rounded to out_dtype.  Arguments
   as for quest_dequantize with b = 4. */
quest_status quest_dequantize_fp4(const uint8_t* codes, const float* scale, int64_t rows, int64_t cols, void* out,
                                  quest_dtype out_dtype, void* stream);

/* 2:4-sparse codes back to the dense reconstruction: (2u - L + 1) s / (L - 1)
   at the kept positions, 0 elsewhere.  b = 1..4; index as written by
   quest_quantize_fwd_sparse24; otherwise as quest_dequantize. */
quest_status quest_dequantize_sparse24(const uint8_t* codes, const uint8_t* index, const float* scale, int64_t rows,
                                       int64_t cols, int b, void* out, quest_dtype out_dtype, void* stream);

/* Bytes of the 2:4-sparse codes: rows * (cols / 2) * b / 8; of the positions:
   rows * cols / 8 (0 on invalid sizes: cols a positive multiple of 64, b 1..4). */
size_t quest_sparse24_codes_bytes(int64_t rows, int64_t cols, int b);
size_t quest_sparse24_index_bytes(int64_t rows, int64_t cols);

/* Bytes of the packed codes: rows * cols * b / 8 (0 on invalid sizes). */
size_t quest_codes_bytes(int64_t rows, int64_t cols, int b);

/* Bytes of the packed mask: rows * cols / 8 (0 on invalid sizes). */
size_t quest_mask_bytes(int64_t rows, int64_t cols);

/* Static English name of a status code ("unknown status" otherwise). */
const char* quest_status_string(quest_status s);

#ifdef __cplusplus
}
#endif

#endif /* QUEST_H */
