/*
 * whtq.h -- C ABI of libwhtq, batched Walsh-Hadamard transforms for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (cited by short key):
 *   [HARP]  "HARP: Hadamard-Preconditioned Adaptive Rotation Processor for
 *           Extreme LLM Quantization" (gist.science explainer), technical
 *           summary: section 1 (randomized Hadamard transform: a fixed random
 *           sign diagonal followed by the Hadamard transform, exactly
 *           orthogonal, O(d log d)); 2.1 (mixed-radix schedule, prod b_t = d,
 *           block-diagonal orthogonal stages on stride-permuted groups); 2.2
 *           (B_{t,c} = Q_{t,c} G_{b_t}, G the normalised Sylvester Hadamard;
 *           Theta = 0 gives back the fixed RHT); 2.4 (O(d log d) stages).
 *   [QWHA]  "QWHA: Quantization-Aware Walsh-Hadamard Adaptation ..."
 *           (gist.science explainer), section 2.1: Delta W = F H^-1, a single
 *           transform on the input side, F sparse from values c and indices E,
 *           +-1 kernel computed with additions and subtractions only.
 *
 * Conventions fixed by this library where the pages leave them open:
 *   - Hn = H / sqrt(n), H the Sylvester matrix H[i][j] = (-1)^popcount(i & j)
 *     (natural order, not sequency order).
 *   - Sign diagonal S: bit j (LSB first) of uint32 word j / 32 set means
 *     s_j = -1; one vector per layer, shared by every row.
 *   - RHT forward y = Hn (S x); inverse x = S Hn y.
 *   - Quantiser: per group of g consecutive transformed coordinates,
 *     s = fp16_rne(max|y| / qmax) with qmax = 2^(b-1) - 1, q = rint(y / s)
 *     (half to even; s = 0 gives q = 0), codes in [-qmax, qmax].
 *   - Codes: row-major, each row a little-endian bit stream of n codes of
 *     b bits (code i in bits [b*i, b*i + b), LSB first, two's complement);
 *     row stride n*b/8 bytes.  Scales: IEEE fp16 bits, [rows][n/g].
 *   - QWHA: F is [d_out x d_in] in CSR; Delta W = F Hn; y = (x Hn) F^T.
 *   - HARP digits: i = sum_t i_t * prod_{u<t} b_u; stage t acts on digit t;
 *     block index c = i with digit t removed (remaining digits in increasing
 *     significance); a block maps out_sub[k] = sum_j B[k][j] in_sub[j].
 *
 * Common rules for every entry point:
 *   - All pointers are device pointers owned by the caller, except
 *     `radices` (host) and those of the host helper qwha_csr_transpose.
 *     The library keeps no pointer after returning and allocates no memory
 *     (scratch space, where an operation needs it, is a caller-provided
 *     workspace argument).
 *   - `stream` is a hipStream_t (NULL = the default stream).  WHTQ_OK means
 *     the work was enqueued; faults surface at the caller's next
 *     synchronisation.  Nothing is read back to the host.
 *   - Every argument check runs before any HIP call, so an error status
 *     means no work was enqueued.
 *   - Matrices are row-major with the transform along the contiguous last
 *     dimension; ld* are row strides in elements (>= the row length).
 *   - Alignment: device base pointers must be 16-byte aligned and
 *     ld * element_size a multiple of 16 bytes, unless a whole row is
 *     shorter than 16 bytes (then element alignment suffices).  Violations
 *     return WHTQ_EALIGN; there is no slower fallback path.
 */
#ifndef WHTQ_H
#define WHTQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WHTQ_ABI_VERSION 4

typedef enum {
  WHTQ_OK = 0,
  WHTQ_EINVAL = 1,       /* bad size, null pointer, bits/group/schedule out of rule */
  WHTQ_EUNSUPPORTED = 2, /* valid request this build has no kernel for            */
  WHTQ_EALIGN = 3,       /* pointer or row stride not 16-byte aligned              */
  WHTQ_EHIP = 4,         /* HIP runtime / launch failure, including no device      */
  WHTQ_ESCRATCH = 5      /* sizes need more than the library's fixed scratch array */
} whtq_status;

typedef enum { WHTQ_F32 = 0, WHTQ_BF16 = 1, WHTQ_F16 = 2, WHTQ_I8 = 3 } whtq_dtype;  /* I8: HARP parameters only */

typedef enum {
  WHTQ_SIGN_NONE = 0,   /* y = Hn x        */
  WHTQ_SIGN_BEFORE = 1, /* y = Hn (S x)    (forward RHT) */
  WHTQ_SIGN_AFTER = 2   /* y = S (Hn x)    (inverse RHT) */
} whtq_sign_mode;

/*
 * wht_batched -- orthonormal (or raw) Sylvester WHT of `rows` rows of length
 * n.  [QWHA] 2.1 (+-1 kernel, add/subtract-only fast transform); [HARP] 1
 * (RHT = sign diagonal then Hadamard).
 *   x [rows][ldx] in x_dtype; y [rows][ldy] in y_dtype.  x == y (exact alias,
 *   equal ld and dtype) is allowed; partial overlap is undefined.
 *   n: power of two in [2, 8192].
 *   dtypes: (f32->f32), (bf16->bf16), (f16->f16), (bf16->f32), (f16->f32).
 *   sign_bits: uint32[ceil(n/32)], required unless sign_mode is NONE.
 *   normalize: 1 -> Hn = H / sqrt(n); 0 -> the raw +-1 product.
 * Arithmetic: fp32 throughout; 16-bit outputs are rounded once (nearest even).
 */
whtq_status wht_batched(const void* x, whtq_dtype x_dtype, void* y, whtq_dtype y_dtype,
                        int64_t rows, int64_t n, int64_t ldx, int64_t ldy,
                        const uint32_t* sign_bits, int sign_mode, int normalize, void* stream);

/*
 * rht_quantize_rtn -- y = Hn (S w) per row, then per-group absmax RTN to
 * signed b-bit codes with fp16 scales.  [HARP] 1 (RHT as incoherence
 * processing before low-bit quantisation, 2-4 bits).
 *   w [rows][ldw] in w_dtype (bf16, f32 or f16).
 *   n: power of two in [64, 8192].  bits: 2, 3 or 4.  group: power of two in
 *   [8, 256] dividing n.  sign_bits: uint32[n/32] or NULL (all +1).
 *   codes: uint8 [rows][n*bits/8] (written).  scales: uint16 fp16 bits
 *   [rows][n/group] (written).
 */
whtq_status rht_quantize_rtn(const void* w, whtq_dtype w_dtype, int64_t rows, int64_t n, int64_t ldw,
                             const uint32_t* sign_bits, int bits, int group,
                             uint8_t* codes, uint16_t* scales, void* stream);

/*
 * rht_dequantize_inverse -- out = S Hn (q * s): unpack codes, scale by the
 * group's fp16 scale, inverse RHT.  Inverse of rht_quantize_rtn up to the
 * quantisation error ([HARP] 1: the transform is exactly orthogonal).
 *   codes / scales as written by rht_quantize_rtn with the same n, bits,
 *   group.  out [rows][ldo] in out_dtype (bf16, f32 or f16).
 */
whtq_status rht_dequantize_inverse(const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t n,
                                   const uint32_t* sign_bits, int bits, int group,
                                   void* out, whtq_dtype out_dtype, int64_t ldo, void* stream);

/*
 * rht_lowbit_gemv -- y[t][o] = sum_i x[t][i] W_hat[o][i], the product of
 * activations with weights held as rht_quantize_rtn codes, W_hat[o] =
 * S Hn (q[o] * s[o]) (the rows rht_dequantize_inverse would write).  The
 * rotation is applied to the activations instead of the weights ([HARP] 1
 * and 2.4: low-bit weights in the rotated basis, the RHT applied online in
 * fused O(d log d) kernels): y[t][o] = sum_k q[o][k] s[o][k/g] (Hn S x_t)[k].
 *   x [tokens][ldx] bf16; y [tokens][ldy] bf16 (column o of row t is the
 *   output of weight row o; ldy >= rows).  codes / scales as written by
 *   rht_quantize_rtn with the same n, bits, group and sign_bits.
 *   n: 4096 or 8192.  bits: 2 or 4.  group: power of two in [32/bits, 256].
 *   Arithmetic: (Hn S x_t) in fp32, multiplied by a per-token power of two
 *   sigma that puts its largest magnitude in [2^13, 2^14) and rounded to
 *   16-bit integers X (fixed point); the code x X products of one scale
 *   group are summed exactly in int32 (4-bit integer dot products), then
 *   y += s * acc in fp32, y * 1/(sigma sqrt(n)) rounded once to bf16.  Tokens are processed in
 *   passes of up to 4 (n = 4096) or 2 (n = 8192), each reading the codes
 *   once: a decode-size product, not a GEMM.
 *   Errors: EINVAL for bad sizes or NULL pointers, EUNSUPPORTED for other
 *   n, bits = 3 or smaller groups, EALIGN as in the common rules (y needs
 *   2-byte alignment only).
 */
whtq_status rht_lowbit_gemv(const void* x, int64_t tokens, int64_t ldx, const uint8_t* codes,
                            const uint16_t* scales, int64_t rows, int64_t n, const uint32_t* sign_bits,
                            int bits, int group, void* y, int64_t ldy, void* stream);

/*
 * qwha_adapter_forward -- y[t][o] = sum_{k in row o of F} F[o][k] * (Hn x_t)[k],
 * the QWHA adapter output x Delta W^T with Delta W = F Hn ([QWHA] 2.1).
 *   x [tokens][ldx] bf16; y [tokens][ldy] bf16; d_in a power of two in
 *   [64, 8192] (others: WHTQ_EUNSUPPORTED).
 *   F: CSR [d_out x d_in]: row_ptr int32[d_out + 1] (row_ptr[0] = 0,
 *   row_ptr[d_out] = nnz, non-decreasing), col_idx int32[nnz] in [0, d_in),
 *   vals[nnz] in val_dtype (bf16 or f32).  The library does not read the CSR
 *   on the host: a malformed CSR gives undefined results.
 *   d_out in [1, 4096] (any value); col_idx and vals 16-byte aligned (the
 *   common rule).  Accumulation in fp32; Hn x is kept on chip in fp16 with a
 *   per-token power-of-two scale; each output is rounded once to bf16.
 *   Widths other than 4096 use two exact identities of the Sylvester matrix:
 *   for d_in < 4096, (Hn x)[k] is the k-th entry of the 4096-point transform
 *   of x zero-extended, times 64 / sqrt(d_in); for d_in = 8192, the half h of
 *   H_8192 x is H_4096 (x_lo + x_hi) or H_4096 (x_lo - x_hi) over 1/sqrt(2),
 *   and each token's fp16 scale then comes from the bound 64 ||x||_2 rather
 *   than from max |(Hn x)_k| (fewer bits for small entries of that token).
 */
whtq_status qwha_adapter_forward(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t d_in,
                                 int64_t ldx, const int32_t* row_ptr, const int32_t* col_idx,
                                 const void* vals, whtq_dtype val_dtype, int64_t d_out, int64_t nnz,
                                 void* y, whtq_dtype y_dtype, int64_t ldy, void* stream);

/*
 * ---- Forward plans.  In [QWHA] 2.1 the support of F (its row_ptr and
 * col_idx) is chosen once and then fixed while only the values train, so the
 * forward's per-chunk bookkeeping, which depends on row_ptr alone (rows cut
 * into segments of at most 128 entries and ordered by length for the
 * gather), can be computed once and reused by every call and every token
 * tile.  A plan holds it for one (tokens, d_out, nnz, row_ptr) on one device;
 * it is an opaque device buffer the caller allocates.
 *
 * qwha_forward_plan_bytes -- bytes a plan needs for these sizes on the
 *   current device (the split of F's rows across blocks follows the token
 *   count and the device's CU count); 0 for d_in = 8192 (that kernel needs
 *   no plan); -1 for invalid sizes (as in qwha_adapter_forward, tokens >= 1)
 *   or when no device is present.
 */
int64_t qwha_forward_plan_bytes(int64_t tokens, int64_t d_in, int64_t d_out, int64_t nnz);

/*
 * qwha_forward_plan -- builds the plan into `plan` (device, 16-byte aligned,
 *   plan_bytes >= qwha_forward_plan_bytes(...), caller-owned) from row_ptr
 *   (device int32[d_out + 1], the CSR rules of qwha_adapter_forward) on
 *   `stream`.  Reads nothing but row_ptr; asynchronous like the other device
 *   calls.  d_in = 8192: returns WHTQ_OK and writes nothing.
 *   Errors: WHTQ_EINVAL (sizes, null pointers, plan_bytes too small),
 *   WHTQ_EALIGN, WHTQ_EUNSUPPORTED (d_in, d_out > 4096), WHTQ_EHIP.
 */
whtq_status qwha_forward_plan(int64_t tokens, int64_t d_in, const int32_t* row_ptr, int64_t d_out, int64_t nnz,
                              void* plan, int64_t plan_bytes, void* stream);

/*
 * qwha_adapter_forward_planned -- qwha_adapter_forward with a plan (or
 *   plan = NULL, the same as qwha_adapter_forward).  Arguments, layouts and
 *   errors as qwha_adapter_forward, plus: plan 16-byte aligned, plan_bytes
 *   its size (>= 256 when plan is not NULL).  Results are bit-identical with
 *   and without a plan.  A plan whose header does not match (another d_out,
 *   nnz or split of the rows, one that ran out of room, or one larger than
 *   plan_bytes) is ignored and the call prepares its chunks itself; a plan
 *   built from a different row_ptr with the same sizes gives undefined
 *   results, so rebuild it whenever the support changes.
 */
whtq_status qwha_adapter_forward_planned(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t d_in,
                                         int64_t ldx, const int32_t* row_ptr, const int32_t* col_idx,
                                         const void* vals, whtq_dtype val_dtype, int64_t d_out, int64_t nnz,
                                         const void* plan, int64_t plan_bytes, void* y, whtq_dtype y_dtype,
                                         int64_t ldy, void* stream);

/*
 * ---- QWHA adapter backward (training).  [QWHA] 2.1 makes the adapter linear
 * in its input x and in the value vector c placed at the index list E, so
 * its gradients for an upstream dy = dL/dy are the adjoint products:
 *   dx   = dy Delta W = (dy F) Hn                  (Hn is symmetric)
 *   dc_e = sum_t dy[t][o_e] (Hn x_t)[k_e]          (entry e at row o_e, column k_e of F)
 */

/*
 * qwha_csr_transpose -- HOST helper: the CSR of F^T from the CSR of F.
 *   All pointers are HOST pointers (caller-owned).  Inputs: row_ptr
 *   int32[d_out + 1], col_idx int32[nnz] (the CSR of F, d_out x d_in).
 *   Outputs: t_row_ptr int32[d_in + 1], t_col_idx int32[nnz] (the rows o of F
 *   holding each entry, ascending within a column), t_perm int32[nnz] (entry j
 *   of F^T is entry t_perm[j] of F).  The support E is fixed during training,
 *   so this runs once; the values are re-permuted per step by
 *   qwha_permute_values.  Unlike the device entry points this one reads the
 *   CSR and returns WHTQ_EINVAL if it is malformed (row_ptr[0] != 0,
 *   row_ptr[d_out] != nnz, decreasing row_ptr, a column outside [0, d_in)).
 */
whtq_status qwha_csr_transpose(const int32_t* row_ptr, const int32_t* col_idx, int64_t d_out, int64_t d_in,
                               int64_t nnz, int32_t* t_row_ptr, int32_t* t_col_idx, int32_t* t_perm);

/*
 * qwha_permute_values -- out[j] = vals[perm[j]], j < nnz (device).  With the
 * t_perm of qwha_csr_transpose it gives the values of F in the entry order of
 * F^T.  vals / out: bf16 or f32 (val_dtype), out must not alias vals; perm
 * entries must lie in [0, nnz) (not checked on the host).
 */
whtq_status qwha_permute_values(const void* vals, whtq_dtype val_dtype, const int32_t* perm, int64_t nnz,
                                void* out, void* stream);

/*
 * qwha_adapter_backward_input -- dx = (dy F) Hn: dx[t][k] = (Hn u_t)[k] with
 * u_t[j] = sum_{o in row j of F^T} F[o][j] dy[t][o].
 *   dy [tokens][lddy] bf16 (d_out columns; 2-byte alignment suffices, 16-byte
 *   aligned rows are read with 16-byte loads); dx [tokens][lddx] bf16 (d_in
 *   columns, a power of two in [64, 8192]; d_out in [1, 4096]).  F^T as CSR: t_row_ptr int32[d_in + 1],
 *   t_col_idx int32[nnz] in [0, d_out), t_vals[nnz] (bf16 or f32), e.g. from
 *   qwha_csr_transpose + qwha_permute_values; 16-byte aligned t_col_idx and
 *   t_vals.  A malformed CSR gives undefined results (it is not read on the
 *   host).
 *   Arithmetic: dy is kept on chip in fp16 with a per-token power-of-two
 *   scale (exact for bf16 inputs in range), fp32 accumulation of dy F, whose
 *   rows are rounded once to bf16 on chip before the fp32 transform; each
 *   output rounded once to bf16.  d_in other than 4096: the identities of
 *   qwha_adapter_forward (zero extension below 4096, the top-bit split at
 *   8192).
 */
whtq_status qwha_adapter_backward_input(const void* dy, whtq_dtype dy_dtype, int64_t tokens, int64_t d_out,
                                        int64_t lddy, const int32_t* t_row_ptr, const int32_t* t_col_idx,
                                        const void* t_vals, whtq_dtype val_dtype, int64_t d_in, int64_t nnz,
                                        void* dx, whtq_dtype dx_dtype, int64_t lddx, void* stream);

/*
 * qwha_grad_values_workspace_bytes -- size in bytes of the workspace that
 * qwha_adapter_grad_values needs for these sizes (a function of the sizes
 * only); -1 for invalid sizes (d_in must be a power of two in [64, 8192]), 0
 * when tokens or nnz is 0.
 */
int64_t qwha_grad_values_workspace_bytes(int64_t tokens, int64_t d_in, int64_t nnz);

/*
 * qwha_adapter_grad_values -- dc[e] = sum_t dy[t][o_e] * (Hn x_t)[col_idx[e]]
 * for every entry e of F's CSR, o_e its row (the gradient of the values c).
 *   x [tokens][ldx] bf16 (d_in a power of two in [64, 8192]); dy
 *   [tokens][lddy] bf16 (d_out in
 *   [1, 4096], 2-byte alignment suffices); row_ptr int32[d_out + 1], col_idx int32[nnz] (the CSR of F;
 *   not read on the host: malformed input gives undefined values, never an
 *   access outside x, dy, dc or the workspace); dc float32[nnz] (written, in
 *   CSR entry order).  tokens = 0 gives dc = 0.
 *   workspace: device memory of at least
 *   qwha_grad_values_workspace_bytes(tokens, d_in, nnz) bytes, 16-byte
 *   aligned, overwritten (Hn x in fp32 and per-token-slab partial sums);
 *   a smaller workspace_bytes returns WHTQ_EINVAL.
 *   Arithmetic: Hn x in fp32 (d_in < 4096: the 4096-point transform of x
 *   zero-extended, scaled; d_in = 8192: the two 4096-point halves of the
 *   top-bit split); products and sums in fp32, over tokens in order within
 *   fixed token slabs, then over slabs in order (deterministic).
 */
whtq_status qwha_adapter_grad_values(const void* x, const void* dy, whtq_dtype dtype, int64_t tokens,
                                     int64_t d_in, int64_t d_out, int64_t ldx, int64_t lddy,
                                     const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, float* dc,
                                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qwha_adapter_grad_values_noalloc -- qwha_adapter_grad_values without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments (minus workspace / workspace_bytes), kernels,
 * arithmetic and results; the scratch space lives in a file-scope device
 * array of WHTQ_QWHA_DC_SCRATCH_BYTES bytes that each GPU the library runs
 * on holds until the process ends.  The call allocates nothing.
 *   Sizes whose qwha_grad_values_workspace_bytes exceeds
 *   WHTQ_QWHA_DC_SCRATCH_BYTES return WHTQ_ESCRATCH before any HIP call
 *   (64 MiB covers 2048 tokens x 262,144 entries at d_in <= 4096; roughly
 *   tokens * 16 KiB (32 KiB at d_in = 8192) + token slabs * nnz * 4 bytes).
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (different streams, or different host threads) race and give
 *   undefined results.  Calls ordered on one stream are safe; nothing carries
 *   over from one call to the next (every scratch byte a call reads, the
 *   same call has written).
 */
#define WHTQ_QWHA_DC_SCRATCH_BYTES (64ll << 20)
whtq_status qwha_adapter_grad_values_noalloc(const void* x, const void* dy, whtq_dtype dtype, int64_t tokens,
                                             int64_t d_in, int64_t d_out, int64_t ldx, int64_t lddy,
                                             const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                             float* dc, void* stream);

/*
 * harp_rotate -- y = Stage_{m-1}( ... Stage_0( P x ) ), P = Hn S if
 * precondition else I; stage t applies d / b_t independent b_t x b_t blocks
 * along digit t ([HARP] 2.1, 2.2).
 *   x, y [tokens][ld] in dtype, WHTQ_BF16 or WHTQ_F32 (both the same
 *   dtype; WHTQ_F16 rows are WHTQ_EUNSUPPORTED); x == y not allowed.
 *   radices: HOST int32[n_stages], each >= 2, product == d ([HARP] 2.1:
 *   e.g. 8, 8, 8, 5, 2 for d = 5120).  This build runs radices up to 16,
 *   d <= 8192 and up to 16 stages (WHTQ_EUNSUPPORTED otherwise).
 *   precondition: Hn is the Sylvester matrix, so it needs d a power of two
 *   (WHTQ_EINVAL otherwise).
 *   blocks: device, stage-major, stage t as [d / b_t][b_t][b_t] row-major
 *   (B[k][j] at k * b_t + j), in blocks_dtype: WHTQ_F32 or WHTQ_F16 (half
 *   the bytes read per call).
 *   Arithmetic, bf16 rows with d = 4096 and radices (16, 16, 16): each token row is scaled
 *   by an exact power of two that puts its L2 norm in [2^13, 2^14) and kept
 *   on chip in fp16; the preconditioning Hn = (H16 / 4) (x) (H16 / 4) (x)
 *   (H16 / 4) and every block stage run as 16 x 16 x 16 MFMAs with fp16
 *   operands and fp32 accumulation (fp32 blocks are rounded to fp16 in the
 *   kernel, so both block dtypes give the same result for the same
 *   fp16-representable values), the result of each rounded to fp16.  Every
 *   other schedule, and fp32 rows with any schedule: fp32 on chip and fp32
 *   arithmetic (fp16 blocks widened exactly), the preconditioning as
 *   in-register Hadamard butterflies.  bf16 output is rounded once (nearest
 *   even); fp32 output is the fp32 result.
 *   sign_bits: uint32[ceil(d/32)] or NULL (all +1); used when
 *   precondition != 0.
 */
whtq_status harp_rotate(const void* x, void* y, whtq_dtype dtype, int64_t tokens, int64_t d,
                        int64_t ldx, int64_t ldy, const uint32_t* sign_bits, int precondition,
                        const int32_t* radices, int n_stages, const void* blocks,
                        whtq_dtype blocks_dtype, void* stream);

/*
 * harp_build_blocks -- the blocks B_{t,c} = Q_{t,c}(theta) G_{b_t} that
 * harp_rotate takes, from their parameters ([HARP] 2.2: Q a Givens rotation
 * for b_t = 2, a Cayley map for b_t > 2, G a fixed base mixer; theta = 0
 * gives B = G, the fixed Hadamard rotation; [HARP] 2.4: int8 storage).
 *   Conventions: Givens Q = [[cos t, -sin t], [sin t, cos t]] (one angle per
 *   block); Cayley Q = (I - A)(I + A)^-1 with A skew-symmetric, its
 *   b(b-1)/2 parameters the strict upper triangle row by row (A[i][j] = p,
 *   i < j, A[j][i] = -p).
 *   params: device, stage-major, stage t as [d / b_t][P_t] with P_t = 1
 *   (b_t = 2) or b_t (b_t - 1) / 2; WHTQ_F32 values, or WHTQ_I8 codes q with
 *   theta = scales[t] * q (scales: device float32[n_stages], required then).
 *   radices: HOST int32[n_stages], each in [2, 16] in this build, product d.
 *   mixers: device float32, stage-major b_t x b_t matrices G_t (row-major),
 *   or NULL for the normalised Sylvester Hadamard (every radix a power of
 *   two, else WHTQ_EINVAL).
 *   blocks: device, written in harp_rotate's layout ([d / b_t][b_t][b_t] per
 *   stage, stage-major), WHTQ_F32 or WHTQ_F16 (rounded once).
 *   Arithmetic: fp32; Q by Gauss-Jordan elimination of [I + A | I - A]
 *   (I + A has the identity as symmetric part: no pivoting needed).
 */
whtq_status harp_build_blocks(const void* params, whtq_dtype params_dtype, const float* scales, int64_t d,
                              const int32_t* radices, int n_stages, const float* mixers, void* blocks,
                              whtq_dtype blocks_dtype, void* stream);

/*
 * QWHA adapter initialisation ([QWHA] 2.2: AdaAlloc spreads a parameter
 * budget over the output channels in proportion to their activation error,
 * with a per-channel minimum, and keeps each channel's largest-magnitude
 * coefficients; refinement then sets the kept values by least squares on
 * the layer output error).  With Delta W = F Hn ([QWHA] 2.1), Q the RHT +
 * RTN quantiser above and x [T][n] calibration tokens:
 *   F_dense = (W - Q(W)) Hn,   Z = x Hn,   G = Z^T Z,   P = F_dense G,
 *   e_o = ||x (W - Q(W))[o]^T|| = sqrt(F_dense[o] G F_dense[o]^T),
 *   c_o solves G[E_o][E_o] c = P[o][E_o]   (least squares on support E_o).
 * A full initialisation is error_coeffs, gram (once per calibration batch,
 * accumulate = 1 after the first), channel_errors, allocate (on the host),
 * select, refine.  All arithmetic is fp32 (fp32 accumulation); the
 * allocation is fp64 on the host.  n (d_in) is a power of two in
 * [256, 8192] (WHTQ_EUNSUPPORTED otherwise; error_coeffs takes the
 * quantiser's range); float matrices are 16-byte aligned with row strides a
 * multiple of 4 elements.
 *
 * qwha_init_error_coeffs -- f[rows][ldf] (fp32, device) = (W - Q(W)) Hn for
 *   stored codes/scales of W (as from rht_quantize_rtn with the same signs,
 *   bits, group).  w must not alias f.
 */
#define WHTQ_QWHA_INIT_MAX_SUPPORT 128 /* largest per-channel budget refine takes */

whtq_status qwha_init_error_coeffs(const void* w, whtq_dtype w_dtype, int64_t rows, int64_t n, int64_t ldw,
                                   const uint8_t* codes, const uint16_t* scales, const uint32_t* sign_bits,
                                   int bits, int group, float* f, int64_t ldf, void* stream);

/*
 * qwha_init_gram -- g (device fp32 [n][n], row stride n) = Z^T Z, or
 *   g + Z^T Z with accumulate = 1, Z = x Hn for tokens rows of x (bf16, fp16
 *   or fp32, row stride ldx).  z: device fp32 workspace [tokens][n] that
 *   receives Z (z == g is WHTQ_EINVAL).  tokens = 0 with accumulate = 0
 *   zeroes g.
 */
whtq_status qwha_init_gram(const void* x, whtq_dtype x_dtype, int64_t tokens, int64_t n, int64_t ldx, float* z,
                           float* g, int accumulate, void* stream);

/*
 * qwha_init_channel_errors -- p (device fp32 [rows][n], row stride n) =
 *   F_dense G and err[o] (device fp32[rows]) = sqrt(max(0, p[o] . f[o])),
 *   the activation error of channel o.  g symmetric (from qwha_init_gram).
 *   p or err equal to f, g or each other is WHTQ_EINVAL.
 */
whtq_status qwha_init_channel_errors(const float* f, int64_t rows, int64_t n, int64_t ldf, const float* g,
                                     float* p, float* err, void* stream);

/*
 * qwha_init_allocate -- HOST call on host arrays: per-channel budgets
 *   n_o in [floor, cap] with sum n_o = total, written as a CSR row pointer
 *   row_ptr[rows + 1] (row_ptr[0] = 0).  Reading of [QWHA] 2.2: real budgets
 *   clip(lam e_o, floor, cap) with lam found by bisection so that they sum
 *   to total (the largest lam found whose sum does not exceed it), rounded
 *   down, then one more to the channels of largest fractional part (ties to
 *   the lower index; capped channels excluded); all-zero err gives total /
 *   rows each.  WHTQ_EINVAL: total outside [floor rows, cap rows] or above
 *   INT32_MAX, cap > n, negative or non-finite err, or a total that channels
 *   with zero error (held at the floor) make unreachable;
 *   WHTQ_EUNSUPPORTED: cap > WHTQ_QWHA_INIT_MAX_SUPPORT.
 */
whtq_status qwha_init_allocate(const float* err, int64_t rows, int64_t n, int64_t total, int floor, int cap,
                               int32_t* row_ptr);

/*
 * qwha_init_select -- for each row the budget row_ptr[o+1] - row_ptr[o]
 *   (device row_ptr, each budget in [0, n]) column indices of largest
 *   |f[o][k]|, ties to the lower k, written ascending to device
 *   col_idx[row_ptr[o] ..].  Rows whose budget is outside [0, n] are left
 *   unwritten.  row_ptr must start at 0 and be non-decreasing, and col_idx
 *   must hold at least row_ptr[rows] entries: neither is read on the host,
 *   and a row_ptr that points past col_idx writes out of bounds.
 */
whtq_status qwha_init_select(const float* f, int64_t rows, int64_t n, int64_t ldf, const int32_t* row_ptr,
                             int32_t* col_idx, void* stream);

/*
 * qwha_init_refine -- vals[row_ptr[o] + a] (device fp32, CSR order) = c_a
 *   with G[E][E] c = P[o][E], E = col_idx[row_ptr[o] .. row_ptr[o+1]) (from
 *   qwha_init_select), p row stride n.  Cholesky factorisation in fp32; a row
 *   whose G[E][E] is not positive definite (fewer calibration tokens than
 *   its budget) gives values without meaning, NaN where a pivot is zero or
 *   negative (a zero G gives NaN throughout); a row whose budget exceeds
 *   WHTQ_QWHA_INIT_MAX_SUPPORT gives NaN.  row_ptr must start at 0 and be
 *   non-decreasing, col_idx and vals must hold at least row_ptr[rows]
 *   entries, and every col_idx entry must lie in [0, n): they are not read
 *   on the host, and values outside these rules read or write out of bounds.
 */
whtq_status qwha_init_refine(const float* g, int64_t n, const float* p, int64_t rows, const int32_t* row_ptr,
                             const int32_t* col_idx, float* vals, void* stream);

/*
 * whtq_stream_probe -- measurement helper, not part of the transform path:
 *   reads in_bytes of src and writes out_bytes of dst (an index pattern) with
 *   coalesced 16-byte accesses, blocks split between the two streams in
 *   proportion to their bytes.  It is the plain-copy reference against which
 *   a kernel moving the same bytes reports its "% achievable" bandwidth.
 *   Sizes must be non-negative multiples of 16 (EINVAL), pointers 16-byte
 *   aligned (EALIGN); src is only read, dst's contents are overwritten.
 */
whtq_status whtq_stream_probe(const void* src, int64_t in_bytes, void* dst, int64_t out_bytes, void* stream);

const char* whtq_status_string(whtq_status s);
int whtq_last_hip_error(void); /* hipError_t behind this thread's last WHTQ_EHIP */
int whtq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WHTQ_H */
