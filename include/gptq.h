/*
 * gptq.h - C ABI of the MI355X (gfx950) GPTQ per-layer quantization solve.
 *
 * The solve follows the GPTQ description of "GPTQ 实战" chapter 5 (CSDN),
 * section 5.1.8 (quantize one column, spread its error over the columns not
 * yet quantized with the Cholesky factor of the inverse Hessian, lazy batches
 * of 128 columns) and the BaseQuantizeConfig fields of the AutoGPTQ examples
 * walkthrough, section 1.4 (bits, group_size, damp_percent, desc_act,
 * static_groups, sym).  A layer is solved by four calls:
 *
 *   gptq_hessian_accumulate   S += X^T X over token chunks      (any number)
 *   gptq_prepare_hinv         H = 2 S / N, damping, act-order, inverse factor U
 *   gptq_quantize_layer       column sweep -> codes, scales, zeros, g_idx
 *   gptq_pack                 codes -> int32 qweight
 *
 * and the quantized layer is applied with
 *
 *   gptq_dequant_matmul       y = x W^T, W dequantized from qweight / scales / zeros / g_idx
 *
 * and a layer quantized with act-order (desc_act) groups can first be put in
 * group order once, so that the product reads one scale per 32 codes:
 *
 *   gptq_dequant_order            channels sorted by group, codes repacked
 *   gptq_dequant_matmul_ordered   y = x W^T on the reordered layer
 *
 * Conventions shared by every call
 *   - All array pointers are DEVICE pointers on the current HIP device; the
 *     caller owns every buffer (inputs, outputs, workspaces).  The library
 *     allocates no device memory.
 *   - Matrices are row-major.  W is [d_out, d_in] (nn.Linear layout), X is
 *     [n_tokens, d_in] with row stride ldx elements.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns; results are valid once
 *     the stream has reached that point.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns GPTQ_ERR_INVALID_ARG and enqueues nothing.  A failed
 *     kernel launch returns GPTQ_ERR_HIP.
 *   - Sizes: d_in and d_out at most 2^20, token counts (n_tokens, m) at most
 *     2^40; larger (or non-positive where a positive size is required)
 *     values return GPTQ_ERR_INVALID_ARG, and 0 from the size queries.
 *   - Workspaces: query the size with the matching *_workspace_size call and
 *     pass at least that many bytes, 256-byte aligned.  Their contents on
 *     entry do not matter and are undefined on exit.  Concurrent calls must
 *     not share a workspace.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1,  /* rejected on the host, nothing enqueued */
  GPTQ_ERR_NOT_SPD = 2,      /* reserved for host wrappers reading info_dev */
  GPTQ_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed */
  GPTQ_ERR_WORKSPACE = 4,    /* workspace missing, too small or misaligned */
  GPTQ_ERR_TOO_LARGE = 5     /* needs more than the library's fixed scratch buffer */
} gptq_status;

/* Element types of X, W and x, passed as int32_t (any other value:
 * GPTQ_ERR_INVALID_ARG, or 0 from a size query). */
typedef enum { GPTQ_F32 = 0, GPTQ_BF16 = 1 } gptq_dtype;

/*
 * Quantization parameters, named after BaseQuantizeConfig (AutoGPTQ examples
 * walkthrough, section 1.4; OLMo AutoGPTQ quick-start, section 三):
 *   bits          2, 3, 4 or 8
 *   group_size    -1 (one group per output row) or > 0 input columns per group
 *   damp_percent  in (0, 1): H += damp_percent * mean(diag H) * I
 *   desc_act      nonzero: sweep columns by descending diag(H) (act-order)
 *   static_groups nonzero: every group's scale/zero comes from the original
 *                 weights before the sweep; zero: a group's parameters are
 *                 taken from the current (compensated) weights when the sweep
 *                 reaches the group's first column
 *   sym           nonzero: symmetric range [-max|w|, max|w|], zero = 2^(bits-1)
 *   block_size    lazy-batch width; must be 128 (chapter 5, section 5.1.8)
 */
typedef struct {
  int32_t bits;
  int32_t group_size;
  float damp_percent;
  int32_t desc_act;
  int32_t static_groups;
  int32_t sym;
  int32_t block_size;
} gptq_config;

/* Host-only check of the rules above plus the solve's own constraint that a
 * group either divides the 128-column block or is a multiple of it (so the
 * lazy batches reproduce the plain column-by-column sweep).  Returns GPTQ_OK or
 * GPTQ_ERR_INVALID_ARG. */
gptq_status gptq_config_validate(const gptq_config* cfg);

/* Human-readable name of a status code (static storage); any int32 value is
 * accepted ("unknown status" for values outside gptq_status). */
const char* gptq_status_string(int32_t status);

/*
 * S += X^T X  (chapter 5, section 5.1.7: the layer Hessian is X X^T up to a
 * constant, estimated from calibration activations).
 *   S        [d_in, d_in] fp32, full symmetric storage, read-modify-write;
 *            zero it before the first chunk of a layer.
 *   X        [n_tokens, ldx] bf16 (GPTQ_BF16) or fp32 (GPTQ_F32); the first
 *            d_in entries of each row are used.  Needs 16-byte alignment and
 *            ldx a multiple of 8 (bf16) or 4 (fp32).
 *   n_tokens >= 0; 0 leaves S unchanged.
 * Products are formed exactly (bf16) or in fp32 and summed in fp32.  The sum
 * is deterministic: a fixed token split and a fixed reduction order.  fp32 X
 * with n_tokens * d_in^2 >= 4e9 and d_in <= 8192 runs on the bf16 matrix
 * cores: each value is split exactly into three bf16 parts (x = hi + mid +
 * lo), and S takes the part products above 2^-24 of the total (hi hi, hi mid,
 * mid hi, hi lo, lo hi, mid mid), each formed exactly and summed in fp32, so
 * the result keeps fp32-product accuracy (every entry below the diagonal is
 * written as a copy of its mirror); smaller calls use the fp32 matrix cores.
 * The workspace size
 * depends on d_in, n_tokens and the dtype (the fp32 path on the bf16 matrix
 * cores also holds the bf16 parts of up to 512 MiB of X at a time).
 */
size_t gptq_hessian_workspace_size(int64_t d_in, int64_t n_tokens, int32_t xt);
gptq_status gptq_hessian_accumulate(float* S, int64_t d_in, const void* X, int32_t xt,
                                    int64_t n_tokens, int64_t ldx, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * From the accumulated S of n_total tokens:
 *   H = (2 / n_total) S                  written back into S_to_H (kept for checks)
 *   lambda = damp_percent * mean(diag H), H_d = H + lambda I
 *                                        (chapter 5, section 5.1.8, damping)
 *   perm: desc_act ? stable sort of columns by descending diag(H) (ties: lower
 *         index first) : identity.  perm[i] = original column swept at position i.
 *   U = upper-triangular factor with (H_d[perm][:, perm])^-1 = U^T U
 *       (chapter 5, section 5.1.8: "Cholesky(inverse(H))"), [d_in, d_in] fp32,
 *       zeros below the diagonal.
 *   info_dev (device int32): 0 on success; -1 when diag(H) holds a NaN or an
 *       infinity (non-finite calibration inputs; perm is then still a
 *       permutation, NaN channels last, and U is undefined); k > 0 when the
 *       damped Hessian is not positive definite (an all-zero S, for one, gives
 *       lambda = 0 and fails at once, k = d_in).  The factorization runs from the last sweep
 *       position backwards and stops at its first failed pivot, so k - 1 is
 *       the LARGEST sweep position p for which the trailing block
 *       H_d[perm][:, perm][p:, p:] is not positive definite (as computed in
 *       fp32); every trailing block past p is.  U is then undefined.  Read it
 *       after synchronising.
 * n_total must be > 0.
 * Arithmetic: fp32 throughout.  The factorization's large products run on the
 * bf16 matrix cores with each fp32 operand split exactly into three bf16
 * parts (six part products, summed in fp32): the accuracy of an fp32 product,
 * not its bit pattern.  U is deterministic for a given S and cfg.
 */
size_t gptq_prepare_workspace_size(int64_t d_in);
gptq_status gptq_prepare_hinv(float* S_to_H, int64_t d_in, int64_t n_total, const gptq_config* cfg,
                              float* U, int32_t* perm, int32_t* info_dev, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * The GPTQ column sweep (chapter 5, section 5.1.8, the implementation-level
 * pseudocode), in sweep order perm, over lazy blocks of 128 columns:
 *   per column i: q = clamp(rint(w / s) + z, 0, 2^bits - 1), w_hat = s (q - z),
 *   err = (w - w_hat) / U[i, i], later columns of the block -= err * U[i, :];
 *   after each block the remaining columns -= Err_block @ U[block, rest].
 *   W        [d_out, d_in] fp32 or bf16 (not modified)
 *   U, perm  from gptq_prepare_hinv
 *   codes    [d_out, d_in] uint8, ORIGINAL column order
 *   scales   [n_groups, d_out] fp32, zeros [n_groups, d_out] int32, with
 *            n_groups = ceil(d_in / group_size), or 1 for group_size -1
 *   g_idx    [d_in] int32: group of each original column
 *   Q_or_null        optional [d_out, d_in] fp32 dequantized weights, original order
 *   row_loss_or_null optional [d_out] fp32: sum of err^2 over the row, which
 *                    equals (w - w_hat) H_d (w - w_hat)^T
 * Requires d_in % (32 / bits) == 0 (d_in % 32 == 0 for 3 bits).
 * The products that carry errors past each group of 1024 columns run as
 * three-part bf16 products (fp32 accuracy, see gptq_prepare_hinv); the rest in
 * fp32.  Outputs are deterministic for given inputs.
 * gptq_workspace_size depends on cfg (its group layout picks the launch
 * plan's buffers); it returns 0 for an invalid cfg or size.
 */
size_t gptq_workspace_size(int64_t d_out, int64_t d_in, const gptq_config* cfg);
gptq_status gptq_quantize_layer(const void* W, int32_t wt, int64_t d_out, int64_t d_in,
                                const float* U, const int32_t* perm, const gptq_config* cfg,
                                uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx,
                                float* Q_or_null, float* row_loss_or_null, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * qweight[w, n] holds bits [32 w, 32 w + 32) of output row n's code stream,
 * in which code (n, j) occupies bits [bits * j, bits * j + bits) (least
 * significant first; 3-bit codes straddle words).  qweight is
 * [d_in * bits / 32, d_out] int32 (the AutoGPTQ examples walkthrough names
 * the packed tensor qweight; the practitioner blog, section 3.3, gives the
 * density: 128 4-bit codes fill 64 bytes).  Codes must lie in [0, 2^bits).
 * Requires d_in % (32 / bits) == 0 (d_in % 32 == 0 for 3 bits).
 */
gptq_status gptq_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits,
                      int32_t* qweight, void* stream);

/*
 * y = x W^T with W dequantized on the fly: W[n, k] = scales[g, n] *
 * (code(n, k) - zeros[g, n]), g = g_idx[k] (chapter 5, section 5.1.10: a group
 * shares one scale and zero point; the pages' inference kernels read the packed
 * codes and dequantize inside the product).  Summed in fp32 in a fixed order
 * (deterministic).  32 consecutive k of one group are summed as
 * s (sum x q - z sum x), so the rounding error is bounded by
 * (d_in + 64) 2^-24 sum_k |x_k| s (q_k + z); with bf16 x and 4-bit codes the
 * codes enter as 16 + q against 16 + z (v_dot2 for 1-2 tokens, bf16 MFMA for
 * 3 or more), so there the bound has q_k + z + 32.  bf16 x with 3 or more
 * tokens runs on bf16 MFMA with the integer codes as the exact operand; 32 k
 * spread over several groups (act-order) use s (q - z) split into two bf16
 * parts there, so those products carry a relative error of about 2^-16.
 *   x        [m, d_in] bf16 or fp32, row-major, m >= 1 (any count; passes of 16 rows)
 *   qweight  [d_in * bits / 32, d_out] int32 as written by gptq_pack
 *   scales   [n_groups, d_out] fp32, zeros [n_groups, d_out] int32, g_idx [d_in]
 *            int32 as written by gptq_quantize_layer; every g_idx entry must lie
 *            in [0, n_groups) and every zero point in [0, 2^bits) (not checked
 *            on the device)
 *   y        [m, d_out] fp32 (overwritten)
 *   ws       device workspace of gptq_dequant_workspace_size(m, d_in, d_out)
 *            bytes, 256-byte aligned (partial sums of K slices); may be null
 *            when that size is 0
 * Requires d_in % 32 == 0, and qweight and scales each under 2^31 bytes
 * (d_in * d_out * bits / 8 and n_groups * d_out * 4).  INVALID_ARG on bad
 * sizes, bits or null pointers; WORKSPACE when ws is too small or misaligned.
 */
size_t gptq_dequant_workspace_size(int64_t m, int64_t d_in, int64_t d_out);
gptq_status gptq_dequant_matmul(const void* x, int32_t xt, int64_t m, int64_t d_in,
                                const int32_t* qweight, const float* scales, const int32_t* zeros,
                                const int32_t* g_idx, int32_t bits, int64_t d_out, int32_t n_groups,
                                float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * gptq_dequant_matmul for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same y, bit for bit, with the partial
 * sums of the K slices in a buffer the library owns instead of a caller
 * workspace.  The buffer is a fixed device array of gptq_dequant_scratch_bytes()
 * bytes (16 MiB) per GPU, held until the process ends; its device address is
 * looked up once per device, on that device's first call.  The call allocates
 * nothing (no hipMalloc, no library allocation).
 *   Arguments as for gptq_dequant_matmul, without ws / ws_bytes.
 *   gptq_dequant_noalloc_need(m, xt, d_in, bits, d_out) gives the scratch
 *   bytes a call needs (at most 14.7 MB for every layer shape up to
 *   28672 x 8192 with bf16 x at any m, or fp32 x at up to 8 tokens); a call
 *   needing more than the buffer returns GPTQ_ERR_TOO_LARGE and enqueues
 *   nothing.  The buffer needs no clearing: each call writes every partial
 *   sum it reads.
 *   Every call on one GPU shares the buffer: calls that may overlap in time
 *   on one GPU (different streams, or host threads) race and must be
 *   serialised by the caller.
 */
size_t gptq_dequant_scratch_bytes(void);
size_t gptq_dequant_noalloc_need(int64_t m, int32_t xt, int64_t d_in, int32_t bits, int64_t d_out);
gptq_status gptq_dequant_matmul_noalloc(const void* x, int32_t xt, int64_t m, int64_t d_in,
                                        const int32_t* qweight, const float* scales, const int32_t* zeros,
                                        const int32_t* g_idx, int32_t bits, int64_t d_out, int32_t n_groups,
                                        float* y, void* stream);

/*
 * Group order for the dequantizing product of an act-order layer.  With
 * desc_act (the AutoGPTQ examples walkthrough, section 1.4) g_idx assigns the
 * input channels to groups in the order the columns were quantized, so 32
 * consecutive channels usually span several groups and the product reads a
 * scale and zero point per code.  This call sorts the channels by group,
 * stably (order[j] = the original channel at sorted position j; channels of
 * one group keep increasing k), repacks the codes in that order and writes
 * g_idx in that order (non-decreasing).  y = x W^T is a sum over k, so
 * gptq_dequant_matmul_ordered on these outputs gives the product of the
 * original layer (chapter 5, section 5.1.10) with its terms in another order.
 * A one-time step (when a layer is loaded): d_in^2 comparisons.
 *   qweight, g_idx   as for gptq_dequant_matmul (every g_idx entry in
 *                    [0, n_groups); not checked on the device)
 *   qweight_out      [d_in * bits / 32, d_out] int32; must not overlap qweight
 *   g_idx_out        [d_in] int32, order [d_in] int32 (a permutation of 0..d_in-1)
 * Requires d_in % 32 == 0 and qweight under 2^31 bytes.  INVALID_ARG on bad
 * sizes, bits or null pointers.
 */
gptq_status gptq_dequant_order(const int32_t* qweight, const int32_t* g_idx, int32_t bits, int64_t d_in,
                               int64_t d_out, int32_t* qweight_out, int32_t* g_idx_out, int32_t* order,
                               void* stream);

/*
 * gptq_dequant_matmul on a layer put in group order by gptq_dequant_order:
 * x's channels are gathered in that order into the workspace, then the
 * product runs on the reordered codes (same y as gptq_dequant_matmul on the
 * original tensors, summed in the sorted channel order, same error bound).
 *   x        [m, d_in] bf16 or fp32 in the ORIGINAL channel order
 *   qweight, g_idx, order   the outputs of gptq_dequant_order
 *   scales, zeros           the layer's, unchanged ([n_groups, d_out])
 *   ws       device workspace of gptq_dequant_ordered_workspace_size(m, d_in, d_out)
 *            bytes, 256-byte aligned (the gathered x, then the partial sums)
 * Other arguments, requirements and errors as for gptq_dequant_matmul.
 */
size_t gptq_dequant_ordered_workspace_size(int64_t m, int64_t d_in, int64_t d_out);
gptq_status gptq_dequant_matmul_ordered(const void* x, int32_t xt, int64_t m, int64_t d_in,
                                        const int32_t* qweight, const float* scales, const int32_t* zeros,
                                        const int32_t* g_idx, const int32_t* order, int32_t bits, int64_t d_out,
                                        int32_t n_groups, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Per-phase launch timing, a measurement aid (not part of the solve; the pages
 * fix nothing here).  gptq_phase_timing(1) clears the record and switches it
 * on: from then on every launch of the calls above records a HIP event just
 * before and just after itself on its stream, and is counted under its phase
 * (gptq_phase_name: hessian_partial, hessian_reduce, prepare_elementwise,
 * cholesky_panel, cholesky_update, triangular_inverse, quantize_elementwise,
 * sweep, trailing_update, pack).  gptq_phase_timing(0) switches it off (the
 * default; a launch site then costs one atomic load).  gptq_phase_read waits
 * for the recorded events and writes, for phases 0 .. n-1, the summed event
 * time of their launches (ms) and the launch count.  Host-global state: not
 * for calls that run concurrently on several host threads while switched on.
 */
gptq_status gptq_phase_timing(int32_t enable);
int32_t gptq_phase_count(void);
const char* gptq_phase_name(int32_t phase);
gptq_status gptq_phase_read(float* ms, int32_t* launches, int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H */
