/*
 * mxattn.h -- C ABI of the MXFP4 attention library (libmxattn.so) for AMD
 * MI355X (gfx950).
 *
 * Method: "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
 * Quantization for MXFP4 Attention" (arXiv 2607.24377), abstract.  The
 * abstract defines the pieces this library computes:
 *   - MXFP4 quantization with power-of-two block scales, in two modes: OCP
 *     MXFP4 (the baseline it compares against) and Universal Optimal Scaling
 *     (UOS, the fixed data-free boundary Qmax = 7.25);
 *   - attention whose Q.K^T and P.V products run on MXFP4 operands;
 *   - Pre-Normalization Quantization (PNQ): the unnormalized softmax
 *     exponentials are quantized before they are summed into the row sum, so
 *     the row sum and P.V use the same quantized values.
 *
 * Number format (the abstract does not fix it; this library reads MXFP4 as
 * OCP MX does): blocks of 32 elements, each element an E2M1 code (4 bits,
 * bit 3 = sign, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), each block one E8M0
 * scale byte s meaning 2^(s-127).  Two codes per byte: element 2i of a block
 * in bits 3:0 of byte i, element 2i+1 in bits 7:4.  Encoding rounds to the
 * nearest magnitude, ties to the even code, saturating at 6; the sign bit of
 * the input is kept, so a negative value that rounds to zero gives code 0x8.
 * Block exponent e (clamped to [-127, 127], an all-zero block gives -127):
 *   MXQ_MODE_OCP: e = floor(log2(amax)) - 2
 *   MXQ_MODE_UOS: e = the smallest integer with amax <= 7.25 * 2^e
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory) owned
 *     by the caller, 16-byte aligned; the library never allocates or frees
 *     device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call except mxq_dump only enqueues work on `stream` and returns
 *     without waiting for it.
 *   - Return value: MXQ_OK (0) or a negative mxq_status.  All argument checks
 *     run on the host before anything is enqueued, so a rejected call has no
 *     effect; a failed launch is reported as MXQ_ERR_HIP.
 *   - Inputs must be finite bf16 values (non-finite input is a precondition
 *     violation; the results are then unspecified).  Attention scores and
 *     GEMM outputs are accumulated in fp32, so they must also fit fp32: a
 *     product of the dequantized operands that overflows fp32 is outside the
 *     supported range.
 *   - The library keeps no global state apart from mxattn_fwd_noalloc's
 *     device array (see there); every other call may run concurrently with
 *     others on different streams as long as they do not write the same
 *     buffers.
 */
#ifndef MXATTN_H
#define MXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MXQ_MODE_OCP = 0, MXQ_MODE_UOS = 1 } mxq_mode;

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad mode or axis, misaligned */
    MXQ_ERR_UNSUPPORTED = -2, /* valid request this build does not implement (e.g. d) */
    MXQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    MXQ_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    MXQ_ERR_IO = -5           /* mxq_dump could not write its file */
} mxq_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *mxq_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int mxattn_version(void);

/*
 * mxq_quantize -- MXFP4 quantization of a bf16 tensor (MXAttention abstract:
 * OCP MXFP4 baseline and UOS).
 *
 * x_bf16: bf16 values viewed as [batch][rows][cols], contiguous.
 * axis:   1 -> blocks of 32 run along cols (the contiguous axis);
 *         0 -> blocks of 32 run along rows (one column at a time).
 * Output (canonical, block-axis-major), nb = number of 32-blocks per vector:
 *   axis 1: codes [batch][rows][nb*16] bytes, scales [batch][rows][nb], nb = ceil(cols/32)
 *   axis 0: codes [batch][cols][nb*16] bytes, scales [batch][cols][nb], nb = ceil(rows/32)
 * A partial last block is zero-padded (padding codes are 0; the scale comes
 * from the valid elements only).  Empty tensors (any size 0) are a no-op.
 * Errors: MXQ_ERR_INVALID_ARG for a null pointer with a non-empty tensor,
 * negative sizes, axis not 0/1, mode not OCP/UOS, or a pointer that is not
 * 16-byte aligned (x and codes; scales may have any alignment).
 */
int mxq_quantize(const void *x_bf16, int64_t batch, int64_t rows, int64_t cols, int axis,
                 int mode, uint8_t *codes, uint8_t *scales, void *stream);

/*
 * mxq_quantize_strided -- mxq_quantize of a strided [B][H][rows][cols] view
 * with contiguous columns: element (b, h, r, c) at x + b*strides[0] +
 * h*strides[1] + r*strides[2] + c (elements; strides a host array of 3).
 * Output: the canonical layout of mxq_quantize with batch = B*H, bit-identical
 * to quantizing a dense copy.  Requires cols % 32 == 0, strides non-negative
 * multiples of 8, x and codes 16-byte aligned, B*H <= 65535.
 * Errors: MXQ_ERR_INVALID_ARG, MXQ_ERR_UNSUPPORTED, MXQ_ERR_HIP.
 */
int mxq_quantize_strided(const void *x_bf16, int64_t B, int64_t H, int64_t rows, int64_t cols,
                         const int64_t *strides, int axis, int mode, uint8_t *codes, uint8_t *scales,
                         void *stream);

/*
 * mxattn_kv_tile -- number of keys per key tile of the attention kernel for
 * head dimension d (0 if d is unsupported).  The running row maximum is
 * updated once per key tile, in ascending key order, and the quantized
 * exponentials are formed against that running maximum; the key tile is
 * therefore part of the definition of the result (the abstract only speaks of
 * the online softmax; this is the flash-attention reading).
 */
int mxattn_kv_tile(int64_t d);

/* Bytes of device workspace mxattn_fwd needs for these sizes (0 on bad sizes). */
size_t mxattn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * mxattn_fwd -- non-causal MXFP4 attention forward (MXAttention abstract:
 * MXFP4 Q.K^T, online softmax with PNQ, MXFP4 P.V).
 *
 * q, k, v, o: bf16 [B][H][N][d], contiguous.  d in {64, 128}; N >= 1.
 * mode: block-scale rule for Q, K, V and for the softmax exponentials.
 * pnq:  1 -> the row sum adds the quantized exponentials (PNQ);
 *       0 -> it adds the unquantized fp32 exponentials (P.V still uses the
 *            quantized ones; this is the normalization error PNQ removes).
 * softmax_scale: multiplies Q.K^T; <= 0 selects 1/sqrt(d).
 * Steps on `stream`: quantize K along d and V along N into the workspace
 * (mxq_quantize layouts with batch = B*H: K axis 1 with rows = N, cols = d;
 * V axis 0 with rows = N, cols = d), then one fused kernel that quantizes Q
 * along d itself (same rule and codes as mxq_quantize) and attends.  For
 * every query row and key tile of mxattn_kv_tile(d) keys: S = Q_q K_q^T
 * (fp32), times softmax_scale; running max m; p = exp(s - m) in fp32;
 * p quantized in 32-key blocks aligned to the key index (scale rule = mode);
 * l = alpha*l + sum(p_q or p); O = alpha*O + p_q V_q; finally O/l rounded to
 * bf16 (round to nearest even).
 * workspace: device memory of at least mxattn_workspace_bytes(B, H, N, d).
 * Errors: MXQ_ERR_INVALID_ARG (null or misaligned pointer, B/H < 1, N < 1,
 * bad mode or pnq), MXQ_ERR_UNSUPPORTED (d not 64/128, or B*H*N*d too large),
 * MXQ_ERR_WORKSPACE, MXQ_ERR_HIP.
 */
int mxattn_fwd(const void *q, const void *k, const void *v, int64_t B, int64_t H, int64_t N,
               int64_t d, int mode, int pnq, float softmax_scale, void *o, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * mxattn_fwd_noalloc -- mxattn_fwd without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The quantized K and V go
 * to a device array inside the library (mxattn_noalloc_max_bytes() = 256 MiB,
 * one copy per GPU, held until the process ends) instead of a workspace; the
 * call allocates nothing.  Arguments, kernels and results are those of
 * mxattn_fwd (bit-identical).  The array's address is looked up on the first
 * call on each device, with the caller's current device, which must be the
 * device of `stream` and of the tensors.  Every call on one GPU uses that
 * GPU's one array: calls that overlap in time on one GPU race, so callers
 * order them (one stream, or synchronization between streams).
 * Errors as mxattn_fwd; MXQ_ERR_WORKSPACE when mxattn_workspace_bytes(B, H,
 * N, d) exceeds mxattn_noalloc_max_bytes().
 */
int mxattn_fwd_noalloc(const void *q, const void *k, const void *v, int64_t B, int64_t H, int64_t N,
                       int64_t d, int mode, int pnq, float softmax_scale, void *o, void *stream);

/* Size in bytes of mxattn_fwd_noalloc's device array (its largest workspace). */
size_t mxattn_noalloc_max_bytes(void);

/*
 * mxattn_fwd_quantized -- the fused kernel alone, on operands already in the
 * canonical layouts of mxq_quantize (batch = B*H):
 *   qc, kc: [B*H][N][d/2], qs, ks: [B*H][N][d/32]   (axis 1, rows = N, cols = d)
 *   vc: [B*H][d][ceil(N/32)*16], vs: [B*H][d][ceil(N/32)]   (axis 0)
 * mode is the scale rule used for the softmax exponentials.  Other arguments
 * and errors as mxattn_fwd (no workspace).
 */
int mxattn_fwd_quantized(const uint8_t *qc, const uint8_t *qs, const uint8_t *kc, const uint8_t *ks,
                         const uint8_t *vc, const uint8_t *vs, int64_t B, int64_t H, int64_t N,
                         int64_t d, int mode, int pnq, float softmax_scale, void *o, void *stream);

/*
 * mxattn_fwd_kv_quantized -- the fused kernel of mxattn_fwd alone: bf16 Q as
 * in mxattn_fwd (quantized inside the kernel), K and V already quantized in
 * the layouts of mxattn_fwd_quantized (for callers that keep K_q and V_q, and
 * for timing the kernel by itself).  The result is bit-identical to
 * mxattn_fwd_quantized on mxq_quantize(Q), and to mxattn_fwd.  Other
 * arguments and errors as mxattn_fwd (no workspace).
 */
int mxattn_fwd_kv_quantized(const void *q, const uint8_t *kc, const uint8_t *ks, const uint8_t *vc,
                            const uint8_t *vs, int64_t B, int64_t H, int64_t N, int64_t d, int mode,
                            int pnq, float softmax_scale, void *o, void *stream);

/*
 * mxattn_fwd_strided -- mxattn_fwd on strided views, for callers whose
 * tensors are not dense [B][H][N][d]: element (b, h, n, c) of X (Q, K, V or
 * O) sits at X + b*s[0] + h*s[1] + n*s[2] + c elements, with s = the
 * tensor's three strides (host arrays of 3 int64, in elements; d is
 * contiguous).  [B][N][H][d] (BNHD) is s = {N*H*d, d, H*d}; dense BHND is
 * {H*N*d, N*d, d}; slices of a packed [B][N][3][H][d] QKV tensor work as
 * they are.  Strides must be non-negative multiples of 8 (16-byte rows) and
 * O must not overlap Q, K or V.  The result is bit-identical to mxattn_fwd
 * on dense copies.  Workspace as mxattn_fwd (mxattn_workspace_bytes).
 * Errors as mxattn_fwd; MXQ_ERR_UNSUPPORTED also when B*H > 65535.
 */
int mxattn_fwd_strided(const void *q, const void *k, const void *v, void *o, int64_t B, int64_t H,
                       int64_t N, int64_t d, const int64_t *q_strides, const int64_t *k_strides,
                       const int64_t *v_strides, const int64_t *o_strides, int mode, int pnq,
                       float softmax_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mxattn_varlen_workspace_bytes -- bytes of device workspace mxattn_fwd_varlen
 * needs for `batch` sequences over T tokens (0 on bad sizes): K codes and
 * scales [H][T], V codes and scales [H][d][ceil(T/32) + batch blocks], and a
 * table of 4 (batch + 1) ints built from cu_seqlens.
 */
size_t mxattn_varlen_workspace_bytes(int64_t batch, int64_t T, int64_t H, int64_t d);

/*
 * mxattn_fwd_varlen -- mxattn_fwd over a batch of sequences of different
 * lengths packed along one token axis (the variable-length layout of DiT and
 * LLM pipelines).  Sequence s holds tokens [cu_seqlens[s], cu_seqlens[s+1]);
 * every sequence is its own non-causal attention problem, computed exactly
 * as mxattn_fwd would compute it alone (same K/V quantization along d and
 * along the sequence's own tokens, 32-token V blocks starting at the
 * sequence's first token, same key tiles), so the result is bit-identical to
 * one mxattn_fwd call per sequence.
 * q, k, v, o: bf16, element (t, h, c) of X at X + t*s_tok + h*s_head + c,
 *   with strides = {q_tok, q_head, k_tok, k_head, v_tok, v_head, o_tok,
 *   o_head} (host array of 8 int64, elements; non-negative multiples of 8),
 *   or strides = NULL for packed [T][H][d] (s_tok = H*d, s_head = d).
 * cu_seqlens: device array of batch + 1 int32 prefix offsets, 4-byte
 *   aligned, expected non-decreasing from 0 to T.  The kernels read it
 *   clamped to [0, T] and made non-decreasing, so a malformed array gives
 *   wrong results, never an access outside the tensors; tokens outside every
 *   sequence are not written.
 * batch >= 1, T >= 0 (T = 0 does nothing), H >= 1, d in {64, 128}.
 * workspace: at least mxattn_varlen_workspace_bytes(batch, T, H, d).
 * Other arguments as mxattn_fwd.
 * Errors: MXQ_ERR_INVALID_ARG (null or misaligned pointer, bad sizes, mode,
 * pnq or strides), MXQ_ERR_UNSUPPORTED (d, or batch > 2^20, T > 2^24,
 * H > 65535, or sizes past the 32-bit offsets of the kernels),
 * MXQ_ERR_WORKSPACE, MXQ_ERR_HIP.
 */
int mxattn_fwd_varlen(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens,
                      int64_t batch, int64_t T, int64_t H, int64_t d, const int64_t *strides, int mode,
                      int pnq, float softmax_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mxgemm_quantized -- Y = X W^T on MXFP4 operands (the MXAttention abstract's
 * UOS is data-free, so the same quantizer serves the linear layers around
 * attention).  X [M][K] and W [N][K] are quantized along K in the canonical
 * layout of mxq_quantize (batch = 1, axis 1): codes [rows][K/2], scales
 * [rows][K/32].  Products are exact, sums are fp32 (MFMA), and y receives
 * bf16 [M][N] rounded to nearest even.  Requires K % 128 == 0 and
 * N % 4 == 0; code pointers and y 16-byte aligned, scale pointers 4-byte
 * aligned.  All pointers are device memory owned by the caller.
 * Errors: MXQ_ERR_INVALID_ARG (null or misaligned pointer, M/N/K < 1),
 * MXQ_ERR_UNSUPPORTED (K or N not a supported multiple, sizes too large),
 * MXQ_ERR_HIP.
 */
int mxgemm_quantized(const uint8_t *xc, const uint8_t *xs, const uint8_t *wc, const uint8_t *ws,
                     int64_t M, int64_t N, int64_t K, void *y, void *stream);

/* Bytes of device workspace mxgemm needs for X [M][K] (0 on bad sizes). */
size_t mxgemm_workspace_bytes(int64_t M, int64_t K);

/*
 * mxgemm -- the same with bf16 X [M][K]: X is quantized along K with `mode`
 * into the workspace (mxq_quantize), then multiplied by the pre-quantized W
 * (weights are quantized once, with mxq_quantize on W [N][K], axis 1).  Other
 * arguments and errors as mxgemm_quantized, plus MXQ_ERR_WORKSPACE.
 */
int mxgemm(const void *x, const uint8_t *wc, const uint8_t *ws, int64_t M, int64_t N, int64_t K,
           int mode, void *y, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mxqkv_proj_quantized -- the QKV projection of one sequence of T tokens,
 * Y = X W^T (as mxgemm_quantized, with N = 3*H*d), written straight into the
 * operand formats of the attention kernel (the MXAttention abstract notes
 * that quantization fused into the attention pipeline costs little): Y's
 * columns are [Q | K | V], each H*d wide, head-major inside each part.
 *   q:  bf16 [H][T][d]                       (Q, for mxattn_fwd_kv_quantized)
 *   kc: [H][T][d/2],  ks: [H][T][d/32]       (K quantized along d)
 *   vc: [H][d][ceil(T/32)*16], vs: [H][d][ceil(T/32)]   (V quantized along T)
 * K and V are rounded to bf16 (nearest even) and then quantized with `mode`,
 * exactly as mxq_quantize would quantize that bf16 K and V, so the codes and
 * scales equal those of mxgemm_quantized followed by mxq_quantize of the K
 * and V parts; the last V block of each channel is zero-padded.  These are
 * the layouts mxattn_fwd_kv_quantized takes with B = 1, N = T.
 * xc, xs, wc, ws: X [T][C] and W [3*H*d][C] quantized along C (canonical
 * layout).  Requires C % 128 == 0, d in {64, 128}; code pointers and q 16-byte
 * aligned, xs and ws 4-byte aligned; all pointers device memory owned by the
 * caller.
 * Errors: MXQ_ERR_INVALID_ARG (null or misaligned pointer, T/C/H < 1, mode),
 * MXQ_ERR_UNSUPPORTED (d, C, or sizes past the GEMM's or the attention's
 * limits), MXQ_ERR_HIP.
 */
int mxqkv_proj_quantized(const uint8_t *xc, const uint8_t *xs, const uint8_t *wc, const uint8_t *ws,
                         int64_t T, int64_t C, int64_t H, int64_t d, int mode, void *q, uint8_t *kc,
                         uint8_t *ks, uint8_t *vc, uint8_t *vs, void *stream);

/*
 * mxqkv_proj -- mxqkv_proj_quantized from bf16 X [T][C]: X is quantized with
 * `mode` into the workspace first (mxgemm_workspace_bytes(T, C) bytes), W as
 * for mxqkv_proj_quantized.  Errors as mxqkv_proj_quantized, plus
 * MXQ_ERR_WORKSPACE.
 */
int mxqkv_proj(const void *x, const uint8_t *wc, const uint8_t *ws, int64_t T, int64_t C, int64_t H,
               int64_t d, int mode, void *q, uint8_t *kc, uint8_t *ks, uint8_t *vc, uint8_t *vs,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * mxq_dump -- write quantized data in the reference format "MXQ1": a 256-byte
 * header of ASCII JSON padded with spaces and ending in '\n'
 *   {"magic":"MXQ1","version":1,"mode":"ocp"|"uos","axis":A,"batch":B,
 *    "nvec":V,"L":L,"block":32,"elem":"e2m1","scale":"e8m0","nibble":"lo-first"}
 * followed by batch*nvec*ceil(L/32)*16 code bytes and batch*nvec*ceil(L/32)
 * scale bytes in the canonical layout (nvec = vectors per batch entry, L =
 * their length: rows/cols for axis 1, cols/rows for axis 0).
 * codes/scales may be device pointers (copied on `stream`, which is then
 * synchronized) or host pointers (read directly), both of the same kind.
 * Synchronous.
 * Errors: MXQ_ERR_INVALID_ARG (also for one device and one host pointer),
 * MXQ_ERR_HIP (copy failed), MXQ_ERR_IO.
 */
int mxq_dump(const char *path, const uint8_t *codes, const uint8_t *scales, int64_t batch,
             int64_t nvec, int64_t L, int axis, int mode, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXATTN_H */
