/*
 * fa.h — C ABI of the MI355X (gfx950) FlashAttention-2 forward library, libfa.so.
 *
 * What is computed. For every (batch or sequence, head):
 *   O = softmax(softmax_scale * Q K^T) V,   L_i = m_i + ln l_i,
 * with m_i the maximum of row i of the scaled (and masked) scores and
 * l_i = sum_j exp(S_ij - m_i). The N x N score matrix never reaches memory:
 * the forward works on query tiles and streams key/value tiles through an
 * online-softmax update (running max m, running sum l), normalises O by l at
 * the end and writes the log-sum-exp L per row.
 *   Definition: "FlashAttention/zh" (marovi.ai wiki), section
 *     為何標準注意力運行緩慢 (why standard attention is slow).
 *   Online softmax and the tiled forward with L = m + log l: same page,
 *     sections 在線 softmax 技巧 and FlashAttention 算法.
 *   FlashAttention-2 work split (outer loop over query blocks, inner loop over
 *     key/value blocks): same page, section 變體與後續版本.
 *   Half-precision only, device tensors only, no attention weights returned,
 *     packed variable-length batches described by cumulative lengths plus a
 *     maximum length: "InternViT-6B-448px-V1-2 如何加速注意力计算", section
 *     FlashAttention 封装类三条执行路径 (硬性约束 and 变长路径).
 * "log" in L is the natural logarithm.
 *
 * Conventions shared by every entry point.
 *   - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller, 16-byte aligned, densely packed (row-major, no strides)
 *     except in the *_strided entry points.
 *     The library keeps no pointer after it returns and allocates no memory.
 *   - Q, K, V and O are bfloat16 (passed as void*), or fp16 where the
 *     *_strided entry points say so; L is float32.
 *   - Head dimension d must be 32, 64, 128 or 256 (every entry point and
 *     mask, the FP8 path aside).
 *   - softmax_scale may be any finite value, 0 and negative values included
 *     (callers normally pass 1/sqrt(d)); L is computed on the scaled scores.
 *   - causal = 1 applies the lower-triangular mask of self-attention (query i
 *     sees keys j <= i) and needs as many queries as keys; causal = 0 is
 *     unmasked attention.
 *   - stream is a hipStream_t (NULL = the null stream). The call only enqueues
 *     work: it returns before the GPU has finished, and a fault inside the
 *     kernel surfaces at the caller's next synchronisation.
 *   - Errors: arguments are checked on the host before any HIP call; a bad
 *     argument returns FA_ERR_INVALID_ARGUMENT, an unsupported shape or device
 *     FA_ERR_UNSUPPORTED, a failed HIP call FA_ERR_HIP. Nothing is enqueued
 *     when a check fails. fa_last_error() gives a message for the calling
 *     thread's most recent failure.
 *   - Thread-safe. Outputs may not alias inputs.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_HIP = 3
} fa_status;

/*
 * Equal-length batch.
 *   q   : (B, Nq, H, d) bfloat16
 *   k, v: (B, Nk, H, d) bfloat16
 *   o   : (B, Nq, H, d) bfloat16, written
 *   lse : (B, H, Nq)    float32,  written (natural-log log-sum-exp per row)
 * Requires B, Nq, Nk, H >= 1; causal requires Nq == Nk. Every element of o
 * and lse is written; nothing else is touched.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                 float softmax_scale, int32_t causal, void* stream);

/*
 * Packed variable-length batch (no padding).
 *   q, k, v, o : (total, H, d) bfloat16; o written
 *   lse        : (H, total) float32, written
 *   cu_seqlens : DEVICE int32[num_seqs + 1]; sequence s occupies rows
 *                [cu_seqlens[s], cu_seqlens[s+1]) of q, k, v and o and attends
 *                only to its own rows. The contents must satisfy
 *                cu_seqlens[0] = 0, non-decreasing, cu_seqlens[num_seqs] = total
 *                and every length <= max_seqlen; they live on the device and
 *                are not checked by the library (rows outside every sequence
 *                are not written; lengths above max_seqlen are not processed
 *                past max_seqlen).
 * Requires num_seqs >= 1, H >= 1, total >= 0, max_seqlen >= 0 (0 or total = 0
 * enqueues nothing). Queries and keys share the boundaries, so causal masking
 * is per sequence.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                        int32_t total, int32_t H, int32_t d, float softmax_scale,
                        int32_t causal, void* stream);

/*
 * Banded (sliding-window) mask, equal-length batch. Same tensors, layouts and
 * requirements as fa_fwd, with the causal flag replaced by a band: query i
 * sees key j iff
 *     i + (Nk - Nq) - window_left <= j <= i + (Nk - Nq) + window_right,
 * i.e. the band is centred on the query's position aligned so that the last
 * query meets the last key (for Nq == Nk, on the diagonal). window_left and
 * window_right are >= 0, or -1 for no bound on that side: (-1, 0) is causal
 * attention (also for Nq != Nk, aligned as above), (-1, -1) is unmasked.
 * Key tiles outside every row's band are neither loaded nor computed. A row
 * that sees no key gets o = 0 and lse = -inf (the log of an empty sum).
 *   Source: FlashAttention composes with banded masks, "FlashAttention/zh",
 *   section 變體與後續版本; each token attends a local window and window
 *   attention skips the key blocks outside it, "YOLOv12官版镜像集成Flash
 *   Attention v2，提速原理浅析", section 4.2 (dynamic sparse attention).
 * Errors: as fa_fwd; a window side below -1 is FA_ERR_INVALID_ARGUMENT;
 * Nq or Nk above 2^29 is FA_ERR_UNSUPPORTED.
 */
fa_status fa_fwd_band(const void* q, const void* k, const void* v, void* o, float* lse,
                      int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                      float softmax_scale, int32_t window_left, int32_t window_right,
                      void* stream);

/*
 * Banded mask, packed variable-length batch. Same tensors, layouts and
 * requirements as fa_fwd_varlen; within each sequence (queries and keys have
 * the same length, so the alignment offset is 0) query i sees key j iff
 * i - window_left <= j <= i + window_right, sides >= 0 or -1 as above.
 * Errors: as fa_fwd_varlen; a window side below -1 is
 * FA_ERR_INVALID_ARGUMENT; max_seqlen above 2^29 is FA_ERR_UNSUPPORTED.
 */
fa_status fa_fwd_varlen_band(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                             int32_t total, int32_t H, int32_t d, float softmax_scale,
                             int32_t window_left, int32_t window_right, void* stream);

/* Element type of q, k, v and o for the strided entry points. */
enum {
  FA_DTYPE_BF16 = 0,
  FA_DTYPE_F16 = 1
};

/*
 * Equal-length batch with any strides and either half-precision type; the
 * general form of fa_fwd and fa_fwd_band.
 *   q, o : (B, Nq, H, d) views; k, v: (B, Nk, H, d) views. Element (b, n, h, e)
 *          of tensor X sits at X + b*X_strides[0] + n*X_strides[1]
 *          + h*X_strides[2] + e (elements; d is contiguous). Any strides that
 *          are multiples of 8 (rows 16-byte aligned), with token strides up to
 *          2^24, are accepted: e.g. the packed (B, S, 3, H, d) QKV tensor passes
 *          as three views with token stride 3*H*d and head stride d, with no
 *          copy. Outputs must not overlap each other or the inputs.
 *   q_strides .. o_strides : HOST int64[3] each: batch, token, head strides.
 *   lse  : (B, H, Nq) float32, contiguous, written.
 *   dtype: FA_DTYPE_BF16 or FA_DTYPE_F16 for all of q, k, v and o (fp16
 *          attention runs on the fp16 matrix cores with fp32 accumulation and
 *          P rounded to fp16).
 *   causal / window_left / window_right: causal = 1 with both sides -1 is the
 *          causal mask (Nq == Nk); causal = 0 with both sides -1 is unmasked;
 *          causal = 0 with a side >= 0 is the band of fa_fwd_band.
 *   Source for the two element types and the packed QKV layout:
 *     "InternViT-6B-448px-V1-2 如何加速注意力计算", section
 *     FlashAttention 封装类三条执行路径 (fp16/bf16 inputs; the unmasked path
 *     passes a packed (B, S, 3, H, D) QKV tensor).
 * Errors: as fa_fwd and fa_fwd_band; a stride that is negative or not a
 * multiple of 8, a null stride array, an unknown dtype, or causal with a
 * window side other than -1 is FA_ERR_INVALID_ARGUMENT; a token stride
 * above 2^24 is FA_ERR_UNSUPPORTED.
 */
fa_status fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                         int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                         const int64_t* q_strides, const int64_t* k_strides,
                         const int64_t* v_strides, const int64_t* o_strides, int32_t dtype,
                         float softmax_scale, int32_t causal, int32_t window_left,
                         int32_t window_right, void* stream);

/*
 * Packed variable-length batch with any token and head strides and either
 * half-precision type; the general form of fa_fwd_varlen and
 * fa_fwd_varlen_band. Row r (packed token index), head h, element e of
 * tensor X sits at X + r*X_strides[0] + h*X_strides[1] + e; the stride
 * arrays are HOST int64[2] (token, head), with the rules of fa_fwd_strided.
 * cu_seqlens, max_seqlen, total and lse are as in fa_fwd_varlen; dtype and
 * the mask arguments as in fa_fwd_strided.
 */
fa_status fa_fwd_varlen_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int32_t* cu_seqlens, int32_t num_seqs, int32_t max_seqlen,
                                int32_t total, int32_t H, int32_t d, const int64_t* q_strides,
                                const int64_t* k_strides, const int64_t* v_strides,
                                const int64_t* o_strides, int32_t dtype, float softmax_scale,
                                int32_t causal, int32_t window_left, int32_t window_right,
                                void* stream);

/*
 * Padded batch with a key padding mask (self-attention): the result of
 * removing the padding positions, attending over the valid tokens of each
 * batch row and putting the result back in the padded shape, computed in
 * place without copies ("InternViT-6B-448px-V1-2 如何加速注意力计算", section
 * FlashAttention 封装类三条执行路径, 带掩码路径).
 *   q, k, v, o        : (B, S, H, d) dtype, densely packed; o written
 *   lse               : (B, H, S) float32, written
 *   key_padding_mask  : DEVICE uint8 (B, S); nonzero = valid token, 0 = padding
 *   dtype, causal     : as in fa_fwd_strided; causal runs over the order of
 *                       the valid tokens (query i sees valid keys j <= i)
 * Padding positions get o = 0 and lse = -inf (they take no part in the
 * attention). Tiles whose 64 keys are all valid take the unmasked path.
 * Errors: as fa_fwd_strided; a null mask is FA_ERR_INVALID_ARGUMENT.
 */
fa_status fa_fwd_padded(const void* q, const void* k, const void* v, void* o, float* lse,
                        const uint8_t* key_padding_mask, int32_t B, int32_t S, int32_t H,
                        int32_t d, int32_t dtype, float softmax_scale, int32_t causal,
                        void* stream);

/*
 * Backward pass, equal-length batch: the gradients of O with respect to Q, K
 * and V for an incoming gradient dO, with S and P recomputed from the saved
 * log-sum-exp instead of stored ("FlashAttention/zh" (marovi.ai wiki),
 * section 反向傳遞與重計算). With P_ij = exp(softmax_scale q_i.k_j - L_i):
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
 *     dQ = softmax_scale dS K,   dK = softmax_scale dS^T Q
 * (the chain rule through the definition; the page gives no formulas).
 *   q, o, dout, dq : (B, Nq, H, d), dtype; dq written
 *   k, v, dk, dv   : (B, Nk, H, d), dtype; dk, dv written
 *   lse            : (B, H, Nq) float32, the forward's L (natural log)
 *   delta          : (B, H, Nq) float32, caller-owned; written with D (it is
 *                    also the backward's scratch: the library allocates none)
 *   dtype          : FA_DTYPE_BF16 or FA_DTYPE_F16 for q, k, v, o, dout, dq,
 *                    dk, dv; P and dS enter the matrix cores in that type
 *   causal         : as in fa_fwd (Nq == Nk)
 *   d              : 32, 64, 128 or 256 ("FlashAttention/zh", section
 *                    局限性, puts the fused kernel's reach at head
 *                    dimensions up to about 256). At 256 the dK/dV pass runs two workgroups per
 *                    key tile, one per half of the head dimension, each
 *                    recomputing S and dP over the full d.
 * All tensors densely packed and 16-byte aligned; o and lse are those the
 * forward returned for the same q, k, v, scale and mask. Every element of dq,
 * dk, dv and delta is written.
 * Errors: as fa_fwd; an unknown dtype is FA_ERR_INVALID_ARGUMENT; H * d above
 * 2^24, or B * Nq * H (varlen: total * H) above 2^31 - 1, is
 * FA_ERR_UNSUPPORTED.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int32_t B,
                 int32_t Nq, int32_t Nk, int32_t H, int32_t d, int32_t dtype,
                 float softmax_scale, int32_t causal, void* stream);

/*
 * Backward pass, packed variable-length batch: tensors (total, H, d), lse
 * and delta (H, total), cu_seqlens / num_seqs / max_seqlen / total as in
 * fa_fwd_varlen; each sequence's gradients involve only its own rows.
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                        int32_t max_seqlen, int32_t total, int32_t H, int32_t d, int32_t dtype,
                        float softmax_scale, int32_t causal, void* stream);

/*
 * Decode: one query per (batch, head) against a KV cache, the step of token
 * generation. The scores are a matrix-vector product, so the cache is split
 * into chunks processed by separate workgroups, and the partial results
 * (O_s, L_s) are merged exactly through their log-sum-exps:
 * L = ln sum_s e^{L_s}, O = sum_s e^{L_s - L} O_s (the forward's L = m + log l,
 * "FlashAttention/zh" (marovi.ai wiki), section FlashAttention 算法).
 *   q, o      : (B, 1, H, d) dtype, densely packed; o written
 *   k, v      : (B, Nk, H, d) dtype, the cache, densely packed
 *   lse       : (B, H) float32, written (natural log)
 *   seqlens_k : DEVICE int32[B] or NULL; batch b attends to its first
 *               min(max(seqlens_k[b], 0), Nk) keys (NULL: all Nk). A batch
 *               with no key gets o = 0 and lse = -inf.
 *   workspace : DEVICE buffer of at least fa_decode_workspace_bytes(B, Nk, H,
 *               d) bytes, 16-byte aligned, owned by the caller (the partial
 *               results; the library allocates nothing). Calls that overlap on
 *               one workspace race.
 * Scores, softmax and P V are computed in fp32 (no 16-bit rounding of P).
 * Errors: as fa_fwd_strided; a null or too small workspace is
 * FA_ERR_INVALID_ARGUMENT; d must be 32, 64, 128 or 256.
 */
fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* seqlens_k, int32_t B, int32_t Nk, int32_t H, int32_t d,
                    int32_t dtype, float softmax_scale, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Workspace bytes fa_decode needs for these sizes (0 for sizes below 1). */
size_t fa_decode_workspace_bytes(int32_t B, int32_t Nk, int32_t H, int32_t d);

/*
 * FP8 forward on block-scaled operands ("FlashAttention/zh" (marovi.ai
 * wiki), section 變體與後續版本: the FP8 generation with block scaling; section
 * 局限性: low precision needs careful scaling). The block-scaled format is
 * OCP MX: 32 consecutive elements share one power-of-two scale stored as an
 * E8M0 byte (value 2^(byte - 127)); the elements are FP8 E4M3 ("fn": bias 7,
 * largest magnitude 448, subnormals down to 2^-9) bytes. A block's exponent
 * is floor(log2(max |x|)) - 8 clamped to [-127, 127] (an all-zero block gets
 * -127); elements are x / 2^exponent rounded to nearest even and saturated to
 * +-448. Head dimension d = 128 only.
 *
 * fa_fwd_mx8 computes O = softmax(softmax_scale Q K^T) V and L as fa_fwd does,
 * with Q, K and V the dequantised block-scaled operands:
 *   q, k  : (B, Nq or Nk, H, d) E4M3 bytes, densely packed, 16-byte aligned
 *   qe, ke: (B, Nq or Nk, H, d/32) E8M0 bytes (blocks along d), 4-byte aligned
 *   vt    : V transposed, (B, H, d, Np) E4M3 bytes, Np = fa_mx8_tokens_padded(Nk)
 *           (tokens padded with zeros to a multiple of 64)
 *   vte   : (B, H, Np/32, d) E8M0 bytes: for each block of 32 tokens, the d
 *           exponents of its rows of V^T
 *   o     : (B, Nq, H, d) bfloat16, written; lse: (B, H, Nq) float32, written
 *   softmax_scale: any finite value; causal: 0 or 1 (1 needs Nq == Nk).
 * Inside, P (at most 2^8 after the running offset) is rounded to E4M3 with a
 * scale of 1 before P V; row sums stay fp32.
 * Errors: d != 128 or sizes beyond the kernel's 32-bit tile offsets
 * (Nk * H * d > 2^30) are FA_ERR_UNSUPPORTED; otherwise as fa_fwd.
 */
fa_status fa_fwd_mx8(const uint8_t* q, const uint8_t* qe, const uint8_t* k, const uint8_t* ke,
                     const uint8_t* vt, const uint8_t* vte, void* o, float* lse, int32_t B,
                     int32_t Nq, int32_t Nk, int32_t H, int32_t d, float softmax_scale,
                     int32_t causal, void* stream);

/* Np, the padded token count of vt for N tokens (N rounded up to a multiple of
 * 64); -1 for N < 0 or too large. */
int32_t fa_mx8_tokens_padded(int32_t N);

/* Q or K (rows x d, 16-bit of dtype, densely packed, e.g. (B, N, H, d) with
 * rows = B N H) to the MX format above: xq (rows x d) E4M3 bytes and xe
 * (rows x d/32) E8M0 bytes, blocks along d. d must be 128. */
fa_status fa_mx8_quantize_qk(const void* x, int32_t dtype, int64_t rows, int32_t d, uint8_t* xq,
                             uint8_t* xe, void* stream);

/* V (B, N, H, d) 16-bit of dtype, densely packed, to vt (B, H, d, Np) and vte
 * (B, H, Np/32, d), blocks of 32 tokens, padding tokens zero. d must be 128. */
fa_status fa_mx8_quantize_v(const void* v, int32_t dtype, int32_t B, int32_t N, int32_t H,
                            int32_t d, uint8_t* vt, uint8_t* vte, void* stream);

/* Bytes of the scratch array fa_decode_noalloc holds on each GPU. */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * fa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation calls. Same arguments and results as
 * fa_decode minus the workspace; the partial results go to a scratch array
 * of FA_DECODE_NOALLOC_SCRATCH_BYTES (8 MiB) that the library's code object
 * reserves on each GPU it runs on, held until the process ends. The call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); its first call on a device looks the array's address up once.
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (each call overwrites every part it reads, so nothing needs
 * clearing): calls that overlap on one GPU (other streams, other threads)
 * race. Errors: as fa_decode; sizes whose partial results
 * (fa_decode_workspace_bytes) exceed the array are FA_ERR_UNSUPPORTED.
 */
fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* seqlens_k, int32_t B, int32_t Nk, int32_t H,
                            int32_t d, int32_t dtype, float softmax_scale, void* stream);

/*
 * Local window on a token map plus global anchor tokens (self-attention):
 * the detector's mix of local-window attention and a few global tokens
 * ("YOLOv12官版镜像集成Flash Attention v2，提速原理浅析", section 4.2, dynamic
 * sparse attention; the map of section 4.1). Tokens [0, n_global) are the
 * anchors; tokens n_global.. form a row-major map of map_w tokens per row
 * (token t at row (t - n_global) / map_w, column (t - n_global) % map_w; the
 * last row may be short). Query i sees key j iff
 *     i < n_global  or  j < n_global  or
 *     |row_i - row_j| <= win_rows and |col_i - col_j| <= win_cols,
 * and, when causal = 1, j <= i. So every query sees the anchors and an
 * anchor query sees every key; a 5 x 5 window is win_rows = win_cols = 2.
 * Only the anchor key tiles and the key tiles of the map rows in reach are
 * read; every row sees at least itself, so no row is empty.
 *   q, k, v, o  : (B, N, H, d) dtype, densely packed; o written
 *   lse         : (B, H, N) float32, written
 *   dtype       : FA_DTYPE_BF16 or FA_DTYPE_F16; d: 32, 64, 128 or 256
 *   n_global >= 0 (values above N mean every token is an anchor),
 *   map_w >= 1, win_rows >= 0, win_cols >= 0 (values beyond the map's
 *   extent mean no bound).
 * Errors: a negative pattern size or map_w < 1 is FA_ERR_INVALID_ARGUMENT;
 * N above 2^28 or H*d above 2^24 is FA_ERR_UNSUPPORTED; otherwise as fa_fwd.
 */
fa_status fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                       int32_t B, int32_t N, int32_t H, int32_t d, int32_t dtype,
                       float softmax_scale, int32_t causal, int32_t n_global, int32_t map_w,
                       int32_t win_rows, int32_t win_cols, void* stream);

/*
 * Backward of the banded forward (fa_fwd_band / fa_fwd_varlen_band): the
 * arguments of fa_bwd / fa_bwd_varlen with the causal flag replaced by the
 * window of the forward call (sides >= 0, or -1 for unbounded). Rows that
 * saw no key get zero gradients. Errors: as fa_bwd; a window side below -1
 * is FA_ERR_INVALID_ARGUMENT; Nq or Nk (max_seqlen) above 2^29 is
 * FA_ERR_UNSUPPORTED.
 */
fa_status fa_bwd_band(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float* delta, int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                      int32_t dtype, float softmax_scale, int32_t window_left,
                      int32_t window_right, void* stream);
fa_status fa_bwd_varlen_band(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                             int32_t max_seqlen, int32_t total, int32_t H, int32_t d,
                             int32_t dtype, float softmax_scale, int32_t window_left,
                             int32_t window_right, void* stream);

/*
 * Backward of the padded forward (fa_fwd_padded): tensors (B, S, H, d), lse and
 * delta (B, H, S), the same key_padding_mask (DEVICE uint8 (B, S), nonzero =
 * valid) and causal flag. The gradients are those of attention over the
 * valid tokens; padding positions get zero dq, dk, dv. Errors: as fa_bwd; a
 * null mask is FA_ERR_INVALID_ARGUMENT.
 */
fa_status fa_bwd_padded(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* delta, const uint8_t* key_padding_mask, int32_t B, int32_t S,
                        int32_t H, int32_t d, int32_t dtype, float softmax_scale, int32_t causal,
                        void* stream);

/*
 * Backward pass on strided views: the general form of fa_bwd and
 * fa_bwd_band, as fa_fwd_strided is of the forward, so that a model that
 * keeps Q, K and V in one packed (B, S, 3, H, d) tensor (the layout of the
 * unmasked path in "InternViT-6B-448px-V1-2 如何加速注意力计算", section
 * FlashAttention 封装类三条执行路径) trains without copying them, and can
 * write dQ, dK and dV straight into the matching views of a packed gradient.
 *   q, k, v, o, dout, dq, dk, dv : views of the shapes of fa_bwd. Element
 *       (b, n, h, e) of tensor X sits at X + b*sb + n*st + h*sh + e
 *       (elements; d contiguous), with (sb, st, sh) X's entries of strides.
 *   strides : HOST int64[24]: (batch, token, head) strides of q, k, v, o,
 *       dout, dq, dk, dv, in that order. Every stride a multiple of 8 (rows
 *       16-byte aligned), token strides at most 2^24. The outputs dq, dk, dv
 *       must not overlap one another or any input.
 *   lse, delta : (B, H, Nq) float32, contiguous, as in fa_bwd.
 *   causal / window_left / window_right : as in fa_fwd_strided.
 *   dtype, softmax_scale : as in fa_bwd.
 * The results equal fa_bwd's (fa_bwd_band's) on contiguous copies of the
 * same values, bit for bit.
 * Errors: as fa_bwd and fa_bwd_band; a null stride array, a stride that is
 * negative or not a multiple of 8, or causal with a window side other than -1
 * is FA_ERR_INVALID_ARGUMENT; a token stride above 2^24 is
 * FA_ERR_UNSUPPORTED.
 */
fa_status fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, int32_t B, int32_t Nq, int32_t Nk, int32_t H, int32_t d,
                         const int64_t* strides, int32_t dtype, float softmax_scale,
                         int32_t causal, int32_t window_left, int32_t window_right,
                         void* stream);

/*
 * Backward pass, packed variable-length batch on strided views: the general
 * form of fa_bwd_varlen and fa_bwd_varlen_band. Row r (packed token index),
 * head h, element e of tensor X sits at X + r*st + h*sh + e.
 *   strides : HOST int64[16]: (token, head) strides of q, k, v, o, dout, dq,
 *       dk, dv, in that order, with the rules of fa_bwd_strided.
 * cu_seqlens, num_seqs, max_seqlen, total, lse and delta as in
 * fa_bwd_varlen; the mask arguments as in fa_bwd_strided.
 */
fa_status fa_bwd_varlen_strided(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* delta, const int32_t* cu_seqlens, int32_t num_seqs,
                                int32_t max_seqlen, int32_t total, int32_t H, int32_t d,
                                const int64_t* strides, int32_t dtype, float softmax_scale,
                                int32_t causal, int32_t window_left, int32_t window_right,
                                void* stream);

/* Static description of a status code; never NULL. */
const char* fa_status_string(int32_t status);

/* Message for the calling thread's most recent failed call ("" if none).
 * The pointer stays valid until the thread's next call into the library. */
const char* fa_last_error(void);

/* Version of this ABI (incremented on incompatible change). */
int32_t fa_abi_version(void);

/*
 * Backward of fa_fwd_local (local window on a token map plus global
 * anchors): the arguments of fa_bwd for self-attention (N queries and keys)
 * with the pattern arguments of fa_fwd_local. Pairs outside the pattern carry
 * no gradient. Errors: as fa_bwd; a negative pattern size or map_w < 1 is
 * FA_ERR_INVALID_ARGUMENT; N above 2^28 is FA_ERR_UNSUPPORTED.
 */
fa_status fa_bwd_local(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       float* delta, int32_t B, int32_t N, int32_t H, int32_t d, int32_t dtype,
                       float softmax_scale, int32_t causal, int32_t n_global, int32_t map_w,
                       int32_t win_rows, int32_t win_cols, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
