/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention library (forward and backward).
 *
 * Pages cited:
 *   [PT2CUDA]  aiknowledge.cn, "4.5 注意力优化实战：从PyTorch到CUDA的完整流程".
 *   [MEMWALL]  codechina.net, "GPU 内存墙 ... FlashAttention" article.
 *   [PROFILE3] "Profiling in PyTorch (part 3): Attention is all you profile".
 *
 * The operation (one call = one fused kernel launch):
 *
 *   O[b,h] = softmax(Q[b,h] K[b,h]^T * scale + mask) V[b,h]
 *
 * as written unfused in [PT2CUDA] step 1 (baseline implementation) and
 * [PROFILE3] (naive attention module), computed tile by tile with the online
 * softmax of [PT2CUDA] step 3.1 and [MEMWALL] §3.2 so that the [N_q, N_k]
 * score matrix never reaches device memory.
 *
 * The mask is a rule, not a tensor. Query row i of batch b may attend to key j
 * iff all of:
 *   j <  kv_len[b]   with kv_len[b] = clamp(seqlens_k[b], 0, N_k), or N_k when
 *                    seqlens_k is NULL (variable-length keys marked by a
 *                    valid length, [MEMWALL] §6.2);
 *   i >= qs[b]       with qs[b] = clamp(q_start[b], 0, N_q), or 0 when q_start
 *                    is NULL (leading query rows that attend to nothing);
 *   j <= i           when causal == 1 (the lower-triangular mask of [PROFILE3],
 *                    top-left aligned when N_q != N_k);
 *   j <= i + N_k - N_q  when causal == 2 (the same triangle aligned bottom-right:
 *                    the queries are the last N_q positions of the key
 *                    sequence, as when new rows attend to cached keys; a row
 *                    with i + N_k - N_q < 0 sees no key).
 * A row with no allowed key outputs O = +0 and LSE = -inf, never NaN (the
 * NaN-safe softmax of [PROFILE3], math-backend section). Keys at or beyond
 * kv_len[b] are ignored entirely: their K and V contents are never used, so
 * padding may hold any bit pattern.
 *
 * LSE[b,h,i] = ln(sum over allowed j of exp(S_ij)), S = Q K^T * scale: the
 * natural-log log-sum-exp of the scaled scores, in float32.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by attn_fwd and attn_bwd. */
typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,      /* a required pointer is NULL                          */
  ATTN_ERR_SHAPE = 2,     /* a size is negative or the problem is too large      */
  ATTN_ERR_HEAD_DIM = 3,  /* d is not 64 or 128                                  */
  ATTN_ERR_SCALE = 4,     /* scale is NaN or infinite                            */
  ATTN_ERR_ALIGN = 5,     /* a bf16 tensor not 16-byte aligned, lse/delta 4-byte */
  ATTN_ERR_ALIAS = 6,     /* an output overlaps an input or another output       */
  ATTN_ERR_LAUNCH = 7,    /* the kernel launch failed (hipGetLastError)          */
  ATTN_ERR_MASK = 8,      /* causal not 0/1/2, or a bad mask layout              */
  ATTN_ERR_SCRATCH = 9    /* attn_bwd_noalloc: B*H*N_q above its 2^20-row limit  */
} attn_status;

/*
 * attn_fwd - fused scaled-dot-product attention forward, bf16 in, bf16 out.
 *
 * Arguments (all pointers are DEVICE memory owned by the caller; the library
 * never allocates, frees, synchronises or keeps state, so calls are
 * reentrant and may run on any stream):
 *   q          bf16 [B, H, N_q, d], contiguous, d innermost, read only.
 *   k, v       bf16 [B, H, N_k, d], contiguous, read only. May be NULL iff N_k == 0.
 *   o          bf16 [B, H, N_q, d], contiguous, written in full (every element,
 *              fully masked rows included).
 *   lse        float32 [B, H, N_q] or NULL; when given, written in full.
 *   B, H       batch and head counts (>= 0).
 *   N_q, N_k   query and key sequence lengths (>= 0); one head's K (or V),
 *              N_k * d * 2 bytes, must stay below 2^31 bytes (8M keys at
 *              d = 128), else ATTN_ERR_SHAPE.
 *   d          head dimension: 64 or 128.
 *   scale      multiplier of Q K^T, any finite value (the usual d^-0.5 of
 *              [PT2CUDA] step 1).
 *   causal     0: no causal mask; 1: key j is visible to row i only when
 *              j <= i; 2: only when j <= i + N_k - N_q. Other values:
 *              ATTN_ERR_MASK.
 *   seqlens_k  int32 [B] device array or NULL: valid key count per batch,
 *              clamped to [0, N_k] on the device.
 *   q_start    int32 [B] device array or NULL: rows i < q_start[b] of batch b
 *              attend to nothing, clamped to [0, N_q] on the device.
 *   stream     HIP stream to launch on (0 = null stream).
 *
 * Errors: argument errors are detected on the host and returned BEFORE any HIP
 * call (nothing is launched, no device state is touched). When B*H*N_q == 0
 * the call returns ATTN_OK without launching; then q, o may be NULL. A launch
 * failure returns ATTN_ERR_LAUNCH. Faults inside the kernel surface at the
 * caller's next synchronisation, as usual for HIP. The values of seqlens_k and
 * q_start are never read on the host.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N_q, int N_k, int d, float scale, int causal,
             const int32_t* seqlens_k, const int32_t* q_start, hipStream_t stream);

/*
 * attn_fwd_masked - attn_fwd with a general boolean mask intersected with the
 * rules above (the attn_mask of the pages' interfaces: [PT2CUDA] step 1
 * masks scores where the mask is 0, [PROFILE3] passes attn_mask to SDPA).
 *
 *   mask_bits        uint32 device array, 16-byte aligned, read only: for batch b,
 *                    head h, row i the words mask_bits[b*mask_stride_b +
 *                    h*mask_stride_h + i*mask_row_words + w]; bit t of word w
 *                    set means row i may attend to key 32*w + t. Bits of keys
 *                    >= N_k are ignored.
 *   mask_stride_b,   word strides between batches and heads (>= 0; 0 broadcasts
 *   mask_stride_h    one mask over that dimension).
 *   mask_row_words   words per row: >= ceil(N_k / 32) and a multiple of 8 (so a
 *                    row's words for 8 key slices are one aligned 32-byte piece).
 * Every other argument, and the outputs, as in attn_fwd. A row whose allowed
 * set is empty outputs O = 0, LSE = -inf. Errors: mask_bits NULL (with work to
 * do) ATTN_ERR_NULL, misaligned ATTN_ERR_ALIGN, bad row words or strides
 * ATTN_ERR_MASK, N_q * mask_row_words * 4 >= 2^31 ATTN_ERR_SHAPE.
 */
int attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N_q, int N_k, int d, float scale, int causal,
                    const int32_t* seqlens_k, const int32_t* q_start,
                    const uint32_t* mask_bits, long long mask_stride_b, long long mask_stride_h,
                    int mask_row_words, hipStream_t stream);

/*
 * attn_fwd_block_sparse - attn_fwd computing only the blocks a block mask
 * keeps (block-sparse attention, [MEMWALL] §7): blocks the mask drops are
 * neither loaded nor computed, and their keys get probability 0.
 *
 *   block_mask       uint8 device array, read only: for batch b, head h, query
 *                    tile t (rows 256*t .. 256*t+255) and key block s (keys
 *                    128*s .. 128*s+127) the byte block_mask[b*block_stride_b +
 *                    h*block_stride_h + t*ceil(N_k/128) + s]; nonzero = compute
 *                    the block. Rows of ceil(N_k/128) bytes, ceil(N_q/256) rows
 *                    per (b, h).
 *   block_stride_b,  byte strides between batches and heads (>= 0; 0 broadcasts).
 *   block_stride_h
 * The rules (causal, seqlens_k, q_start) still apply inside kept blocks. A
 * row with no kept, allowed key outputs O = 0, LSE = -inf. N_k is limited to
 * 32768 (1024 slices) on this path (else ATTN_ERR_SHAPE). Other arguments,
 * outputs and errors as in attn_fwd; a NULL block_mask with work to do is
 * ATTN_ERR_NULL, negative strides ATTN_ERR_MASK.
 */
int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N_q, int N_k, int d, float scale, int causal,
                          const int32_t* seqlens_k, const int32_t* q_start,
                          const uint8_t* block_mask, long long block_stride_b, long long block_stride_h,
                          hipStream_t stream);

/*
 * attn_mask_pack - pack a byte mask into the bit layout attn_fwd_masked reads.
 *   mask       uint8 device array [rows, N_k], row major; nonzero = may attend.
 *   bits       uint32 device array [rows, row_words], written in full (bits of
 *              keys >= N_k are 0).
 *   row_words  >= ceil(N_k / 32) (use a multiple of 8 for attn_fwd_masked).
 * One kernel launch on `stream`. Errors: bad sizes ATTN_ERR_SHAPE, NULL
 * pointers ATTN_ERR_NULL, bits not 4-byte aligned ATTN_ERR_ALIGN.
 */
int attn_mask_pack(const uint8_t* mask, uint32_t* bits, long long rows, int N_k, int row_words,
                   hipStream_t stream);

/*
 * attn_bwd - gradients of attn_fwd: dQ, dK, dV (bf16) from dO (bf16).
 *
 * The backward kernel of [PT2CUDA] step 4.2: dQ sweeps every K/V block, dK and
 * dV sweep every Q block, and the probabilities are recomputed from the
 * forward's log-sum-exp instead of being stored. With S, P and the mask of
 * attn_fwd (same q, k, v, scale, causal, seqlens_k, q_start):
 *   P  = exp(S - LSE) on allowed entries, 0 elsewhere;
 *   dV = P^T dO;   dP = dO V^T;   Delta_i = sum_d dO_id O_id;
 *   dS = P * (dP - Delta);   dQ = scale * dS K;   dK = scale * dS^T Q.
 * A row with no allowed key (LSE = -inf) contributes nothing; its dQ row is 0.
 * Keys at or beyond kv_len[b] get dK = dV = 0. Three kernel launches on
 * `stream` (Delta, then dQ, then dK and dV).
 *
 * Arguments (device memory owned by the caller; nothing is allocated, freed,
 * synchronised or kept):
 *   q, k, v     the forward's inputs (layouts as in attn_fwd), read only.
 *   o, lse      the forward's outputs for exactly these inputs and mask: bf16
 *               [B, H, N_q, d] and float32 [B, H, N_q], read only.
 *   dout        bf16 [B, H, N_q, d], the gradient of the loss with respect to o.
 *   dq          bf16 [B, H, N_q, d], written in full.
 *   dk, dv      bf16 [B, H, N_k, d], written in full.
 *   delta       float32 [B, H, N_q, 2] workspace, overwritten: per row
 *               (LSE * log2 e, Delta), with +inf in place of LSE * log2 e on a
 *               row with no allowed key.
 *   B .. q_start, stream  as in attn_fwd.
 * q, o, dout, lse, dq and delta may be NULL iff N_q == 0; k, v, dk and dv iff
 * N_k == 0. Alignment: the bf16 tensors 16 bytes, lse 4 bytes, delta 8 bytes.
 * No output (dq, dk, dv, delta) may overlap an input or another output.
 * Errors as in attn_fwd: argument errors return before any HIP call; when
 * B*H == 0 or N_q == N_k == 0 the call returns ATTN_OK without launching.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             int B, int H, int N_q, int N_k, int d, float scale, int causal,
             const int32_t* seqlens_k, const int32_t* q_start, hipStream_t stream);

/*
 * attn_bwd_noalloc - attn_bwd without the delta workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Computes exactly what attn_bwd computes, with the same kernels; the per-row
 * (LSE * log2 e, Delta) pairs go to a workspace the library owns: a static
 * device array of 2^20 float pairs (8 MiB) on each GPU it runs on, held until
 * the process ends. The call allocates nothing and frees nothing; on its first
 * use on a device it looks up that array's device address (a HIP call that
 * does not allocate) and keeps it. Limit: B * H * N_q <= 1048576 rows, else
 * ATTN_ERR_SCRATCH before any HIP call. Every call on one GPU uses the same
 * array: calls that overlap in time on one GPU (two streams) race and must
 * be serialised by the caller. Other arguments, errors and launches as in
 * attn_bwd.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv,
                     int B, int H, int N_q, int N_k, int d, float scale, int causal,
                     const int32_t* seqlens_k, const int32_t* q_start, hipStream_t stream);

/*
 * attn_bwd_masked - attn_bwd for attn_fwd_masked: the same gradients with the
 * bit-packed mask (same layout, strides and checks as attn_fwd_masked)
 * intersected with the rules. o and lse must come from attn_fwd_masked with
 * the same mask. Keys no row may attend to get dK = dV = 0.
 */
int attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, float* delta,
                    int B, int H, int N_q, int N_k, int d, float scale, int causal,
                    const int32_t* seqlens_k, const int32_t* q_start,
                    const uint32_t* mask_bits, long long mask_stride_b, long long mask_stride_h,
                    int mask_row_words, hipStream_t stream);

/*
 * attn_bwd_block_sparse - attn_bwd for attn_fwd_block_sparse: the same
 * gradients computing only the kept blocks (same block mask layout and
 * strides). o and lse must come from attn_fwd_block_sparse with the same
 * block mask. N_q and N_k are each limited to 32768 on this path (else
 * ATTN_ERR_SHAPE); a NULL block_mask with work to do is ATTN_ERR_NULL.
 */
int attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, float* delta,
                          int B, int H, int N_q, int N_k, int d, float scale, int causal,
                          const int32_t* seqlens_k, const int32_t* q_start,
                          const uint8_t* block_mask, long long block_stride_b, long long block_stride_h,
                          hipStream_t stream);

/*
 * attn_fwd_fp8 - attention forward with FP8 (OCP E4M3) operands.
 *
 * The mixed-precision item of section 9 (future directions) of the
 * codechina.net "GPU memory wall ... FlashAttention" article: both matrix
 * products in FP8, accumulated in fp32 (the page names a 16-bit accumulator;
 * fp32 is at least as precise). Computes, per (b, h) and query row i,
 *   S_ij = scale * (q_descale * Q8_i) . (k_descale * K8_j),
 *   O_i  = sum_j softmax_j(S_i) * v_descale * V8_j,   LSE_i = ln sum_j exp(S_ij),
 * with the causal rules of attn_fwd (0 none, 1 top-left j <= i, 2 bottom-right
 * j <= i + N_k - N_q); X8 is the tensor of decoded E4M3 codes. The
 * probabilities are rounded to E4M3 (after multiplying by 2^8) before the
 * second product; the sum that normalises them is the exact fp32 one.
 *
 *   q   device, [B, H, N_q, d] E4M3 bytes, 16-byte aligned.
 *   k   device, [B, H, N_k, d] E4M3 bytes, 16-byte aligned.
 *   vt  device, V transposed: [B, H, d, vt_row_stride] E4M3 bytes, 16-byte
 *       aligned; row (b, h, c) holds V[b, h, j, c] for keys j = 0 .. N_k-1 at
 *       byte j. vt_row_stride is a multiple of 16 and >= N_k rounded up to 16
 *       (else ATTN_ERR_SHAPE); the bytes past N_k in a row are never used.
 *       N_k * d and d * vt_row_stride (one head's K and V^T bytes) must be
 *       below 2^31 (else ATTN_ERR_SHAPE).
 *   o   device, [B, H, N_q, d] bf16 output, 16-byte aligned.
 *   lse device, [B, H, N_q] fp32 output, natural log, or NULL.
 *   d   64 or 128. scale and the three descales must be finite (any sign).
 * A row with no visible key outputs O = 0 and LSE = -inf. The library
 * allocates nothing; one kernel launch on `stream`; argument errors are
 * returned before any HIP call, as for attn_fwd (NULL, alignment, overlap of
 * o or lse with an input or each other).
 */
int attn_fwd_fp8(const void* q, const void* k, const void* vt, long long vt_row_stride, void* o, float* lse,
                 int B, int H, int N_q, int N_k, int d, float scale, float q_descale, float k_descale,
                 float v_descale, int causal, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
