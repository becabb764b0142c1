/*
 * fa355.h -- C ABI of libfa355, the attention forward pass (and its backward
 * pass, fa_bwd) for AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by site: [nanhubrain] = nanhubrain.csdn.net,
 * FlashAttention in CANN ops-transformer; [pwwt] = www.pwwt.cn/news/2518640;
 * [ascendai] = ascendai.csdn.net, efficient attention in CANN ops-nn):
 *
 *   O = softmax(scale * Q K^T [causal mask]) V            per (batch, head)
 *   LSE_i = ln sum_{j visible to i} exp(scale * q_i . k_j)
 *
 * -- [nanhubrain] "exact source of the quadratic memory" (the three-step
 * definition), [nanhubrain] "tiling skeleton" and "online softmax mathematics"
 * (computed block by block with a running row max and row sum, so the N x N
 * score matrix is never stored), [ascendai] section 3.1 (operator interface:
 * query/key/value/output, a softmax scale whose negative default means
 * 1/sqrt(d), a causal flag) and section 6.1 (causal = the strict upper
 * triangle masked: key j is visible to query i iff j <= i, top-left aligned
 * when Nq != Nk), [pwwt] "standard vs IO-aware" (the BSND layout option).
 * The per-row log-sum-exp is the statistic from which [nanhubrain] "backward
 * recomputation" rebuilds the probabilities: P_ij = exp(scale*q_i.k_j - LSE_i).
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the shared library (built with hidden default visibility). */
#if defined(__GNUC__) || defined(__clang__)
#define FA355_API __attribute__((visibility("default")))
#else
#define FA355_API
#endif

typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad enum, misalignment, NaN/inf scale */
    FA_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement (e.g. d not 64/128) */
    FA_ERR_HIP = 3            /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum fa_layout {
    FA_BHND = 0,   /* [B, H, N, d]: each head's rows contiguous             */
    FA_BSND = 1    /* [B, N, H, d]: batch-seq-head-dim, heads interleaved   */
} fa_layout;

typedef enum fa_dtype {
    FA_BF16 = 0,   /* bfloat16 */
    FA_F32 = 1     /* IEEE float32 */
} fa_dtype;

/*
 * fa_fwd -- enqueue one attention forward pass on `stream`.
 *
 * q        device pointer, Q in `layout` with N = Nq, element type `in_dtype`.
 * k, v     device pointers, K and V in `layout` with N = Nk, type `in_dtype`.
 * o        device pointer, O written in Q's layout ([B,H,Nq,d] or [B,Nq,H,d]),
 *          element type `o_dtype` (FA_F32 or FA_BF16; FA_BF16 only for
 *          bf16 inputs).
 * lse      device pointer to float32 [B, H, Nq] (always this order,
 *          contiguous), natural-log log-sum-exp of each row's scaled scores;
 *          NULL = not written.
 * B, H     batch size and number of heads, >= 1.
 * Nq, Nk   query and key/value sequence lengths, >= 1 (any value: no tile
 *          multiple is required); 2^30 or more is FA_ERR_UNSUPPORTED.
 * d        head dimension: 64 or 128 (else FA_ERR_UNSUPPORTED).
 * scale    softmax scale applied to q.k; a negative value selects 1/sqrt(d);
 *          0 is valid (uniform weights); NaN or infinity is FA_ERR_INVALID_ARG.
 * causal   0: every key is visible; non-zero: key j visible to query i iff
 *          j <= i (top-left alignment for any Nq, Nk).
 * layout   FA_BHND or FA_BSND; all of q, k, v, o are dense (no padding).
 * in_dtype FA_BF16 or FA_F32 (q, k and v share it).
 * o_dtype  FA_F32 or FA_BF16.
 * stream   a hipStream_t (NULL = the null stream).
 *
 * Alignment: q, k, v, o must be 16-byte aligned, lse 4-byte aligned.  o and
 * lse must not overlap q, k, v or each other.
 *
 * Ownership and asynchrony: the caller allocates and owns every buffer; the
 * library allocates no device memory and keeps no per-call state.  The call
 * validates its arguments, launches one kernel on `stream` and returns without
 * synchronising; buffers must stay valid until the stream reaches the kernel's
 * end.  Validation failures return before any HIP call.  Results are
 * deterministic: a fixed reduction order, no atomics.
 */
FA355_API fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                           int layout, int in_dtype, int o_dtype, void* stream);

/*
 * fa_fwd_ex -- fa_fwd with grouped key/value heads and a band of visible keys.
 *
 * Hkv      number of key/value heads, >= 1, dividing H: query head h reads
 *          key/value head h / (H / Hkv) (grouped-query attention; Hkv = 1 is
 *          multi-query, Hkv = H plain).  k and v have Hkv heads in `layout`
 *          ([B,Hkv,Nk,d] or [B,Nk,Hkv,d]).  Only the needed heads are read
 *          ([nanhubrain] "GatherPAKVCache": head selection for GQA/MQA).
 * window_left, window_right
 *          the band of [pwwt] "standard vs IO-aware" (pre_tokens /
 *          next_tokens): key j is visible to query i iff
 *          i - window_left <= j <= i + window_right; a negative value leaves
 *          that side unbounded.  `causal` still applies (j <= i) on top; a
 *          causal sliding window is (w, -1) with causal = 1, or (w, 0).
 *          Key tiles outside a query tile's band are never loaded.  A row
 *          with no visible key gets O = 0 and LSE = -inf.  An edge that
 *          masks nothing (window_left >= Nq, window_right >= Nk) is taken
 *          as unbounded.
 * All other arguments, the alignment, ownership and asynchrony rules are
 * those of fa_fwd; fa_fwd(...) is fa_fwd_ex(..., Hkv = H, window -1, -1).
 * FA_ERR_INVALID_ARG also when H % Hkv != 0; FA_ERR_UNSUPPORTED for fp32
 * inputs with Hkv != H or a band.
 */
FA355_API fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                              int window_left, int window_right, int layout, int in_dtype, int o_dtype,
                              void* stream);

/* Granularity of fa_fwd_sparse's block mask: queries x keys per block. */
#define FA_SPARSE_BQ 256
#define FA_SPARSE_BK 64

/*
 * fa_fwd_sparse -- fa_fwd with a block-sparse mask ([nanhubrain]
 * "SparseFlashAttention": a mask over (query block, key block) pairs; the
 * key blocks it marks as not needed are skipped, never loaded nor computed).
 *
 * block_mask  device pointer, uint8 [B, H, ceil(Nq / FA_SPARSE_BQ),
 *             ceil(Nk / FA_SPARSE_BK)] contiguous: key j is visible to query
 *             i iff block_mask[b][h][i / 256][j / 64] != 0 (and j <= i if
 *             causal).  A row with no visible key gets O = 0, LSE = -inf.
 * All other arguments and rules are those of fa_fwd.  FA_ERR_INVALID_ARG for
 * a NULL mask; FA_ERR_UNSUPPORTED for fp32 inputs or more than 4096 key
 * blocks (Nk > 262144).
 */
FA355_API fa_status fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const unsigned char* block_mask, int B, int H, int Nq, int Nk, int d,
                                  float scale, int causal, int layout, int in_dtype, int o_dtype, void* stream);

/*
 * fa_bwd -- enqueue the attention backward pass on `stream`: the gradients of
 * a loss L with respect to Q, K and V, given dO = dL/dO.
 *
 * The operation ([nanhubrain] "backward recomputation"): the probabilities
 * are rebuilt tile by tile from the forward pass's log-sum-exp,
 * P_ij = exp(scale * q_i.k_j - LSE_i) on visible pairs (0 on masked ones), and
 *   D_i  = sum_j P_ij (dO_i . v_j) = dO_i . O_i      (the whole row)
 *   dS_ij = P_ij (dO_i . v_j - D_i)
 *   dQ_i = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i,
 *   dV_j = sum_i P_ij dO_i.
 * The page's listing sums the row term over one key block only; the softmax
 * derivative needs it over the whole row, which is what is computed here.
 *
 * q, k, v   device pointers, as for fa_fwd (element type `in_dtype`).
 * o         device pointer, the forward output O in Q's layout, element type
 *           `o_dtype` (FA_F32 or FA_BF16); used only for D_i = dO_i . O_i.
 * dout      device pointer, dO in Q's layout, element type `in_dtype`.
 * lse       device pointer, float32 [B, H, Nq] contiguous: the natural-log
 *           log-sum-exp of each row's scaled scores, as fa_fwd writes it.
 * dq        device pointer, dQ written as float32 in Q's layout.
 * dk, dv    device pointers, dK and dV written as float32 in K's layout.
 * delta     device pointer to a caller-owned float32 workspace of B*H*Nq
 *           elements; overwritten with D (its contents on entry do not
 *           matter; on return it holds D_i in [B, H, Nq] order).
 * B, H, Nq, Nk, d, scale, causal, layout: as for fa_fwd (scale < 0 selects
 *           1/sqrt(d); scale must be the one the forward pass used).
 * in_dtype  FA_BF16 (FA_F32 inputs return FA_ERR_UNSUPPORTED).
 * o_dtype   FA_F32 or FA_BF16.
 * stream    a hipStream_t (NULL = the null stream).
 *
 * Alignment: q, k, v, o, dout, dq, dk, dv 16-byte aligned; lse and delta
 * 4-byte aligned.  The outputs and the workspace must not overlap the inputs
 * or each other.
 *
 * Ownership and asynchrony: as for fa_fwd.  The library allocates no device
 * memory; the call validates its arguments (returning before any HIP call
 * on failure), enqueues three kernels on `stream` (D, then dK/dV, then dQ)
 * and returns without synchronising.  Results are deterministic: a fixed
 * reduction order, no atomics.
 */
FA355_API fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, float* dq, float* dk, float* dv, float* delta,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                           int layout, int in_dtype, int o_dtype, void* stream);

/*
 * fa_bwd_ex -- fa_bwd for grouped key/value heads and a band of visible keys:
 * the backward pass of fa_fwd_ex.
 *
 * The operation: query head h reads key/value head h / (H / Hkv) and row i
 * sees keys i - window_left .. i + window_right (and j <= i if causal), as in
 * fa_fwd_ex ([nanhubrain] "GatherPAKVCache" head map, [pwwt] "standard vs
 * IO-aware" pre_tokens / next_tokens).  The gradients are fa_bwd's over each
 * row's visible keys; K and V of one head enter the softmax of every query
 * head of its group, so dK and dV of that head are the sums of the per-head
 * terms over the group (the chain rule through the shared rows).  A row with
 * no visible key (forward: O = 0, LSE = -inf) has no gradient: dQ_i = 0, and
 * it adds nothing to dK or dV.
 *
 * Hkv      number of key/value heads, >= 1, dividing H.  k, v, dk and dv have
 *          Hkv heads in `layout`; q, o, dout, dq and lse have H.
 * window_left, window_right
 *          the band, as for fa_fwd_ex (negative = unbounded); lse must come
 *          from a forward pass with the same band, heads and causal flag.
 * Every other argument, alignment, ownership, asynchrony and determinism as
 * for fa_bwd; fa_bwd(...) is fa_bwd_ex(..., Hkv = H, window -1, -1).
 * FA_ERR_INVALID_ARG also when H % Hkv != 0; FA_ERR_UNSUPPORTED also when
 * Nq or Nk is 2^30 or more.
 */
FA355_API fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, float* dq, float* dk, float* dv, float* delta,
                              int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                              int window_left, int window_right, int layout, int in_dtype, int o_dtype,
                              void* stream);

/*
 * fa_bwd_sparse -- fa_bwd for block-sparse attention: the backward pass of
 * fa_fwd_sparse.
 *
 * The operation: key j is visible to query i iff
 * block_mask[b][h][i / FA_SPARSE_BQ][j / FA_SPARSE_BK] != 0 (and j <= i if
 * causal), as in fa_fwd_sparse ([nanhubrain] "SparseFlashAttention": the
 * blocks the mask leaves off are skipped).  The gradients are fa_bwd's over
 * each row's visible keys; a row with no visible key has no gradient and
 * adds nothing to dK or dV.  Key blocks the mask leaves off are never read
 * for dQ, and query blocks that leave a key block off are never read for its
 * dK and dV.
 *
 * block_mask  device pointer, uint8 [B, H, ceil(Nq/256), ceil(Nk/64)]
 *             contiguous, the mask the forward pass used.
 * Every other argument, alignment, ownership, asynchrony and determinism as
 * for fa_bwd.  FA_ERR_INVALID_ARG also for a NULL mask; FA_ERR_UNSUPPORTED
 * also for more than 4096 key blocks or more than 4096 query blocks, or Nq or
 * Nk of 2^30 or more.
 */
FA355_API fa_status fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                  const float* lse, const unsigned char* block_mask, float* dq, float* dk, float* dv,
                                  float* delta, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                                  int layout, int in_dtype, int o_dtype, void* stream);

/*
 * fa_decode -- enqueue decode attention over a paged KV cache on `stream`.
 *
 * The operation: Nq new tokens of each of B sequences attend to the
 * sequence's cached keys and values.  Token t of sequence b sits at position
 * L_b - Nq + t (L_b = seq_lens[b]); key j < L_b is visible to it (causal: j <=
 * L_b - Nq + t).  O and LSE are those of fa_fwd over the visible keys.  The
 * cache is paged as [nanhubrain] "GatherPAKVCache" describes: logical block i
 * of sequence b is physical block block_tables[b][i], and query head h reads
 * key/value head h / (H / Hkv).  The kernels read the blocks in place (no
 * gathered copy), split each sequence's keys into chunks, and merge the
 * chunks' partial results with the online-softmax merge
 * (LSE = log sum_s exp LSE_s, O = sum_s exp(LSE_s - LSE) O_s).
 *
 * q            device, [B, Nq, H, d] bf16 (the new tokens' queries).
 * k_cache,
 * v_cache      device, [num_blocks, block_size, Hkv, d] bf16.
 * block_tables device, int32 [B, max_blocks]: physical block ids; the first
 *              ceil(L_b / block_size) entries of row b must be valid blocks.
 * seq_lens     device, int32 [B]: L_b, 0 <= L_b <= max_blocks * block_size
 *              (values outside are clamped to that range); causal needs
 *              L_b >= Nq (a token at a negative position sees no key).
 * o            device, [B, Nq, H, d], element type `o_dtype`.
 * lse          device, float32 [B, H, Nq], natural log; NULL = not written.
 *              A row with no visible key (L_b = 0) gets O = 0, LSE = -inf.
 * workspace    device, at least fa_decode_workspace_bytes(B, H, Hkv, Nq, d,
 *              max_blocks * block_size) bytes, 16-byte aligned, caller-owned;
 *              holds the chunks' partial results (overwritten).
 * block_size   tokens per block, a power of two >= 16.
 * scale        as for fa_fwd (negative: 1/sqrt(d)).
 * in_dtype     FA_BF16 (FA_F32 is FA_ERR_UNSUPPORTED); o_dtype FA_F32 or FA_BF16.
 *
 * Errors: FA_ERR_INVALID_ARG for null pointers, sizes < 1, H % Hkv != 0, a
 * block size that is not a power of two >= 16, misalignment, NaN/inf scale or
 * a workspace below the required size; FA_ERR_UNSUPPORTED for d not 64/128.
 * The library allocates nothing; two kernels are enqueued, no synchronisation.
 */
FA355_API fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* block_tables,
                              const int* seq_lens, void* o, float* lse, void* workspace, size_t workspace_bytes,
                              int B, int H, int Hkv, int Nq, int d, int block_size, int max_blocks, float scale,
                              int causal, int in_dtype, int o_dtype, void* stream);

/* Workspace bytes fa_decode needs for these sizes (max_seq_len = max_blocks *
 * block_size); 0 for invalid sizes. */
FA355_API size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int Nq, int d, int max_seq_len);

/* Largest workspace fa_decode_noalloc can stand in for (bytes). */
#define FA_DECODE_NOALLOC_MAX_WORKSPACE (64u << 20)

/*
 * fa_decode_noalloc -- fa_decode without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that may not call hipMalloc).  Same operation, arguments (less workspace
 * and workspace_bytes), kernels and results as fa_decode.  The chunk
 * partials go to a fixed device array of FA_DECODE_NOALLOC_MAX_WORKSPACE
 * bytes inside the library: each GPU it runs on holds its own copy until the
 * process ends; the first call on a device looks up that device's copy
 * (hipGetSymbolAddress, with the device current).  Nothing is allocated: no
 * hipMalloc, no hipFree, no allocating library call.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's partials (every partial a call reads, it first writes).  Calls that
 * overlap on one GPU (concurrent streams, or several host threads) race on it
 * and must be ordered by the caller.
 *
 * Errors: as fa_decode; FA_ERR_UNSUPPORTED when the partials of these sizes
 * (fa_decode_workspace_bytes) exceed FA_DECODE_NOALLOC_MAX_WORKSPACE;
 * FA_ERR_HIP if the array's address cannot be looked up.
 */
FA355_API fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                      const int* block_tables, const int* seq_lens, void* o, float* lse, int B, int H,
                                      int Hkv, int Nq, int d, int block_size, int max_blocks, float scale,
                                      int causal, int in_dtype, int o_dtype, void* stream);

/* A static, human-readable name for a status code (never NULL). */
FA355_API const char* fa_status_str(int status);

/* ABI version of this header (incremented on incompatible change). */
FA355_API int fa_abi_version(void);

#define FA355_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
