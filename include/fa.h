/*
 * fa.h — C ABI of the exact tiled attention library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 *   Exact scaled-dot-product attention, per (batch b, head h):
 *       O = softmax(scale * Q K^T) V            (row-wise softmax over keys)
 *   as defined in aiwiki.page "FlashAttention", section "Attention and the memory
 *   bottleneck" (masks restrict which query-key pairs interact), computed by the tiled
 *   online-softmax method of the same page, section "Tiling and online normalization",
 *   so the N x N score matrix never reaches device memory. Only the per-row log-sum-exp
 *       lse_i = ln sum_{j allowed} exp(scale * q_i . k_j)
 *   is kept (sendsoonai.com "FlashAttention: IO-aware explained", section
 *   "Recomputation and IO complexity": only the softmax statistics are stored), and the
 *   backward pass recomputes each score tile from it.
 *
 * Allowed pairs (all predicates combine with AND)
 *   causal       : key j <= query i (square self-attention, queries and keys share N)
 *   kv_len       : key j <  kv_len[b] (key padding; aiwiki "FlashAttention", section
 *                  "Software integration and limitations": variable-length sequences)
 *   block_mask   : block_mask[i / mask_block][j / mask_block] != 0 (legiblepapers.com
 *                  "Fast and Memory Efficient Exact Attention", summary: block-sparse
 *                  attention skips the zero blocks of a predefined block mask)
 *   Query rows are never masked. A row with no allowed key yields O = 0, lse = -inf and a
 *   zero dQ row.
 *
 * Conventions shared by every entry point
 *   - Tensors q, k, v, o, dout, dq, dk, dv are DEVICE pointers owned by the caller, laid out
 *     [B, H, N, d] row-major (d contiguous), all of the same dtype, 16-byte aligned.
 *     lse is a device float array [B, H, N] (natural log), 4-byte aligned.
 *     kv_len, when not NULL, is a device int32 array [B]; values are clamped to [0, N].
 *     block_mask, when used, is a device uint8 array [nb, nb] row-major with
 *     nb = ceil(N / mask_block), shared by every (b, h).
 *   - Every call validates its arguments synchronously on the host, before touching the
 *     device. On any error nothing is launched and no output is written.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default stream). The library
 *     allocates no device memory and keeps no per-call state: calls are re-entrant and
 *     thread-safe. Faults during execution surface at the caller's stream synchronisation.
 *   - N (and max_seqlen of the packed calls) is at most 2^30 (FA_ERR_UNSUPPORTED beyond).
 *   - bf16 (FA_BF16): d in {16, 32, 64, 128}, forward and backward. fp32 (FA_F32): d in
 *     {32, 64, 128}, forward only. The key/value-cache forward takes its own query and
 *     key counts (Nq, Nk) in place of N; its tensors follow the same layout. The packed
 *     variable-length calls use [total, H, d] tensors and [H, total] lse instead.
 */
#ifndef EXACT_TILED_ATTENTION_FA_H
#define EXACT_TILED_ATTENTION_FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_F32 = 0,  /* IEEE fp32 tensors */
  FA_BF16 = 1  /* bfloat16 tensors; arithmetic accumulates in fp32 */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = 1,     /* bad argument: NULL or misaligned pointer, non-positive or
                             overflowing size, NaN/Inf scale, mask without a valid
                             mask_block, workspace missing or too small */
  FA_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement (dtype / d
                             combination, backward in fp32, too many mask blocks); the
                             caller may fall back to another implementation */
  FA_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} fa_status;

/*
 * Forward pass: O and lse.
 *   dt        element type of q, k, v, o
 *   B, H, N, d  batch, heads, sequence length (queries = keys), head dimension
 *   q, k, v   inputs [B,H,N,d] (read only)
 *   o         output [B,H,N,d]
 *   lse       output [B,H,N] fp32, natural-log log-sum-exp of the scaled scores of each row
 *   scale     multiplier of q.k inside the softmax (1/sqrt(d) for standard attention)
 *   causal    nonzero: key j allowed only for j <= i
 *   kv_len    NULL (every key valid) or device int32 [B] of valid key counts
 * Online-softmax update of aiwiki "FlashAttention", section "Tiling and online
 * normalization" (running max, rescaled running sum and accumulator, final O = u / l).
 */
fa_status fa_fwd(fa_dtype dt, int B, int H, int N, int d,
                 const void* q, const void* k, const void* v,
                 void* o, float* lse,
                 float scale, int causal, const int32_t* kv_len,
                 hipStream_t stream);

/*
 * Block-sparse forward: as fa_fwd, and additionally every key tile whose mask block is
 * zero is skipped without being read (legiblepapers.com "Fast and Memory Efficient Exact
 * Attention", summary paragraph). O is written for every row.
 *   block_mask  device uint8 [nb, nb], nb = ceil(N / mask_block), nonzero = keep
 *   mask_block  side of a square mask block; a positive multiple of 128
 */
fa_status fa_fwd_blocksparse(fa_dtype dt, int B, int H, int N, int d,
                             const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             float scale, int causal, const int32_t* kv_len,
                             const uint8_t* block_mask, int mask_block,
                             hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: the per-row D = rowsum(dO * O) (fp32 [B,H,N],
 * rounded up to 256 bytes), then 4 KB for the block-sparse order of the key tiles. Linear in N (the backward keeps O(N) extra memory; cochat.ai
 * audit of "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness",
 * quoted backward-pass memory claim). Returns 0 for non-positive or overflowing sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass: dQ, dK, dV of L = sum(O * dout) (bf16 only).
 *   q, k, v, o, lse   the inputs and outputs of the matching forward call (same mask
 *                     arguments); o and lse are read, not recomputed
 *   dout              upstream gradient [B,H,N,d]
 *   dq, dk, dv        outputs [B,H,N,d]
 *   block_mask        NULL (dense) or as in fa_fwd_blocksparse; mask_block ignored if NULL;
 *                     with a mask N is at most 131072 (FA_ERR_UNSUPPORTED beyond)
 *   workspace         device memory of at least fa_bwd_workspace_bytes(B,H,N,d) bytes,
 *                     256-byte aligned, owned by the caller; its contents on entry do not
 *                     matter and are overwritten
 * Structure (cochat.ai audit, quoted Theorem 5 proof / App. C): each key/value tile is
 * loaded once and its dK, dV stay on chip while query tiles stream past. dQ is computed by
 * a second, query-major pass that keeps dQ on chip while key tiles stream past. Both
 * recompute the score tile from q, k and lse. No atomics: results are deterministic.
 */
fa_status fa_bwd(fa_dtype dt, int B, int H, int N, int d,
                 const void* q, const void* k, const void* v,
                 const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv,
                 float scale, int causal, const int32_t* kv_len,
                 const uint8_t* block_mask, int mask_block,
                 void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/*
 * Forward and backward with dropout on the attention probabilities (bf16). The cochat.ai
 * audit of "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"
 * quotes the fused kernel applying dropout to the probabilities and the backward
 * regenerating the mask instead of storing it. The generator is Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011). One call
 * covers 4 keys x 2 queries: key j of query i in (b, h) takes 16-bit half i % 2 (0 = low)
 * of word j % 4 of Philox(counter (j / 4, i / 2, h, b), key (seed mod 2^32, seed / 2^32))
 * and is kept iff that value is >= min(floor(dropout_p * 2^16), 65535); kept probabilities
 * are scaled by 1 / (1 - dropout_p). lse is that of the undropped softmax, as fa_fwd's, and
 * fa_bwd_dropout must get the forward's dropout_p and seed to regenerate the same mask.
 *   dropout_p  in [0, 1); 0 gives exactly fa_fwd / fa_bwd (same kernels)
 *   seed       64-bit generator key; a new seed draws a new mask
 * Other arguments as fa_fwd / fa_bwd (no block mask).
 */
fa_status fa_fwd_dropout(fa_dtype dt, int B, int H, int N, int d,
                         const void* q, const void* k, const void* v,
                         void* o, float* lse,
                         float scale, int causal, const int32_t* kv_len,
                         float dropout_p, uint64_t seed,
                         hipStream_t stream);

fa_status fa_bwd_dropout(fa_dtype dt, int B, int H, int N, int d,
                         const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv,
                         float scale, int causal, const int32_t* kv_len,
                         float dropout_p, uint64_t seed,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Packed variable-length sequences with an optional sliding window (bf16, d in {16, 32,
 * 64, 128}).
 * aiwiki "FlashAttention", section "Software integration and limitations", lists
 * variable-length sequences and sliding-window masks among the interfaces; the cochat.ai
 * audit's citation check of the Longformer reference describes sliding-window attention as
 * each query attending a fixed window of keys.
 *   nseq, H, d     sequences, heads, head dimension
 *   total          tokens over all sequences (0 is allowed: nothing is launched)
 *   max_seqlen     an upper bound of every sequence length (sizes the grid; a longer
 *                  sequence leaves its rows past max_seqlen unwritten)
 *   cu_seqlens     device int32 [nseq + 1]: sequence s owns tokens cu[s] .. cu[s+1] - 1;
 *                  cu[0] = 0, nondecreasing, cu[nseq] = total (values are clamped into
 *                  [0, total], so no boundary array makes the kernels access memory
 *                  outside the tensors)
 *   q, k, v, o     [total, H, d] row-major (tokens of all sequences, one after another)
 *   lse            [H, total] fp32, natural log
 *   causal         nonzero: key j allowed only for j <= i (positions inside the sequence)
 *   window_left    >= 0: key j allowed only for j >= i - window_left; -1: unbounded
 *   window_right   >= 0: key j allowed only for j <= i + window_right; -1: unbounded
 *                  (ignored when causal, which already bounds j <= i)
 *                  An extent >= max_seqlen bounds nothing inside a sequence of at most
 *                  max_seqlen tokens and is taken as -1 (so any int is valid, INT_MAX too).
 *   max_seqlen beyond 2^30 is FA_ERR_UNSUPPORTED.
 * Attention never crosses a sequence boundary. A row with no allowed key yields O = 0,
 * lse = -inf and a zero dQ row. The kernels are those of fa_fwd / fa_bwd; key tiles that
 * lie wholly outside a query tile's window are not read.
 */
fa_status fa_fwd_varlen(fa_dtype dt, int nseq, int H, int total, int max_seqlen, int d,
                        const int32_t* cu_seqlens,
                        const void* q, const void* k, const void* v,
                        void* o, float* lse,
                        float scale, int causal, int window_left, int window_right,
                        hipStream_t stream);

/* Bytes of device workspace fa_bwd_varlen needs: D = rowsum(dO * O), fp32 [H, total],
 * rounded up to 256 bytes. Returns 0 for non-positive H or d, negative total or overflow. */
size_t fa_bwd_varlen_workspace_bytes(int H, int total, int d);

/*
 * Backward of fa_fwd_varlen (same arguments; o and lse from the forward call): dq, dk, dv
 * [total, H, d]. workspace: device memory of at least fa_bwd_varlen_workspace_bytes(H,
 * total, d) bytes, 256-byte aligned, owned by the caller, overwritten. Deterministic (no
 * atomics), as fa_bwd.
 */
fa_status fa_bwd_varlen(fa_dtype dt, int nseq, int H, int total, int max_seqlen, int d,
                        const int32_t* cu_seqlens,
                        const void* q, const void* k, const void* v,
                        const void* o, const void* dout, const float* lse,
                        void* dq, void* dk, void* dv,
                        float scale, int causal, int window_left, int window_right,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Bytes of device workspace fa_fwd_kvcache needs for the partial results of its key split:
 * slots*Nq*(4d + 8) bytes (three regions, each rounded up to 256 bytes), where
 * slots = min(2048, B*H*ceil(Nk/32)) + B*H - 1 (at most 2048 waves share the key tiles of
 * all (b, h); each wave leaves one partial result per (b, h) its tiles touch). Returns 0
 * for non-positive or overflowing sizes.
 */
size_t fa_fwd_kvcache_workspace_bytes(int B, int H, int Nq, int Nk, int d);

/*
 * Forward of a few new queries against a key/value cache (inference decoding; aiwiki
 * "FlashAttention", section "Software integration and limitations", lists cached keys and
 * values among the supported interfaces). bf16 only, d in {16, 32, 64, 128}, 1 <= Nq <= 32.
 *   q                 [B,H,Nq,d]: the queries of the last Nq positions of each sequence
 *   k_cache, v_cache  [B,H,Nk,d]: cached keys and values; positions >= the valid length
 *                     are never read into the result (their contents do not matter)
 *   o                 output [B,H,Nq,d]
 *   lse               output [B,H,Nq] fp32, natural log
 *   kv_len            NULL (all Nk cached positions valid) or device int32 [B]: valid
 *                     length L_b of each sequence, clamped to [0, Nk]
 *   causal            nonzero: query i (0-based among the Nq) sits at position
 *                     L_b - Nq + i and attends keys j <= L_b - Nq + i (the mask aligned to
 *                     the bottom-right corner); zero: it attends every key j < L_b
 *   workspace         device memory of at least fa_fwd_kvcache_workspace_bytes(B,H,Nq,Nk,d)
 *                     bytes, 256-byte aligned, owned by the caller, overwritten
 * The valid 32-key tiles of all (b, h) are split into equal contiguous ranges, one per
 * wave, each run with the online softmax of aiwiki "FlashAttention", section "Tiling and
 * online normalization"; a second kernel merges the partial (max, sum, unnormalised
 * output) of each (b, h) with the same update. A query with no allowed key yields O = 0 and
 * lse = -inf. Caches of more than 2^31-1 key tiles over all (b, h) give FA_ERR_UNSUPPORTED.
 */
fa_status fa_fwd_kvcache(fa_dtype dt, int B, int H, int Nq, int Nk, int d,
                         const void* q, const void* k_cache, const void* v_cache,
                         void* o, float* lse,
                         float scale, int causal, const int32_t* kv_len,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * The cache forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, semantics
 * and kernels as fa_fwd_kvcache, without the workspace: the key split's partial results go
 * to a static device array of FA_NOALLOC_SCRATCH_BYTES bytes that the library defines.
 *   - Allocates nothing: no hipMalloc, hipFree or allocating library routine. Each device
 *     the call runs on holds its own copy of the array, from the first call on that device
 *     (which looks up its address once) until the process ends.
 *   - A call whose partial results would need more than FA_NOALLOC_SCRATCH_BYTES bytes
 *     (fa_fwd_kvcache_workspace_bytes(B,H,Nq,Nk,d)) returns FA_ERR_UNSUPPORTED and launches
 *     nothing.
 *   - Every call on one device shares that device's array, which keeps the last call's
 *     contents (every slot a call reads is written by the same call first, so nothing needs
 *     clearing). Calls that overlap on one device (different streams or threads, without
 *     ordering between them) race on the array and must not be issued.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

fa_status fa_fwd_kvcache_noalloc(fa_dtype dt, int B, int H, int Nq, int Nk, int d,
                                 const void* q, const void* k_cache, const void* v_cache,
                                 void* o, float* lse,
                                 float scale, int causal, const int32_t* kv_len,
                                 hipStream_t stream);

/*
 * Measurement hook. The next fa_fwd, fa_fwd_blocksparse, fa_fwd_dropout, fa_fwd_varlen,
 * fa_fwd_kvcache, fa_fwd_kvcache_noalloc, fa_bwd, fa_bwd_dropout or fa_bwd_varlen call on
 * the calling thread that passes validation records events[0] on its stream immediately
 * before its first kernel and events[i] immediately after its i-th kernel, for i < n (at
 * most 8 events; kernels past the supplied events are not bracketed). Kernels in launch
 * order:
 *   forward calls:      the forward kernel (events[0], events[1])
 *   backward calls:     [with a block mask: the key-tile order kernel,] the dQ kernel (whose
 *                       prologue computes D = rowsum(dO * O)), the dK/dV kernel
 *   cache forward:      the key-split kernel, the merge kernel
 * The request is then forgotten. events == NULL, n <= 0 or a NULL entry clears a pending
 * request. The events are owned by the caller.
 */
void fa_time_next_call(const hipEvent_t* events, int n);

/* Static English name of a status code. */
const char* fa_status_string(fa_status s);

/* Human-readable reason for the last non-OK status returned on the calling thread
 * (static per-thread storage, valid until the next call on that thread). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTENTION_FA_H */
