/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention-2 forward library, libfa.so.
 *
 * The library computes, for every batch b, head h and query row i,
 *
 *   O[b,h,i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:]  (+ causal mask) ) V[b,h,j,:]
 *   LSE[b,h,i] = ln sum_j exp( scale * Q[b,h,i,:] . K[b,h,j,:] )   over visible j
 *
 * tile by tile, without materialising the Nq x Nk score matrix.  Sources:
 *   - Ringi, "Lecture 25: FlashAttention principles and Triton practice",
 *     section 1.1 (three-step attention), section 2 (online softmax and the
 *     rescaled output accumulator), experiment 3 (forward with LSE, default
 *     scale 1/sqrt(d)).
 *   - AIInfraGuide 6.2, "FlashAttention V2 explained", section 2 (Q outer, KV
 *     inner), section 5 (causal block skipping) and its forward pseudocode
 *     (saved statistic L = m + log l).
 *   - LLM Infra Atlas, "FA2: parallelism and work partitioning", section 2
 *     (grid over query tiles x batch x heads; split-KV with a combine kernel for
 *     decode) and section 4 (causal key bound offset by seqlen_k - seqlen_q).
 *   - KingOfEgg, "Flash Attention (4): v2.1 forward vs official source",
 *     section 3.5 (inv_sum = 1 when the row sum is 0 or NaN; lse =
 *     row_max * scale + log(sum)).
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, contiguous, row-major: q and o are [B, H, Nq, d];
 *     k and v are [B, H, Nk, d]; lse is float32 [B, H, Nq].  d is innermost.
 *   - q, k, v and o hold the same 16-bit type (dtype).  All device pointers must
 *     be 16-byte aligned.
 *   - Causal visibility is bottom-right aligned: key j is visible to query i iff
 *     j <= i + (Nk - Nq).  With Nq == Nk this is j <= i.  A query that sees no key
 *     (only possible when causal and Nq > Nk) gets O = 0 and LSE = -inf.
 *   - LSE is the natural log-sum-exp of the *scaled* scores.
 *   - scale is used as given (any finite float; negative and zero allowed).
 *   - Outputs are rounded to nearest even into dtype.
 *   - Ownership: the caller owns every buffer.  The library allocates, frees and
 *     synchronises nothing; all work is enqueued on `stream` (a hipStream_t;
 *     NULL is the default stream) and returns before it completes.
 *   - Errors: every argument is validated before any HIP call, so a bad call
 *     returns without touching the device.  A kernel-launch failure reported by
 *     the HIP runtime returns FA_ERR_HIP.  Nothing prints, aborts or throws.
 *   - The results are deterministic: no atomics, fixed reduction orders.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,       /* B, H, Nq, Nk < 1, num_splits out of [1, Nk], H_kv not dividing H,
                               or a size overflows */
    FA_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, unknown dtype, non-finite scale, misaligned pointer */
    FA_ERR_WORKSPACE = 4,   /* a workspace too small for the request */
    FA_ERR_HIP = 5          /* the HIP runtime reported an error at launch */
} fa_status;

/*
 * Prefill / full forward.  Writes o ([B,H,Nq,d], dtype) and lse ([B,H,Nq], fp32).
 * One workgroup per (query tile, b, h) walks the key tiles that the causal bound
 * leaves visible (LLM Infra Atlas, FA2 parallelism, sections 2 and 4).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Nq, int Nk, int d, int causal, float scale,
                 fa_dtype dtype, void* stream);

/*
 * fa_fwd with K/V heads shared by groups of query heads (GQA; MQA when
 * H_kv = 1): k and v are [B, H_kv, Nk, d] and query head h attends to K/V head
 * h / (H / H_kv) (KingOfEgg, Flash Attention (4), section 5: K/V index mapped by
 * group).  H % H_kv must be 0, else FA_ERR_SHAPE.  With H_kv = H this is fa_fwd.
 */
fa_status fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale,
                     fa_dtype dtype, void* stream);

/*
 * Prefill over variable-length sequences packed without padding, with K/V heads
 * shared by groups of query heads (GQA; MQA when H_kv = 1).  Packing skips the
 * work a padded batch would spend on padding (Ringi, Lecture 25, section 7:
 * the varlen interface takes the cumulative sequence offsets cu_seqlens);
 * grouped heads index K/V by h / (H / H_kv) (KingOfEgg, Flash Attention (4),
 * section 5: K/V index mapped by group, entry point with cu_seqlens).
 *
 *   q, o           [total_q, H, d]     dtype (token-major: token t of sequence b
 *                                       is row cu_seqlens_q[b] + t)
 *   k, v           [total_k, H_kv, d]  dtype
 *   lse            [H, total_q]        float32
 *   cu_seqlens_q   int32 device array of B + 1 offsets: 0 = cu[0] <= cu[1] <= ...
 *   cu_seqlens_k   <= cu[B] = total_q (resp. total_k); sequence b's queries are
 *                  tokens [cu_q[b], cu_q[b+1]) and its keys [cu_k[b], cu_k[b+1])
 *   max_seqlen_q/k bounds on every sequence's query / key count
 *
 * Query head h of sequence b attends to K/V head h / (H / H_kv) of the same
 * sequence; causal visibility is bottom-right aligned within each sequence (key
 * j visible to query i iff j <= i + Nk_b - Nq_b), and a query that sees no key
 * (also when Nk_b = 0) gets O = 0 and LSE = -inf.  Requirements: B, H, H_kv >= 1,
 * H % H_kv == 0, 1 <= max_seqlen_q <= total_q, 1 <= max_seqlen_k <= total_k;
 * cu_seqlens 4-byte aligned.  The offsets live on the device and are not read by
 * the host: a sequence whose offsets fall outside [0, total], decrease, or span
 * more than max_seqlen is skipped by the kernel: its rows of o and lse keep
 * whatever the caller's buffers held before the call (the library neither clears
 * nor reports them; a caller that cannot vouch for its offsets clears o to 0 and
 * lse to -inf first), and no memory outside the tensors is accessed.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k,
                        int B, int H, int H_kv, int total_q, int total_k,
                        int max_seqlen_q, int max_seqlen_k, int d, int causal, float scale,
                        fa_dtype dtype, void* stream);

/*
 * Bytes of partial results fa_fwd_splitkv writes for the given shape:
 * num_splits * B * H * Nq * (d + 1) * 4.  Returns 0 for invalid sizes.
 */
size_t fa_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits);

/*
 * Split-KV forward, first half (LLM Infra Atlas, FA2 parallelism, section 2:
 * when seqlen_q is small, split the keys into num_splits chunks, each producing
 * a partial (O, LSE)).  Split s covers keys [s*c, min(Nk, (s+1)*c)) with
 * c = ceil(Nk / num_splits); trailing splits may be empty.  For every split and
 * row it writes the attention restricted to that chunk, *normalised*, in fp32:
 *   o_part   [num_splits, B, H, Nq, d]  float32
 *   lse_part [num_splits, B, H, Nq]     float32  (-inf, with o_part = 0, when the
 *                                                  row sees no key of the chunk)
 * Causal visibility is applied inside each chunk.  1 <= num_splits <= Nk.
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v,
                         float* o_part, float* lse_part,
                         int B, int H, int Nq, int Nk, int d, int causal, float scale,
                         int num_splits, fa_dtype dtype, void* stream);

/*
 * fa_fwd_splitkv with grouped K/V heads: k and v are [B, H_kv, Nk, d], query head
 * h reads K/V head h / (H / H_kv); partials and their combine are as above (one
 * row per query head).  For Nq = 1 a workgroup serves up to 8 query heads of one
 * group and streams their shared K/V chunk once.  H % H_kv must be 0.
 */
fa_status fa_fwd_splitkv_gqa(const void* q, const void* k, const void* v,
                             float* o_part, float* lse_part,
                             int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale,
                             int num_splits, fa_dtype dtype, void* stream);

/*
 * Split-KV decode over a paged K/V cache: one query row per sequence and head
 * (q [B, H, d]) attending to that sequence's cached keys, which are scattered
 * over fixed-size pages (Ringi, "Lecture 25", section 8.3, the PagedAttention
 * question: a K/V cache split into non-contiguous pages, the kernel's address
 * computation going through a page table).
 *   k_cache, v_cache  [num_pages, page_size, H_kv, d]  dtype, 16-byte aligned
 *   block_table       [B, max_pages]  int32, device: physical page of logical
 *                     page j of sequence b (key t lives at row t % page_size of
 *                     page block_table[b][t / page_size])
 *   seqlens_k         [B]  int32, device: cached keys of sequence b
 * Query head h reads K/V head h / (H / H_kv).  Sequence b is split into
 * num_splits chunks of c_b = ceil(seqlens_k[b] / num_splits) keys; split s
 * covers keys [s*c_b, min(len_b, (s+1)*c_b)).  The outputs are the partials of
 * fa_fwd_splitkv with Nq = 1 (o_part [num_splits, B, H, 1, d], lse_part
 * [num_splits, B, H, 1], sized by fa_splitkv_workspace_bytes(B, H, 1, d,
 * num_splits)), merged by fa_splitkv_combine.  A sequence of length 0 gives
 * O = 0 and LSE = -inf.  Requirements: page_size a power of two, H % H_kv == 0,
 * num_splits >= 1, max_pages * page_size <= INT32_MAX; block_table and
 * seqlens_k 4-byte aligned.  The table and lengths live on the device and are
 * not read by the host: a length outside [0, max_pages * page_size] leaves that
 * sequence's partials as the caller's buffers held them (clear o_part to 0 and
 * lse_part to -inf first to have such a sequence combine to O = 0, LSE = -inf),
 * and a page entry outside [0, num_pages) drops its keys; no memory outside the
 * tensors is accessed.
 */
fa_status fa_fwd_splitkv_paged(const void* q, const void* k_cache, const void* v_cache,
                               const int* block_table, const int* seqlens_k,
                               float* o_part, float* lse_part,
                               int B, int H, int H_kv, int d, int page_size, int max_pages, int num_pages,
                               float scale, int num_splits, fa_dtype dtype, void* stream);

/*
 * Split-KV decode over packed variable-length sequences: one query row per
 * sequence and head (q [B, H, d], i.e. the packed query layout [total_q, H, d]
 * with one row per sequence) attending to that sequence's keys, which are
 * stored back to back without padding and located by cumulative offsets (Ringi,
 * "Lecture 25", section 7: the varlen interface; LLM Infra Atlas, "FA2:
 * parallelism", section 2: split-KV for decode).
 *   k, v          [total_k, H_kv, d]  dtype, 16-byte aligned; sequence b owns
 *                 rows [cu_seqlens_k[b], cu_seqlens_k[b+1])
 *   cu_seqlens_k  [B + 1]  int32, device, 4-byte aligned
 * Query head h reads K/V head h / (H / H_kv).  The query row sees every key of
 * its sequence (bottom-right causal alignment puts a single query row after all
 * its keys, so causal and non-causal coincide).  Sequence b is split into
 * num_splits chunks of c_b = ceil(len_b / num_splits) keys as in
 * fa_fwd_splitkv_paged; the outputs are the partials of fa_fwd_splitkv with
 * Nq = 1 (o_part [num_splits, B, H, 1, d], lse_part [num_splits, B, H, 1]),
 * merged by fa_splitkv_combine.  A sequence of length 0 gives O = 0 and
 * LSE = -inf.  Requirements: H % H_kv == 0, num_splits >= 1,
 * 1 <= max_seqlen_k <= total_k.  The offsets live on the device and are not
 * read by the host: a sequence whose offsets leave [0, total_k], decrease or
 * span more than max_seqlen_k keys leaves its partials as the caller's buffers
 * held them; no memory outside the tensors is accessed.
 */
fa_status fa_fwd_splitkv_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens_k,
                                float* o_part, float* lse_part,
                                int B, int H, int H_kv, int total_k, int max_seqlen_k, int d,
                                float scale, int num_splits, fa_dtype dtype, void* stream);

/*
 * FP8 forward (Ringi, "Lecture 25", section 5.4: Q K^T and P V on FP8 operands
 * with per-block scale factors): O and LSE of attention on the dequantized
 * inputs x = code * descale, where
 *   q        [B, H, Nq, d]     e4m3 codes (OCP E4M3FN bytes), 16-byte aligned
 *   k, v     [B, H_kv, Nk, d]  e4m3 codes, 16-byte aligned
 *   q_descale [B, H, ceil(Nq / 128)]     fp32: one per 128 query rows
 *   k_descale [B, H_kv, ceil(Nk / 128)]  fp32: one per 128 keys
 *   v_descale [B, H_kv]                  fp32: one per K/V head
 *   o        [B, H, Nq, d]     bfloat16;  lse [B, H, Nq] fp32 (natural log of the
 *            scaled scores of the dequantized inputs)
 * Query head h reads K/V head h / (H / H_kv); causal alignment and scale as
 * fa_fwd.  P is rounded to e4m3 (after a per-row power-of-two lift that keeps
 * the largest weights at the top of the e4m3 range) before its product with V;
 * its row sum is kept in fp32.  d must be 128.  Descales must be finite and
 * positive (fa_quantize_fp8 produces them).
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                     const float* k_descale, const float* v_descale, void* o, float* lse,
                     int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale, void* stream);

/*
 * Block quantizer for fa_fwd_fp8's inputs (the per-block scale factors of
 * Ringi, "Lecture 25", section 5.4): x [G, N, d] fp16/bf16 -> codes [G, N, d]
 * (e4m3 bytes) and descale [G, ceil(N / block_rows)] fp32.  Per block of
 * block_rows rows: amax = max |x|; descale = amax / 448 (1 for an all-zero
 * block); code = the e4m3 value nearest x * (448 / amax) (fp32 arithmetic,
 * clamped to +-448, ties to even).  For fa_fwd_fp8 use block_rows = 128 for q
 * and k (G = B*H or B*H_kv) and block_rows = N for v.  d a multiple of 8; x and
 * codes 16-byte aligned.  Inputs must be finite.
 */
fa_status fa_quantize_fp8(const void* x, void* x8, float* descale, int G, int N, int d, int block_rows,
                          fa_dtype dtype, void* stream);

/*
 * Split-KV forward, second half: merge the partials with the online-softmax
 * identity (Ringi, Lecture 25, section 2.2).  Per row:
 *   M = max_s lse_part[s];  w_s = exp(lse_part[s] - M) (0 for -inf);
 *   o = sum_s w_s o_part[s] / sum_s w_s  (rounded to dtype);
 *   lse = M + ln sum_s w_s  (-inf, with o = 0, when every split is empty).
 * Splits are summed in index order, so the result is deterministic.
 */
fa_status fa_splitkv_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                             int B, int H, int Nq, int d, int num_splits,
                             fa_dtype dtype, void* stream);

/*
 * Bytes of fp32 workspace fa_bwd needs: B * H * Nq * 8 (two values per query
 * row).  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Nq);

/*
 * Backward pass: gradients dq, dk, dv ([B,H,N,d], dtype) of a loss whose
 * gradient with respect to o is dout, given the forward's inputs, its output o
 * and its lse.  P is recomputed tile by tile from the saved log-sum-exp instead
 * of being stored (Ringi, Lecture 25, section 3.3):
 *   dV = P^T dO;  dP = dO V^T;  dS = P o (dP - rowsum(dP o P));
 *   dQ = scale * dS K;  dK = scale * dS^T Q
 * rowsum(dP o P) equals rowsum(dO o O); the library computes it that way,
 * with lse rescaled to base 2, into `workspace` (fp32, at least
 * fa_bwd_workspace_bytes; its contents on entry do not matter).  dK and dV are accumulated per key block over the query tiles and
 * dQ per query block over the key tiles, so no atomics are used and the results
 * are deterministic (LLM Infra Atlas, FA2 parallelism, section 5).  Same
 * conventions as fa_fwd (causal alignment, scale, rounding); lse and workspace
 * must be 16-byte aligned.  A workspace smaller than required returns
 * FA_ERR_WORKSPACE.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 int B, int H, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype, void* stream);

/*
 * fa_bwd with K/V heads shared by groups of query heads (GQA; MQA when H_kv = 1):
 *   q, o, dout, dq  [B, H, Nq, d]      k, v, dk, dv  [B, H_kv, Nk, d]
 * Query head h reads K/V head h / (H / H_kv), as in fa_fwd_gqa (KingOfEgg, Flash
 * Attention (4), section 5: K/V index mapped by group).  A shared K/V head feeds
 * every query head of its group, so its dK and dV are the sums over that group
 * of the per-head gradients of fa_bwd; the library accumulates them in one pass
 * over the group's query tiles, in head order, without atomics (deterministic).
 * Workspace: fa_bwd_workspace_bytes(B, H, Nq).  H % H_kv must be 0, else
 * FA_ERR_SHAPE.  With H_kv = H this is fa_bwd.
 */
fa_status fa_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                     int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float scale, fa_dtype dtype,
                     void* stream);

/*
 * fa_bwd for packed variable-length sequences with grouped K/V heads: the
 * gradients of fa_fwd_varlen (same layouts, offsets and causal alignment; see
 * there), each sequence on its own rows (KingOfEgg, Flash Attention (4), section
 * 5: per-sequence offsets; Ringi, Lecture 25, section 3.3 for the gradients):
 *   q, o, dout, dq  [total_q, H, d]     dtype
 *   k, v, dk, dv    [total_k, H_kv, d]  dtype (dk, dv summed over each group)
 *   lse             [H, total_q]        float32, as fa_fwd_varlen wrote it
 * A query that sees no key gets dq = 0; a key that no query sees gets dk = dv = 0.
 * Workspace: fa_bwd_workspace_bytes(1, H, total_q) bytes, 16-byte aligned.
 * Requirements as fa_fwd_varlen, and H * d * 128 < 2^31.  The offsets are not
 * read by the host: a sequence whose offsets fall outside [0, total], decrease,
 * or span more than max_seqlen leaves its rows of dq, dk, dv as the caller's
 * buffers held them (not cleared, not reported) and no memory outside the
 * tensors is accessed.  Deterministic (no atomics).
 */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, void* workspace, size_t workspace_bytes, int B, int H, int H_kv,
                        int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d, int causal,
                        float scale, fa_dtype dtype, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_str(fa_status status);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that forbid hipMalloc, harnesses without an allocator):
 * fa_bwd_gqa without the workspace argument.  The D and lse-in-base-2 values
 * that fa_bwd_gqa keeps in the caller's workspace live instead in a scratch
 * array inside the library: FA_BWD_NOALLOC_MAX_ROWS query rows (B * H * Nq) at
 * 8 bytes each, 8 MiB, held on every GPU the library runs on until the process
 * ends.  The caller still passes every input and output; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine) and gives the
 * same results as fa_bwd_gqa bit for bit.  B * H * Nq above the maximum returns
 * FA_ERR_WORKSPACE before any HIP call.  The first call on a device looks up the
 * scratch array's address on that device (hipGetSymbolAddress; FA_ERR_HIP if
 * that fails).  Every call on one GPU uses that GPU's one array: calls that
 * overlap in time on one GPU (different streams, or host threads) race and
 * corrupt each other's gradients; calls enqueued on one stream are ordered and
 * safe.  Nothing in the array needs to start at zero: each call writes every
 * value it reads.  Other arguments and errors as fa_bwd_gqa.
 */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 20)

fa_status fa_bwd_gqa_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq,
                             int Nk, int d, int causal, float scale, fa_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
