/*
 * flashprefill.h -- C ABI of the MI355X (gfx950) FlashPrefill block-sparse
 * prefill-attention library (libflashprefill.so).
 *
 * The path has three calls, each one stage of the method:
 *   fp_discover            mean-pool Q and K per 128-token block
 *   fp_threshold_compact   pooled block scores, max-relative threshold with
 *                          sink / local-window blocks, ascending list compaction
 *   fp_sparse_attn         causal GQA flash attention over the listed blocks
 * plus fp_dense_attn (implicit full causal list, the same-GPU dense baseline)
 * and paged-KV / continuous-batching variants of each.
 *
 * Sources: "FlashPrefill: Near-Zero-Cost Sparsity Discovery for Ultra-Fast
 * Long-Context Prefilling" (zhichai.net), sections Method 1 (instantaneous
 * pattern discovery), 2 (dynamic threshold pruning), 3 (index compaction ->
 * physical jumps); "FlashPrefill V2: Block-Sparse Prefill Attention for
 * Long-Context LLM Serving" (shd-paper.top, English abstract): FP8 inference,
 * paged KV cache and continuous batching.
 *
 * Conventions shared by every call
 *   - Every tensor argument is a DEVICE pointer owned by the caller.  Nothing
 *     is allocated, freed or synchronised inside the library; each call only
 *     enqueues kernels on `stream` (a hipStream_t passed as void*, NULL = the
 *     default stream) and returns, so a sequence of calls on caller-owned
 *     buffers can be captured into a HIP graph and replayed.  There is no
 *     global mutable state apart from a thread-local error message, so calls
 *     from several host threads are safe.
 *   - Head dimension d and block size B must both be 128.  hq % hkv == 0;
 *     query head h reads KV head h / (hq / hkv).
 *   - Strides are in ELEMENTS; the innermost (head-dim) stride is 1.  Data
 *     pointers must be 16-byte aligned and the token/head/page strides must
 *     keep every 128-element head row 16-byte aligned.
 *   - dtype: FP_BF16 (bfloat16 inputs) or FP_FP8_E4M3 (OCP e4m3fn codes,
 *     max 448, with one fp32 scale per head: value = code * scale).  Scales
 *     are device arrays and must be finite and > 0.  Outputs are bf16.
 *   - Return value: FP_OK, or an error code.  All argument checks happen on
 *     the host before anything is enqueued; an error leaves every output
 *     untouched.  FP_EHIP reports a failed kernel launch.  No call aborts or
 *     throws.  fp_last_error() returns a description of the last failure on
 *     the calling thread.
 *   - nb = ceil(L / 128) blocks per sequence.  Lists are stored triangular-
 *     packed: the list of (query head h, query block i) of a single sequence
 *     starts at idx[h * nb*(nb+1)/2 + i*(i+1)/2] and holds counts[h*nb + i]
 *     ascending block ids; the last one is always i.
 *
 * Numerics
 *   - Pooled means are fp64.  Sums of up to 128 bf16 values (or e4m3 codes)
 *     are exact in fp64, so the means are the exact means rounded once.
 *   - Block scores are fp64; the threshold test is s_ij - max_j s_ij >= ln(alpha)
 *     (alpha = 0 keeps every causal block).
 *   - Attention: MFMA products with fp32 accumulation, fp32 online softmax,
 *     probabilities rounded to bf16 (bf16 path) or e4m3 (fp8 path) for the
 *     P*V product, bf16 output, optional fp32 log-sum-exp (natural log).
 */
#ifndef FLASHPREFILL_H
#define FLASHPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp_status {
  FP_OK = 0,
  FP_EINVAL = 1,        /* invalid argument (null pointer, bad size, stride, alignment, alpha) */
  FP_EUNSUPPORTED = 2,  /* valid but not supported here (d != 128, B != 128, unknown dtype)  */
  FP_EHIP = 3           /* a HIP runtime call or kernel launch failed                        */
};

enum fp_dtype {
  FP_BF16 = 0,
  FP_FP8_E4M3 = 1       /* OCP e4m3fn codes + fp32 per-head scales */
};

/* Human-readable name of a status code (static string). */
const char* fp_status_string(int status);
/* Description of the last error returned on this host thread ("" if none). */
const char* fp_last_error(void);
/* Library ABI version (increments on any signature change; this header: 4). */
int fp_abi_version(void);

/* Host helpers: number of blocks ceil(L / block), and the idx capacity in
 * int32 elements for one sequence: hq * nb * (nb + 1) / 2. */
int64_t fp_num_blocks(int64_t L, int block);
int64_t fp_idx_capacity(int hq, int64_t nb);

/* ---------------------------------------------------------------------------
 * fp_discover -- block mean pooling of Q and K (Method 1: each block of B
 * tokens is represented by the mean of its vectors; "mean-proxy").
 *
 *   q          [L, hq, d] at q + t*q_stride_tok + h*q_stride_head
 *   k          [L, hkv, d] likewise
 *   q_scale    fp8 only: [hq] fp32 (ignored for bf16, may be NULL)
 *   k_scale    fp8 only: [hkv] fp32
 *   pooled_q   out [hq, nb, d] fp64, contiguous: mean of the block's tokens
 *   pooled_k   out [hkv, nb, d] fp64, contiguous
 * A partial last block is averaged over its valid tokens.
 * ------------------------------------------------------------------------- */
int fp_discover(const void* q, const void* k, int dtype,
                const float* q_scale, const float* k_scale,
                int L, int hq, int hkv, int d, int block,
                int64_t q_stride_tok, int64_t q_stride_head,
                int64_t k_stride_tok, int64_t k_stride_head,
                double* pooled_q, double* pooled_k, void* stream);

/* ---------------------------------------------------------------------------
 * fp_threshold_compact -- pooled block scores, dynamic threshold and index
 * compaction (Methods 1-3).
 *
 *   s_ij  = softmax_scale * pooled_q[h, i] . pooled_k[h / (hq/hkv), j],  j <= i
 *   keep  = (s_ij - max_{j'<=i} s_ij' >= ln(alpha))      threshold alpha x row max
 *           or j < n_sink                                  attention sinks
 *           or j > i - n_local                             local window (diagonal incl.)
 *   idx    out: ascending kept j per (h, i), triangular-packed (see above);
 *          capacity fp_idx_capacity(hq, nb) int32
 *   counts out: [hq, nb] int32 list lengths (>= 1)
 *   scores optional debug output, NULL to skip: [hq, nb, nb] fp64, 8-byte
 *          aligned; s_ij is written for j <= i, entries j > i are not touched
 *
 * alpha must be finite and >= 0 (alpha = 0 keeps every causal block, alpha > 1
 * keeps only the forced blocks); n_sink >= 0; n_local >= 1.  softmax_scale
 * must be finite and > 0 (normally 1/sqrt(d)).
 * ------------------------------------------------------------------------- */
int fp_threshold_compact(const double* pooled_q, const double* pooled_k,
                         int nb, int hq, int hkv, int d,
                         double softmax_scale, double alpha, int n_sink, int n_local,
                         int32_t* idx, int32_t* counts, double* scores, void* stream);

/* ---------------------------------------------------------------------------
 * fp_sparse_attn -- causal GQA block-sparse flash attention (Method 3: the
 * inner loop visits only the listed key blocks, "physical jumps").
 *
 *   O[t, h] = sum_{c in C(t)} softmax_c(softmax_scale * q_t . k_c) v_c,
 *   C(t)    = { c <= t : c / B in list(h, t / B) }.
 *
 *   q, o       [L, hq, d];  k, v [L, hkv, d]  (strided as in fp_discover)
 *   idx/counts the lists from fp_threshold_compact (each list ascending, each
 *              id in [0, i], ending with i)
 *   v_scale    fp8 only: [hkv] fp32
 *   out        bf16 [L, hq, d] at out + t*o_stride_tok + h*o_stride_head
 *   lse        optional (NULL = skip): fp32 [hq, L], natural-log log-sum-exp of
 *              the scaled logits of each query row
 * ------------------------------------------------------------------------- */
int fp_sparse_attn(const void* q, const void* k, const void* v, int dtype,
                   const float* q_scale, const float* k_scale, const float* v_scale,
                   int L, int hq, int hkv, int d, int block,
                   int64_t q_stride_tok, int64_t q_stride_head,
                   int64_t k_stride_tok, int64_t k_stride_head,
                   int64_t v_stride_tok, int64_t v_stride_head,
                   int64_t o_stride_tok, int64_t o_stride_head,
                   const int32_t* idx, const int32_t* counts, float softmax_scale,
                   void* out, float* lse, void* stream);

/* fp_dense_attn -- the same kernel with the implicit full causal list
 * {0..i} for every query block: plain causal GQA attention.  Arguments as in
 * fp_sparse_attn without idx/counts. */
int fp_dense_attn(const void* q, const void* k, const void* v, int dtype,
                  const float* q_scale, const float* k_scale, const float* v_scale,
                  int L, int hq, int hkv, int d, int block,
                  int64_t q_stride_tok, int64_t q_stride_head,
                  int64_t k_stride_tok, int64_t k_stride_head,
                  int64_t v_stride_tok, int64_t v_stride_head,
                  int64_t o_stride_tok, int64_t o_stride_head,
                  float softmax_scale, void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Logical-skip ablation.  FlashPrefill Method 3 ("Index Compaction -> Physical
 * Jumps") contrasts a loop over every block that tests a mask with the compacted
 * lists the kernel above walks.  These two calls give the mask form of the same
 * decisions and the masked loop, so the two can be timed side by side.  Single
 * sequence, packed K/V.
 *
 * fp_mask_words -- 32-bit words per mask row: ceil(nb / 32).
 *
 * fp_threshold_mask -- the decisions of fp_threshold_compact as a bit-packed
 *   block mask instead of lists:
 *   mask   out uint32 [hq, nb, fp_mask_words(nb)], 4-byte aligned; bit (j % 32)
 *          of word [h, i, j / 32] is keep(h, i, j).  Words that cover some
 *          j <= i are written (their bits for j > i are 0); the others are not
 *          touched.
 *   Other arguments and checks as in fp_threshold_compact.
 *
 * fp_sparse_attn_masked -- fp_sparse_attn driven by that mask: the key-block
 *   loop runs over every j <= i and branches past blocks whose bit is 0, and
 *   the causal mask applies to block i.  It visits the same blocks in the same
 *   order as fp_sparse_attn on lists of the same decisions, so the outputs are
 *   bit-identical.  A row without any set bit gives NaN output.  Other
 *   arguments as in fp_sparse_attn.
 * ------------------------------------------------------------------------- */
int fp_mask_words(int64_t nb);

int fp_threshold_mask(const double* pooled_q, const double* pooled_k,
                      int nb, int hq, int hkv, int d,
                      double softmax_scale, double alpha, int n_sink, int n_local,
                      uint32_t* mask, void* stream);

int fp_sparse_attn_masked(const void* q, const void* k, const void* v, int dtype,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          int L, int hq, int hkv, int d, int block,
                          int64_t q_stride_tok, int64_t q_stride_head,
                          int64_t k_stride_tok, int64_t k_stride_head,
                          int64_t v_stride_tok, int64_t v_stride_head,
                          int64_t o_stride_tok, int64_t o_stride_head,
                          const uint32_t* mask, float softmax_scale,
                          void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * fp_pool -- block mean pooling of any tensor x [L, H, d] (as fp_discover does
 * for Q and K): pooled [H, nb, d] fp64, fp8 inputs scaled per head.  Used to pool
 * V for the mean correction below.
 * ------------------------------------------------------------------------- */
int fp_pool(const void* x, int dtype, const float* scale, int L, int H, int d, int block,
            int64_t stride_tok, int64_t stride_head, double* pooled, void* stream);

/* ---------------------------------------------------------------------------
 * fp_mean_correct -- the FlashPrefill V2 "mean correction term", which the V2
 * abstract names without defining.  This is an ASSUMPTION, off unless called:
 * every causal key block that the list of (h, i) prunes (all lie below the
 * diagonal) still enters the softmax as 128 copies of its mean key with its mean
 * value:
 *     O' = (Z O + sum_j 128 e^{s_j} vbar_j) / (Z + sum_j 128 e^{s_j}),
 *     s_j = softmax_scale * q . kbar_j,  Z = e^{LSE},
 * applied in place to the output and LSE of an fp_sparse_attn call.
 *   pooled_k   [hkv, nb, d] fp64 (from fp_discover)
 *   pooled_v   [hkv, nb, d] fp64 (from fp_pool on V)
 *   idx/counts the per-head lists the sparse call used
 *   out, lse   in: the sparse output and LSE; out: corrected (rows with
 *              nothing pruned are left untouched)
 *   workspace  caller-owned device scratch of at least
 *              fp_mean_correct_workspace_bytes(L, hkv) bytes (16-byte aligned;
 *              3 MB at L = 128K, hkv = 4): the means converted once per KV head
 *              into bf16 tile images.  Its contents are overwritten; calls that
 *              share one workspace must not overlap.  NULL, misaligned or too
 *              small: FP_EINVAL.
 * Single sequence of at most 65536 blocks (longer: FP_EUNSUPPORTED); pooled
 * K/V 16-byte aligned (else FP_EINVAL).  Numerics: logits from the fp64 means
 * split into two bf16 terms (~2^-17 relative), the correction's values and
 * weights in bf16 with fp32 accumulation.  Other arguments as in fp_sparse_attn.
 * ------------------------------------------------------------------------- */
int fp_mean_correct(const void* q, int dtype, const float* q_scale,
                    const double* pooled_k, const double* pooled_v,
                    int L, int hq, int hkv, int d, int block,
                    int64_t q_stride_tok, int64_t q_stride_head,
                    int64_t o_stride_tok, int64_t o_stride_head,
                    const int32_t* idx, const int32_t* counts, float softmax_scale,
                    void* out, float* lse, void* workspace, int64_t workspace_bytes,
                    void* stream);

/* Workspace bytes fp_mean_correct needs for L tokens and hkv KV heads
 * (-1 for L < 0 or hkv < 1).  Host only. */
int64_t fp_mean_correct_workspace_bytes(int L, int hkv);

/* ---------------------------------------------------------------------------
 * fp_mean_correct_varlen -- fp_mean_correct over a packed batch (the serving
 * workload of the FlashPrefill V2 abstract: paged KV cache, continuous
 * batching), applied to every sequence on its own.  Same assumption, off unless
 * called.
 *   q          packed [total_tokens, hq, d]; sequence s owns tokens
 *              cu_seqlens[s] .. cu_seqlens[s+1]-1 (device int32 [n_seqs+1])
 *   pooled_k/v [hkv, total_blocks, d] fp64, sequence s's blocks starting at
 *              sum_{r<s} ceil(len_r/128) (as fp_discover_paged / fp_pool_varlen
 *              write them)
 *   idx/counts the lists of fp_threshold_compact_varlen
 *   out, lse   packed [total_tokens, hq, d] / [hq, total_tokens], in place
 *   workspace  fp_mean_correct_varlen_workspace_bytes(total_blocks, n_seqs, hkv)
 *              bytes, 16-byte aligned (NULL, misaligned or short: FP_EINVAL)
 * Sequences of at most 65536 blocks.  Other arguments and errors as
 * fp_mean_correct and fp_sparse_attn_paged.
 * ------------------------------------------------------------------------- */
int fp_mean_correct_varlen(const void* q, int dtype, const float* q_scale,
                           const double* pooled_k, const double* pooled_v,
                           const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                           int64_t total_tokens, int64_t total_blocks, int64_t total_tri,
                           int hq, int hkv, int d, int block,
                           int64_t q_stride_tok, int64_t q_stride_head,
                           int64_t o_stride_tok, int64_t o_stride_head,
                           const int32_t* idx, const int32_t* counts, float softmax_scale,
                           void* out, float* lse, void* workspace, int64_t workspace_bytes,
                           void* stream);

/* Workspace bytes fp_mean_correct_varlen needs (an upper bound: hkv tile images of
 * 24 KB per 32 blocks of every sequence, i.e. hkv * (ceil(total_blocks/32) +
 * n_seqs) * 24576); -1 for negative sizes.  Host only. */
int64_t fp_mean_correct_varlen_workspace_bytes(int64_t total_blocks, int n_seqs, int hkv);

/* fp_pool over a packed batch: per-sequence block means of x, packed
 * [total_tokens, H, d] (page_table NULL) or a page cache [num_pages, 128, H, d]
 * through page_table [n_seqs, max_pages] -> pooled [H, total_blocks, d] fp64
 * (sequence s's blocks starting at sum_{r<s} ceil(len_r/128); a partial last
 * block is averaged over its valid rows).  Used to pool V for
 * fp_mean_correct_varlen.  Arguments and errors as fp_discover_paged. */
int fp_pool_varlen(const void* x, int dtype, const float* scale,
                   const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                   int64_t total_tokens, int64_t total_blocks,
                   const int32_t* page_table, int max_pages, int num_pages,
                   int H, int d, int block,
                   int64_t stride_page, int64_t stride_tok, int64_t stride_head,
                   double* pooled, void* stream);

/* ---------------------------------------------------------------------------
 * fp_mean_correct_noalloc -- fp_mean_correct for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same pass with its scratch taken from a static
 * buffer inside the library instead of a caller workspace.  Nothing is
 * allocated or freed by the call.
 *   Limit: the scratch holds 8 MiB (8388608 bytes) per GPU, i.e. calls with
 *   fp_mean_correct_workspace_bytes(L, hkv) <= 8388608 (e.g. hkv = 4 up to
 *   348K tokens, hkv = 8 up to 174K); larger calls return FP_EUNSUPPORTED with
 *   the sizes in fp_last_error() and enqueue nothing.
 *   Sharing: every call on one GPU uses that GPU's single scratch buffer, which
 *   keeps the last call's contents; the pass rewrites every byte it reads, so
 *   nothing needs clearing, but calls that overlap on one GPU (concurrent
 *   streams or host threads) race and must be serialised by the caller.
 *   The buffer lives in the library's device code on every GPU it runs on until
 *   the process ends.  Other arguments, numerics and errors as fp_mean_correct.
 * ------------------------------------------------------------------------- */
int fp_mean_correct_noalloc(const void* q, int dtype, const float* q_scale,
                            const double* pooled_k, const double* pooled_v,
                            int L, int hq, int hkv, int d, int block,
                            int64_t q_stride_tok, int64_t q_stride_head,
                            int64_t o_stride_tok, int64_t o_stride_head,
                            const int32_t* idx, const int32_t* counts, float softmax_scale,
                            void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Group-shared lists (a PackGQA-style mode beyond the pages' per-head
 * selection): one list per KV-head group, the union of the lists of its
 * hq/hkv query heads, so every head of a group visits the same key blocks in
 * the same order and the group's K/V tiles are shared in cache.  Each head
 * attends over a superset of its own list.  Single sequence, packed K/V.
 *
 * fp_union_compact -- from the per-head masks of fp_threshold_mask:
 *   mask   [hq, nb, fp_mask_words(nb)] (only bits j <= i of row i are read)
 *   idx    out: ascending union of the group's lists per (g, i),
 *          triangular-packed per group (row i of group g at
 *          g*nb(nb+1)/2 + i(i+1)/2); capacity fp_idx_capacity(hkv, nb)
 *   counts out: [hkv, nb] int32
 *
 * fp_sparse_attn_grouped -- fp_sparse_attn with idx/counts holding one list
 *   per KV group (from fp_union_compact): query head h reads the list of
 *   group h / (hq / hkv).  Other arguments as in fp_sparse_attn.
 * ------------------------------------------------------------------------- */
int fp_union_compact(const uint32_t* mask, int nb, int hq, int hkv,
                     int32_t* idx, int32_t* counts, void* stream);

int fp_sparse_attn_grouped(const void* q, const void* k, const void* v, int dtype,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           int L, int hq, int hkv, int d, int block,
                           int64_t q_stride_tok, int64_t q_stride_head,
                           int64_t k_stride_tok, int64_t k_stride_head,
                           int64_t v_stride_tok, int64_t v_stride_head,
                           int64_t o_stride_tok, int64_t o_stride_head,
                           const int32_t* idx, const int32_t* counts, float softmax_scale,
                           void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Continuous batching and paged KV (V2 abstract: native paged KV cache and
 * continuous batching).  A batch of n_seqs sequences is packed token-major:
 *
 *   cu_seqlens  device int32 [n_seqs + 1], cu_seqlens[0] = 0, non-decreasing,
 *               cu_seqlens[n_seqs] = total_tokens; sequence s owns tokens
 *               cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed Q (and of the
 *               packed K/V when page_table is NULL).  Queries and keys of a
 *               sequence both start at its token 0 (prefill).
 *   max_seqlen  host int >= every sequence length (sizes the launch grid).
 *   Blocks: nb_s = ceil(len_s / B); block i of sequence s has packed block id
 *               cu_blocks[s] + i with cu_blocks[s] = sum_{r<s} nb_r, and
 *               total_blocks = sum_s nb_s.
 *   Lists:  the list of (h, s, i) starts at
 *               idx[h * total_tri + cu_tri[s] + i*(i+1)/2]
 *           with cu_tri[s] = sum_{r<s} nb_r*(nb_r+1)/2, total_tri = sum_s
 *           nb_s*(nb_s+1)/2; counts are [hq, total_blocks].
 *   Paging: when page_table is non-NULL, K and V are caches of 128-token pages
 *           [num_pages, 128, hkv, d] addressed by (page, row, head) strides,
 *           and logical block j of sequence s lives in page
 *           page_table[s * max_pages + j].  A page id outside [0, num_pages)
 *           is never dereferenced; the outputs that depend on it are NaN.
 *           When page_table is NULL, K and V are packed [total_tokens, hkv, d]
 *           like Q (the stride_page arguments are ignored).
 * The host cannot see device metadata: total_tokens / total_blocks / total_tri
 * are the caller's declared extents and kernels never access beyond them.
 * ------------------------------------------------------------------------- */
int fp_discover_paged(const void* q, const void* k, int dtype,
                      const float* q_scale, const float* k_scale,
                      const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                      int64_t total_tokens, int64_t total_blocks,
                      const int32_t* page_table, int max_pages, int num_pages,
                      int hq, int hkv, int d, int block,
                      int64_t q_stride_tok, int64_t q_stride_head,
                      int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                      double* pooled_q, double* pooled_k, void* stream);

int fp_threshold_compact_varlen(const double* pooled_q, const double* pooled_k,
                                const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                                int64_t total_blocks, int64_t total_tri,
                                int hq, int hkv, int d,
                                double softmax_scale, double alpha, int n_sink, int n_local,
                                int32_t* idx, int32_t* counts, void* stream);

/* idx == NULL and counts == NULL selects the implicit full causal list (dense). */
int fp_sparse_attn_paged(const void* q, const void* k, const void* v, int dtype,
                         const float* q_scale, const float* k_scale, const float* v_scale,
                         const int32_t* cu_seqlens, int n_seqs, int max_seqlen,
                         int64_t total_tokens, int64_t total_blocks, int64_t total_tri,
                         const int32_t* page_table, int max_pages, int num_pages,
                         int hq, int hkv, int d, int block,
                         int64_t q_stride_tok, int64_t q_stride_head,
                         int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                         int64_t v_stride_page, int64_t v_stride_tok, int64_t v_stride_head,
                         int64_t o_stride_tok, int64_t o_stride_head,
                         const int32_t* idx, const int32_t* counts, float softmax_scale,
                         void* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Chunked / prefix-cached prefill.  Each sequence brings len_q new query tokens
 * against a K/V cache of len_k >= len_q tokens that already holds them (the
 * prefix plus this chunk): query t of the sequence sits at absolute position
 * len_k - len_q + t and attends causally to keys 0 .. that position (the
 * causal mask is aligned to the bottom-right corner).  With len_q = len_k this is
 * the prefill above.
 *
 *   cu_seqlens_q  device int32 [n_seqs + 1]: query lengths, packed Q / out / LSE
 *   cu_seqlens_k  device int32 [n_seqs + 1]: key lengths, packed K/V when
 *                 page_table is NULL (else K/V pages as in the paged calls)
 *   max_seqlen_q/k  host bounds on the lengths (size the launch grids)
 *   total_q/total_k packed token extents
 *   Query blocks follow absolute positions: block I holds positions
 *   128I .. 128I+127, so a chunk that starts inside a block has a partial first
 *   query block.  Sequence s has nq_s query blocks I0_s .. I0_s+nq_s-1 (I0_s =
 *   (len_k - len_q) / 128) and nk_s = ceil(len_k / 128) key blocks.
 *   pooled_q   [hq, total_qblocks, d], total_qblocks = sum_s nq_s, sequences in
 *              order; a query block is the mean of the chunk's tokens in it
 *   pooled_k   [hkv, total_kblocks, d], total_kblocks = sum_s nk_s
 *   idx        list row of (h, s, I) at h*total_tri + tri_s + (I-I0_s)(I0_s+1)
 *              + (I-I0_s)(I-I0_s-1)/2 with tri_s = sum over earlier sequences of
 *              nq(I0+1) + nq(nq-1)/2 (row I has I+1 slots); total_tri = that sum
 *              over all sequences
 *   counts     [hq, total_qblocks] int32
 *   out, lse   [total_q, hq, d] bf16, [hq, total_q] fp32
 * Selection rules, dtypes and error behaviour as in the calls above; query
 * lengths above the key length are clamped to it.
 * ------------------------------------------------------------------------- */
int fp_discover_chunked(const void* q, const void* k, int dtype,
                        const float* q_scale, const float* k_scale,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seqs,
                        int max_seqlen_q, int max_seqlen_k, int64_t total_q, int64_t total_k,
                        int64_t total_qblocks, int64_t total_kblocks,
                        const int32_t* page_table, int max_pages, int num_pages,
                        int hq, int hkv, int d, int block,
                        int64_t q_stride_tok, int64_t q_stride_head,
                        int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                        double* pooled_q, double* pooled_k, void* stream);

int fp_threshold_compact_chunked(const double* pooled_q, const double* pooled_k,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seqs,
                                 int max_seqlen_q, int max_seqlen_k,
                                 int64_t total_qblocks, int64_t total_kblocks, int64_t total_tri,
                                 int hq, int hkv, int d,
                                 double softmax_scale, double alpha, int n_sink, int n_local,
                                 int32_t* idx, int32_t* counts, void* stream);

int fp_sparse_attn_chunked(const void* q, const void* k, const void* v, int dtype,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seqs,
                           int max_seqlen_q, int max_seqlen_k, int64_t total_q, int64_t total_k,
                           int64_t total_qblocks, int64_t total_kblocks, int64_t total_tri,
                           const int32_t* page_table, int max_pages, int num_pages,
                           int hq, int hkv, int d, int block,
                           int64_t q_stride_tok, int64_t q_stride_head,
                           int64_t k_stride_page, int64_t k_stride_tok, int64_t k_stride_head,
                           int64_t v_stride_page, int64_t v_stride_tok, int64_t v_stride_head,
                           int64_t o_stride_tok, int64_t o_stride_head,
                           const int32_t* idx, const int32_t* counts, float softmax_scale,
                           void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHPREFILL_H */
