/*
 * cosa.h - C ABI of libcosa: CoSA block-sparse causal prefill attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one summarised on the gist.science pages "CoSA:
 * Accelerating Long-Context Inference via Proxy-Kernel Co-Designed Sparse
 * Attention" (technical summary). Stage 1, the Kernel-Aware Proxy (KAP, §2.2),
 * turns downsampled query/key scores into a per-query-block computation-order
 * list; stage 2, the Ordered-Skipping Kernel (OSK, §2.3), runs online-softmax
 * attention over the listed KV pages in that order and skips, in-kernel,
 * blocks whose local maxima sit far below the running maxima.
 *
 * General rules for every entry point:
 *  - Pointers named in a cosa_problem and every tensor argument are DEVICE
 *    pointers unless the name starts with "host_". The caller owns all
 *    memory; the library allocates nothing and keeps no pointer after return.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns without synchronising. No device-to-host copy is made.
 *  - Arguments are validated on the host before any HIP call. A rejected call
 *    returns COSA_ERR_INVALID_ARG or COSA_ERR_UNSUPPORTED and enqueues
 *    nothing; cosa_last_error() then names the offending argument. A failed
 *    kernel launch returns COSA_ERR_HIP.
 *  - Results are deterministic: the same inputs give bitwise-identical
 *    outputs from run to run (no atomics in any accumulation).
 *  - Calls are reentrant; the error message is thread-local.
 *
 * Layouts (element counts, row-major):
 *  q, o        [total_q, h_q, head_dim]   sequences packed back to back;
 *              sequence b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 *              Element (t, h, c) of q sits at q + t*q_stride_tok +
 *              h*q_stride_head + c (likewise o with the o_ strides), so q may
 *              be a view into a larger tensor, e.g. the query part of a fused
 *              QKV projection, read in place (zero-copy access to the
 *              caller's tensors, CompactAttention page, execution stage).
 *              head_dim is always contiguous. Every other tensor argument is
 *              contiguous in the layout stated for it.
 *  k/v pages   [num_pages, h_kv, block, head_dim]: KV-head-major pages, one
 *              page per (logical KV block) so each (page, KV head) slab is
 *              contiguous (layout of the CompactAttention page, execution
 *              stage). block_table[b * max_blocks_k + kb] names the page that
 *              holds keys kb*block .. kb*block+block-1 of sequence b. Key slots
 *              past a sequence's end may hold anything (even NaN): they are
 *              never used.
 *  Causality: sequence b has Lq = cu_seqlens_q[b+1]-cu_seqlens_q[b] queries
 *  and Lk = seqlens_k[b] >= Lq keys. Local query i sits at absolute position
 *  off + i, off = Lk - Lq (a prefill chunk attending to the KV cache that
 *  already holds it), and sees keys j <= off + i.
 *  Blocks: query block qb holds local rows qb*block .. qb*block+block-1; KV
 *  block kb is causal for qb when kb*block <= off + min(qb*block+block-1,
 *  Lq-1); the causal blocks of qb are kb = 0 .. n(qb)-1.
 */
#ifndef COSA_H
#define COSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cosa_status {
  COSA_OK = 0,
  COSA_ERR_INVALID_ARG = -1, /* argument out of its documented domain       */
  COSA_ERR_UNSUPPORTED = -2, /* valid, but a size this build does not handle */
  COSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  COSA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed  */
} cosa_status;

typedef enum cosa_dtype { COSA_F32 = 0, COSA_BF16 = 1 } cosa_dtype;

/* Shape and metadata of one packed prefill batch. */
typedef struct cosa_problem {
  int32_t batch;       /* number of sequences, >= 1                          */
  int32_t h_q;         /* query heads, >= 1                                  */
  int32_t h_kv;        /* KV heads, >= 1, divides h_q (GQA group G=h_q/h_kv) */
  int32_t head_dim;    /* 64 or 128                                          */
  int32_t block;       /* B: query-block rows = KV-block keys = page size;
                          64 or 128                                          */
  int32_t dtype;       /* cosa_dtype of q, k/v pages and o                   */
  float softmax_scale; /* > 0, usually 1/sqrt(head_dim)                      */
  int32_t num_pages;   /* pages in the k/v pools                             */
  int32_t max_blocks_k;/* row length of block_table (>= ceil(Lk/B) for all b)*/
  const int32_t* cu_seqlens_q;      /* device [batch+1], cu[0]=0, nondecreasing */
  const int32_t* seqlens_k;         /* device [batch]                          */
  const int32_t* block_table;       /* device [batch, max_blocks_k], entries
                                       in [0, num_pages)                       */
  const int32_t* host_cu_seqlens_q; /* host copy of cu_seqlens_q              */
  const int32_t* host_seqlens_k;    /* host copy of seqlens_k                  */
  /* Element strides of q and o between consecutive tokens and heads; 0 takes
   * the contiguous value (tok: h_q*head_dim, head: head_dim). Each must be
   * >= 0 and a multiple of 16 bytes (8 bf16 or 4 fp32 elements), and the q
   * and o pointers 16-byte aligned (COSA_ERR_INVALID_ARG otherwise). The o
   * strides must not make two output elements share memory: the smaller
   * stride (with more than one token or head along it) is >= head_dim and
   * the larger >= the smaller times that extent. q may alias itself freely
   * (it is only read). */
  int64_t q_stride_tok, q_stride_head;
  int64_t o_stride_tok, o_stride_head;
} cosa_problem;

/* Padded extents derived from a problem (see cosa_dims). */
typedef struct cosa_dims_t {
  int32_t total_q; /* cu_seqlens_q[batch]                                   */
  int32_t max_nq;  /* max_b ceil(Lq_b / B): query blocks per sequence (padded)*/
  int32_t max_nk;  /* max_b ceil(Lk_b / B): KV blocks per sequence (padded)    */
  int32_t max_nr;  /* max_b ceil(Lq_b / pool): pooled query rows (padded)      */
  int32_t kmax;    /* widest order list under `budget` (closed form, >= 1)     */
} cosa_dims_t;

/* Host-only check of a problem (no HIP call, usable without a GPU).
 * Returns COSA_OK or the reason it was rejected. */
cosa_status cosa_validate(const cosa_problem* problem);

/* Host-only: padded extents for this problem, pool factor and budget.
 * kmax = max over rows of k(qb) = clamp(ceil(budget*n(qb) - 1e-9), 1, n(qb)),
 * evaluated in IEEE double (the budget rule of the CoSA summary §2.2, read
 * as a per-row fraction of the causal blocks). pool may be 0 when only the
 * attention extents are needed (max_nr is then 0); budget may be 0 for the
 * same purpose (kmax is then 0). */
cosa_status cosa_dims(const cosa_problem* problem, int32_t pool, double budget,
                      cosa_dims_t* out /* host */);

/* Host-only: width of the proxy's order lists under `budget` in (0, 1]
 * (cosa_dims(problem, 0, budget).kmax); 0 for an invalid problem or budget. */
size_t cosa_kap_kmax(const cosa_problem* problem, double budget);

/* Bytes of device workspace cosa_kap_order needs; `with_scores` = 0 when the
 * caller passes its own proxy_scores buffer (the scores then live there).
 * Returns 0 for an invalid problem or pool. */
size_t cosa_kap_workspace_size(const cosa_problem* problem, int32_t pool, int32_t with_scores);

/* Stage 1, Kernel-Aware Proxy (CoSA summary §2.2: block ranking, HRM flag
 * generation, flag-grouped sorting; §2.1: the output prescribes an order).
 *
 *  pool    p: tokens per pooled vector, 1 <= p <= B and p divides B. Q and K
 *          are mean-pooled over p consecutive tokens (a ragged last window
 *          averages the tokens that exist).
 *  budget  beta in (0, 1]: each row keeps k(qb) of its n(qb) causal blocks.
 *  Proxy scores: P[b,h,r,kb] = max over the pooled keys j of block kb that
 *          pooled row r may see (j*p <= off + min(r*p+p-1, Lq-1)) of
 *          softmax_scale * qpool[r,h] . kpool[j, h/G]; -inf when none.
 *  MaxNorm: c = exp32(P - rowmax(P)) (fp32, see below).
 *  HRM:    block kb is flagged for (b, g, qb) when P[b,h,r,kb] equals the
 *          row max for some pooled row r of qb and some query head h of KV
 *          group g.
 *  Score:  s[b,g,qb,kb] = sum of c over the group's heads (ascending), then
 *          qb's pooled rows (ascending), one rounded fp32 add at a time.
 *  Order:  the causal blocks of the row sorted by (HRM first, s descending,
 *          kb ascending), truncated to the first k(qb).
 *  exp32(x): 0 unless x >= -87; t = x*fp32(log2 e); n = rint(t) (ties even);
 *          f = t-n; Horner p = c7, p = f*p + c_k (k=6..0) with
 *          c_k = fp32(ln2^k/k!); result p*2^n. Every * and + is one fp32
 *          operation, never fused. Given the same fp32 P, order, hrm and s
 *          are reproducible bit for bit on any IEEE machine.
 *
 * Outputs (device):
 *  order        int32 [batch, h_kv, max_nq, kmax]: listed KV blocks, -1 pad.
 *  hrm          uint8 [batch, h_kv, max_nq, kmax]: 1 where the listed block
 *               is an HRM block, 0 otherwise and in the padding.
 *  count        int32 [batch, h_kv, max_nq]: k(qb); 0 for qb past a
 *               sequence's last query block.
 *  kmax         the caller's list width; must be >= cosa_dims().kmax.
 *  proxy_scores nullable fp32 [batch, h_q, max_nr, max_nk]: P, with -inf in
 *               every padding or non-visible entry.
 *  block_scores nullable fp32 [batch, h_kv, max_nq, max_nk]: s for
 *               kb < n(qb), 0 elsewhere.
 *  workspace    device scratch of cosa_kap_workspace_size(problem, pool,
 *               proxy_scores == NULL) bytes, 256-byte aligned; its contents
 *               on entry do not matter.
 * Limits: max_nk <= 4096 (COSA_ERR_UNSUPPORTED beyond). */
cosa_status cosa_kap_order(const cosa_problem* problem, const void* q, const void* k_pages,
                           int32_t pool, double budget, int32_t* order, uint8_t* hrm,
                           int32_t* count, int32_t kmax, float* proxy_scores,
                           float* block_scores, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Stage 2, Ordered-Skipping Kernel (CoSA summary §2.3: mask-skipped pages are
 * never touched, retained blocks may be skipped in-kernel, the rest is
 * computed; §1 for the per-tile veto).
 *
 * For each (b, query head h, qb) the kernel walks t = 0 .. count[b,g,qb]-1
 * over the list of KV group g = h / group, gathers page
 * block_table[b, order[b,g,qb,t]] in place and computes the scaled scores of
 * all valid rows of qb against its visible keys. With skip_threshold tau in
 * (0, 1) the block is skipped when, for every valid row i with a visible key
 * in it, m_loc_i - m_i < ln(tau) (m_loc_i its max scaled score in the block,
 * m_i the running max before the block, -inf before any block); a skipped
 * block leaves the running max, sum and accumulator unchanged. Otherwise the
 * online-softmax update runs and the P.V product is accumulated. tau = 0
 * never skips. O = acc / sum per row (0 for a row that saw no key).
 *
 *  order, count  as written by cosa_kap_order (any list of distinct causal
 *                blocks is accepted; an entry that is not a causal block of
 *                its row makes that row's output NaN).
 *  group         must equal h_q / h_kv.
 *  o             [total_q, h_q, head_dim] in the problem's dtype.
 *  visited       int32 [batch, h_q, max_nq]: listed blocks walked (= count).
 *  skipped       int32 [batch, h_q, max_nq]: blocks skipped in-kernel.
 *  skip_bits     nullable uint8 [batch, h_q, max_nq, kmax]: 0 computed,
 *                1 skipped, 255 padding.
 *  lse           nullable fp32 [h_q, total_q]: natural-log sum-exp of the
 *                computed scores of each row (-inf for a row that saw none).
 * For qb past a sequence's end, visited and skipped are 0 and skip_bits 255. */
cosa_status cosa_osk_attention(const cosa_problem* problem, const void* q, const void* k_pages,
                               const void* v_pages, const int32_t* order, const int32_t* count,
                               int32_t kmax, int32_t group, float skip_threshold, void* o,
                               int32_t* visited, int32_t* skipped, uint8_t* skip_bits, float* lse,
                               void* stream);

/* Dense causal softmax attention, the baseline of the CoSA summary §4: the
 * same tile engine walking every causal block of each row in ascending order,
 * with no list and no skip test. o and lse as in cosa_osk_attention. */
cosa_status cosa_dense_attention(const cosa_problem* problem, const void* q, const void* k_pages,
                                 const void* v_pages, void* o, float* lse, void* stream);

/* ---- Pooled keys kept across calls (decode loops) ------------------------------
 * cosa_kap_pool_keys writes the proxy's pooled keys (mean over p consecutive
 * keys, as inside cosa_kap_order) into a caller-owned buffer
 * pooled_keys [num_pages, h_kv, B/p, head_dim] in the problem's dtype, laid
 * out like the pages so the block table applies. last_block_only = 0 pools
 * every KV block of every sequence; 1 pools only the last block of each
 * sequence, the one a decode step appends to, so a loop that keeps the
 * buffer pools one page per step instead of the whole cache.
 * cosa_kap_order_pooled is cosa_kap_order reading those pooled keys instead
 * of pooling k_pages (same outputs, workspace and limits). */
cosa_status cosa_kap_pool_keys(const cosa_problem* problem, const void* k_pages, int32_t pool,
                               void* pooled_keys, int32_t last_block_only, void* stream);
cosa_status cosa_kap_order_pooled(const cosa_problem* problem, const void* q, const void* pooled_keys,
                                  int32_t pool, double budget, int32_t* order, uint8_t* hrm,
                                  int32_t* count, int32_t kmax, float* proxy_scores,
                                  float* block_scores, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ---- Ranking from given scores; second-order scores ---------------------------
 * cosa_kap_rank runs the proxy's MaxNorm, HRM flags, sort and budget (as in
 * cosa_kap_order, bit for bit) on a caller's score tensor
 * scores fp32 [batch, h_q, max_nr, max_nk] (-inf where a pooled row sees no
 * key of a block), so any block score can drive the computation order.
 * Limits as cosa_kap_order. */
cosa_status cosa_kap_rank(const cosa_problem* problem, int32_t pool, double budget,
                          const float* scores, int32_t* order, uint8_t* hrm, int32_t* count,
                          int32_t kmax, float* block_scores, void* stream);

/* Second-order block scores (COBS page §2.2-2.3: rank blocks by the first two
 * cumulants of their log attention mass, q.k_mean + 1/2 q^T Sigma q). For
 * pooled query row r (mean of p queries, as in cosa_kap_order) and KV block
 * kb, with s_j = softmax_scale * q_pooled[r] . k_j over the raw keys j of kb
 * that the row's window may see (j <= off + min(r*p+p-1, Lq-1)):
 *   scores[b, h, r, kb] = mean_j s_j + 1/2 var_j s_j   (population variance)
 * i.e. the page's score with the exact per-block key mean and covariance, no
 * compression; -inf where no key is visible and in all padding. It costs a
 * (pooled rows x keys) product per head, B/p times the max-pooled score's.
 * workspace: cosa_cobs_workspace_size bytes (pooled queries), 256-byte
 * aligned. bf16 only. */
size_t cosa_cobs_workspace_size(const cosa_problem* problem, int32_t pool);
cosa_status cosa_cobs_scores(const cosa_problem* problem, const void* q, const void* k_pages,
                             int32_t pool, float* scores, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ---- Decode step ---------------------------------------------------------------
 * One new query token per sequence (cu_seqlens_q steps of 0 or 1; the token
 * sits at absolute position seqlens_k[b] - 1, its key and value already in
 * the cache). The pages name decoding as future work without a method; this
 * keeps the walk of cosa_osk_attention (listed pages only, list order, skip
 * per query head) and splits each (b, g) list into n_splits contiguous
 * segments, entries [floor(s*n/S), floor((s+1)*n/S)), walked by separate
 * workgroups from an empty state (so a segment's first block is never
 * skipped) and merged exactly by log-sum-exp. With skip_threshold 0 the
 * result is softmax attention over the listed keys for every n_splits.
 *  order, count  the proxy's lists for the single query block (cosa_kap_order
 *                on the decode problem), kmax their width.
 *  o             [total_q, h_q, head_dim] bf16; visited / skipped
 *                [batch, h_q, 1] summed over the segments; lse as in
 *                cosa_osk_attention (nullable).
 *  workspace     cosa_osk_decode_workspace_size(problem, n_splits) bytes,
 *                256-byte aligned (per-segment partial results).
 * bf16 only; G = h_q / h_kv <= 32; 1 <= n_splits <= 1024. */
size_t cosa_osk_decode_workspace_size(const cosa_problem* problem, int32_t n_splits);
cosa_status cosa_osk_decode(const cosa_problem* problem, const void* q, const void* k_pages,
                            const void* v_pages, const int32_t* order, const int32_t* count,
                            int32_t kmax, int32_t group, float skip_threshold, int32_t n_splits,
                            void* o, int32_t* visited, int32_t* skipped, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the decode
 * step of cosa_osk_decode, same arguments and results bit for bit, with the
 * per-segment partial results kept in a fixed scratch array inside the
 * library instead of a caller's workspace. The call allocates nothing.
 * Limit: cosa_osk_decode_workspace_size(problem, n_splits) must not exceed
 * 32 MiB (33554432 bytes), e.g. batch 64 x 64 query heads x 15 segments at
 * head_dim 128; larger problems are rejected with COSA_ERR_UNSUPPORTED before
 * any launch. Every call on one GPU uses that GPU's single array, which keeps
 * the last call's contents (no part of it needs clearing: every partial
 * result the merge reads is written by the same call), so calls that can
 * overlap on one GPU (different streams or threads) race: order them on one
 * stream. The array (32 MiB per GPU) is held from the library's first use on
 * a device until the process ends. */
cosa_status cosa_osk_decode_noalloc(const cosa_problem* problem, const void* q, const void* k_pages,
                                    const void* v_pages, const int32_t* order, const int32_t* count,
                                    int32_t kmax, int32_t group, float skip_threshold, int32_t n_splits,
                                    void* o, int32_t* visited, int32_t* skipped, float* lse, void* stream);

/* ---- Binary block masks (comparison modes) -----------------------------------
 * The CoSA summary contrasts its computation-order list (§2.1) with the
 * binary masks of earlier proxies, and its page-remapped walk (§2.3,
 * "mask-skipped" blocks are jumped over) with the control-flow skipping of
 * standard sparse kernels; its ablation (§4) separates ordered selection,
 * in-kernel skipping and remapping. These calls run one selection either way.
 *
 * mask  uint64 [batch, h_kv, max_nq, mask_words]: bit (kb % 64) of word
 *       kb / 64 selects KV block kb for (b, g, qb). mask_words >=
 *       ceil(max_nk / 64). Bits of non-causal blocks (kb >= n(qb)) are
 *       ignored by every reader and cleared by cosa_mask_from_order. */

/* mask = the set of causal blocks listed in order[.., 0 .. count-1] (entries
 * outside 0 .. n(qb)-1 are ignored; the visit order is dropped). Rows past a
 * sequence's end are all zero. Limits: mask_words <= 64. */
cosa_status cosa_mask_from_order(const cosa_problem* problem, const int32_t* order,
                                 const int32_t* count, int32_t kmax, uint64_t* mask,
                                 int32_t mask_words, void* stream);

/* order = the selected causal blocks of each row in ascending kb, truncated to
 * the first kmax; count = the number written; -1 pads the row. mask may be
 * NULL: every causal block is selected (with kmax >= max_nk, the dense walk
 * as a list, so in-kernel skipping can run without any proxy). Rows past a
 * sequence's end get count 0. Limits: max_nk <= 4096 (mask_words <= 64). */
cosa_status cosa_order_from_mask(const cosa_problem* problem, const uint64_t* mask,
                                 int32_t mask_words, int32_t* order, int32_t* count, int32_t kmax,
                                 void* stream);

/* cosa_osk_attention over a binary mask instead of a list: each row walks all
 * of its causal blocks in ascending order, tests the block's bit and branches
 * over unselected blocks (control-flow skipping). A selected block is
 * prefetched only while the previous block is selected too; after a gap its
 * pages are fetched on arrival. Selected blocks get the same skip test and
 * update as in cosa_osk_attention, so the output equals that of
 * cosa_osk_attention on cosa_order_from_mask's ascending list, bit for bit.
 * visited = selected causal blocks walked; skipped = blocks skipped in-kernel.
 * bf16 only (COSA_ERR_UNSUPPORTED for fp32). */
cosa_status cosa_osk_attention_masked(const cosa_problem* problem, const void* q,
                                      const void* k_pages, const void* v_pages,
                                      const uint64_t* mask, int32_t mask_words, int32_t group,
                                      float skip_threshold, void* o, int32_t* visited,
                                      int32_t* skipped, float* lse, void* stream);

/* Block-union tables for chunked prefill (CompactAttention page, selection
 * stage: a union over the query blocks of the chunk, on top of the union over
 * the query heads of a KV group that the lists already are; execution stage:
 * a dense paged walk over the table). For each (b, g) the table is the set of
 * causal blocks listed by any query block of the sequence; each query block
 * gets the table's blocks that are causal for it, ascending, in
 * union_order[b, g, qb, 0 .. union_count-1] (-1 pad, truncated to
 * union_kmax; union_kmax >= max_nk never truncates). Walking these lists
 * with cosa_osk_attention and skip_threshold 0 is the union method's
 * execution; every block any query block selected stays covered.
 * Limits: max_nk <= 4096. */
cosa_status cosa_union_order(const cosa_problem* problem, const int32_t* order,
                             const int32_t* count, int32_t kmax, int32_t* union_order,
                             int32_t* union_count, int32_t union_kmax, void* stream);

/* Exact attention mass of every causal block, the ranking of the oracle
 * selector on the COBS page ("Oracle Sparse Attention": keep the blocks that
 * hold the most exact softmax mass), against which a proxy's selection can be
 * scored (a diagnostic; it costs the QK^T of dense attention).
 *  lse   fp32 [h_q, total_q]: natural-log sum-exp of each row over its
 *        visible keys, as cosa_dense_attention writes it.
 *  mass  fp32 [batch, h_q, max_nq, max_nk]: sum over the valid rows of qb and
 *        the visible keys of kb of exp(softmax_scale * q.k - lse); 0 for
 *        non-causal blocks and rows past a sequence's end; NaN for a block
 *        whose page is outside the pool. A query row's masses add up to 1.
 * bf16 only (COSA_ERR_UNSUPPORTED for fp32). */
cosa_status cosa_block_mass(const cosa_problem* problem, const void* q, const void* k_pages,
                            const float* lse, float* mass, void* stream);

/* Static description of a status code. */
const char* cosa_status_string(cosa_status status);

/* Thread-local message of the last rejected or failed call on this thread
 * ("" after a successful call). */
const char* cosa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t cosa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COSA_H */
