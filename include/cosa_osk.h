/*
 * cosa_osk.h -- C ABI of the MI355X (gfx950) ordered-skipping block-sparse
 * prefill attention library (libcosa_osk.so).
 *
 * What the library computes
 * -------------------------
 * Block-sparse causal prefill attention over a paged KV cache, as the CoSA
 * paper ("Accelerating Long-Context Inference via Proxy-Kernel Co-Designed
 * Sparse Attention") defines its Ordered-Skipping Kernel (OSK): section 4.3 and
 * Appendix C, Algorithm A (attention loop).  Every query block i of a
 * sequence visits the logical KV pages listed in its computation-order mask
 * (section 4.2, Eq. (14): kept ids in visit order, -1 padding), in mask order,
 * through the sequence's page table (physical page jumping and any-order page
 * visiting, section 4.3).  It runs the tiled online softmax of section 3.1,
 * Eq. (1)-(2), and skips the value side of a visited page in-kernel when the
 * skip scale Delta > 0 and max_r(m_loc[r] - m[r]) < ln(Delta / N) (section 3.3,
 * Eq. (5); Algorithm A, the skip test), N being the sequence's valid length, the max
 * taken over the block's valid rows, and m updated before the test.  A query
 * at causal position c attends to the tokens of its visited, non-skipped pages
 * with t < L and t <= c (PageWeaver notes, section 2.1, Eq. (1)-(2)); an empty
 * support gives a zero output.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array pointers are DEVICE pointers owned by the caller.  The library
 *   allocates and frees nothing; scratch space is the caller's workspace.
 * - Calls are asynchronous on `stream` (0 = the null stream).  A negative status
 *   is returned synchronously, before anything is launched, for a bad argument;
 *   a launch failure is reported as COSA_ERR_HIP.
 * - The library keeps no state between calls; calls are thread-safe.  Calls
 *   that share a workspace must be ordered on one stream.
 * - An empty batch (total_qblocks == 0: every sequence has length 0) reads and
 *   writes nothing: the prefill and builder calls check dims and their scalar
 *   arguments, launch nothing and return COSA_OK; their pointers may then be NULL
 *   and no workspace is needed.  cosa_validate_order_mask still zeroes its
 *   counters.
 * - Blocks and pages (CoSA Appendix D.1, "CoSA settings": the block size b and
 *   the page size b_p of the paged cache are two separate settings, so one
 *   logical block may span several physical pages).  The logical block -- the query
 *   block, the mask's key block, the unit of a skip vote -- is b = block_size = 64
 *   or 128 tokens (Appendix D.1 uses 128: one vote per 128-row query tile).  The KV
 *   cache's physical pages hold b_p = page_size = 16, 32 or 64 tokens, or 128 when
 *   b = 128: logical block j of a sequence is its tokens b j .. b j + b - 1, token
 *   t stored in physical page page_table[s][t / b_p] at row t % b_p.  A logical
 *   block is used only if every physical page holding one of its tokens t < L is a
 *   valid page id (0 <= id < num_phys_pages); otherwise it is not visited, like an
 *   invalid id.  max_blocks = ceil(max_pages_per_seq * page_size / b) logical
 *   blocks per sequence are addressable; mask ids, the mask-width helpers and the
 *   builders' score rows count logical blocks.
 * - Supported: head_dim = 128, block_size 64 or 128, page_size dividing it (16,
 *   32, 64, 128), bfloat16 Q/K/V/out, num_q_heads % num_kv_heads == 0.
 *   Limits: total_qblocks <= 16384, max_mask_len <= 8191,
 *   max_blocks <= 16384 (<= 8192 for the mask builders),
 *   kv_stride_tok <= 2^24 elements (a page's byte offsets fit in 32 bits).
 *   Anything else returns COSA_ERR_UNSUPPORTED.
 * - Layouts (element strides; head_dim is contiguous; strides are multiples of
 *   8 elements and the base pointers are 16-byte aligned; the strides of q and out
 *   are not checked when total_q_tokens is 0, those of the pools when
 *   num_phys_pages is 0):
 *     q, out        [total_q_tokens, num_q_heads, 128]   (sequences packed on T)
 *     k_pool,v_pool [num_phys_pages, num_kv_heads, page_size, 128] (same strides)
 *     page_table    int32 [num_seqs, max_pages_per_seq]   page-sized token range -> physical page
 *     cu_seqlens    int32 [num_seqs + 1]  token offsets; L_s = difference
 *     cu_qblocks    int32 [num_seqs + 1]  prefix sums of ceil(L_s / b)
 *     order_mask    int32 [total_qblocks, num_kv_heads, max_mask_len]
 *     mask_len      int32 [total_qblocks, num_kv_heads]
 *   A query block's global index is qb = cu_qblocks[s] + i.  The q heads of a KV
 *   head share its mask row (grouped-query heads share one page set per KV head,
 *   PageWeaver notes section 2); skip votes are taken per q head.
 */
#ifndef COSA_OSK_H
#define COSA_OSK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COSA_ABI_VERSION 2

typedef enum {
  COSA_OK = 0,
  COSA_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad stride/alignment */
  COSA_ERR_UNSUPPORTED = -2,  /* outside the supported shapes/limits listed above  */
  COSA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required         */
  COSA_ERR_HIP = -4           /* a HIP launch reported an error                      */
} cosa_status_t;

/* Decision-log codes (one byte per (query block, q head, mask position)). */
#define COSA_DECISION_COMPUTED 0u    /* value side computed                          */
#define COSA_DECISION_SKIPPED 1u     /* skipped in-kernel by Eq. (5)                 */
#define COSA_DECISION_NOT_VISITED 2u /* padding, id outside [0, n_pages), id > i,
                                        repeated id, or physical id outside the pool */

/* Mask-builder flags: pages always kept. */
#define COSA_FORCE_FIRST 1u  /* logical page 0 (attention sink)   */
#define COSA_FORCE_DIAG 2u   /* the block's own (diagonal) page i */

typedef struct cosa_osk_dims {
  int32_t num_seqs;           /* >= 1 */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;           /* must be 128 */
  int32_t page_size;          /* tokens per physical KV page: 16, 32, 64 (128 if block_size is 128) */
  int32_t total_q_tokens;     /* T = cu_seqlens[num_seqs] */
  int32_t total_qblocks;      /* cu_qblocks[num_seqs] */
  int32_t max_pages_per_seq;  /* row stride of page_table (physical pages per sequence); >= 1, or 0 in an empty batch */
  int32_t num_phys_pages;     /* pool size; a physical id outside [0, n) is not visited */
  int32_t max_mask_len;       /* row stride of order_mask and of the decision log */
  float sm_scale;             /* logit scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t block_size;         /* tokens per logical block b: 64 (0 selects 64) or 128 */
  int64_t q_stride_tok, q_stride_head;                  /* elements */
  int64_t o_stride_tok, o_stride_head;                  /* elements */
  int64_t kv_stride_page, kv_stride_head, kv_stride_tok; /* elements, K and V alike */
} cosa_osk_dims_t;

/* ABI version of the loaded library (COSA_ABI_VERSION it was built with). */
int cosa_abi_version(void);

/* Static, human-readable text of a status code. */
const char* cosa_status_string(cosa_status_t status);

/* Bytes of workspace cosa_osk_prefill needs for these dims (the unit schedule).
 * Returns 0 if dims is NULL. Host-only. */
size_t cosa_osk_workspace_bytes(const cosa_osk_dims_t* dims);

/* Host-only validation of dims and the workspace size, the same checks
 * cosa_osk_prefill runs before launching; touches no device. */
cosa_status_t cosa_osk_check_args(const cosa_osk_dims_t* dims, size_t workspace_bytes);

/*
 * Ordered-skipping prefill attention (CoSA section 4.3; Appendix C, Algorithm A,
 * attention loop; skip rule section 3.3, Eq. (5); per-query semantics PageWeaver
 * notes section 2.1, Eq. (1)-(2)).
 *
 *   q, k_pool, v_pool  bfloat16 inputs (layouts above); read only.
 *   page_table, cu_seqlens, cu_qblocks, order_mask, mask_len  int32; read only.
 *       order_mask rows hold logical page ids in visit order; entries at
 *       positions >= mask_len are ignored; inside the row, ids < 0, ids >=
 *       ceil(L_s/b), ids > i and repeats of an earlier id are not visited
 *       (cosa_validate_order_mask reports them).
 *   budget2   the skip scale Delta of Eq. (5).  Delta <= 0 disables in-kernel
 *             skipping (Delta = -1 is the pages' "off" value).  Otherwise the
 *             threshold of sequence s is tau_s = ln(Delta / L_s) in natural-log
 *             units of the scaled logits; a page is skipped iff the largest
 *             (over the block's valid rows r) of m_loc[r] - m_new[r] is < tau_s.
 *             Delta > L_s skips every page of that sequence (zero output).
 *   out       bfloat16 [T, Hq, 128]; written for every valid token.
 *   lse       nullable fp32 [T, Hq]: natural-log log-sum-exp of the scaled logits
 *             over the computed keys (-inf where nothing was computed).
 *   decisions nullable uint8 [total_qblocks, Hq, max_mask_len]: COSA_DECISION_*.
 *   margins   nullable fp32, same shape: max_r(m_loc[r] - m_new[r]) in natural-
 *             log units for visited positions, NaN elsewhere (requires decisions;
 *             margins without decisions is COSA_ERR_INVALID_ARG).
 *   workspace device scratch of >= cosa_osk_workspace_bytes(dims) bytes, 16-byte
 *             aligned; its contents are overwritten.  After the call completes, the
 *             int32 at byte offset cosa_osk_workspace_bytes(dims) - 256 is a health
 *             word: the number of workgroups that could not complete their visits
 *             (nonzero would mean the output of those blocks is not valid).  The
 *             kernels synchronise their waves with workgroup barriers only, so it
 *             is 0 after every call; it is kept for callers that check it.  A
 *             library built with COSA_OSK_CHECKED (libcosa_osk_checked.so) also
 *             counts there every index invariant its prefill kernels find broken
 *             (schedule position, mask or page-table column, physical page id,
 *             output row); 0 means none was.  A call on an empty batch launches
 *             nothing and leaves the workspace, health word included, untouched.
 * Numerics: fp32 accumulation of bf16 products for Q K^T, fp32 running max/sum,
 * probabilities rounded to bf16 for the P V product, fp32 output accumulator,
 * bf16 output.
 */
cosa_status_t cosa_osk_prefill(const cosa_osk_dims_t* dims,
                               const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* page_table, const int32_t* cu_seqlens,
                               const int32_t* cu_qblocks, const int32_t* order_mask,
                               const int32_t* mask_len, float budget2,
                               void* out, float* lse, uint8_t* decisions, float* margins,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * cosa_osk_prefill for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * kernels and results, with no workspace argument.  The workspace lives in a
 * library-held device array of COSA_OSK_NOALLOC_SCRATCH_BYTES bytes, one copy per
 * GPU, kept until the process ends; its address is looked up on the first call on
 * each device (that call must run with the device current, as every call does).
 * Limit: the workspace must fit the array (cosa_osk_workspace_bytes(dims) <=
 * COSA_OSK_NOALLOC_SCRATCH_BYTES, which holds for every total_qblocks the library
 * accepts); a larger need returns COSA_ERR_WORKSPACE before anything is launched.
 * The call allocates nothing (no hipMalloc / hipFree, no allocating library call);
 * each call rewrites the whole scratch it uses with kernels, so no state carries
 * over between calls.  Every call on one GPU shares that GPU's array: calls that
 * may overlap on one GPU (different streams, or different host threads without
 * ordering) race and give undefined results -- order them on one stream.  The
 * health word of cosa_osk_prefill stays in the scratch and is not reported.
 * Arguments and errors otherwise as for cosa_osk_prefill.
 */
#define COSA_OSK_NOALLOC_SCRATCH_BYTES 66048
cosa_status_t cosa_osk_prefill_noalloc(const cosa_osk_dims_t* dims,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* page_table, const int32_t* cu_seqlens,
                                       const int32_t* cu_qblocks, const int32_t* order_mask,
                                       const int32_t* mask_len, float budget2,
                                       void* out, float* lse, uint8_t* decisions, float* margins,
                                       hipStream_t stream);

/*
 * The same prefill with a page set per q head (PageWeaver notes, section 2.2: the q
 * heads of a KV group traverse the union of their sets, and a membership mask keeps
 * each head's softmax to its own pages).  order_mask row (qb, g) is the union in
 * visit order; membership uint8 [total_qblocks, Hq, max_mask_len] (device, read
 * only) marks with a nonzero byte the entries k < mask_len that belong to q head
 * h of KV head g.  A head takes part in a visit -- logits, running max, skip vote,
 * value side -- only at its own entries, so it sees its own blocks in the union's
 * order; every other entry is logged COSA_DECISION_NOT_VISITED for it, margin NaN.
 * A repeated id is not visited by any head (its first occurrence counts, whoever
 * it belongs to), and an entry no head of a workgroup's heads owns is not gathered.
 * All 1 membership gives exactly cosa_osk_prefill.  membership may be NULL only
 * when max_mask_len == 0; otherwise every argument is as for cosa_osk_prefill.
 */
cosa_status_t cosa_osk_prefill_union(const cosa_osk_dims_t* dims,
                                     const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* page_table, const int32_t* cu_seqlens,
                                     const int32_t* cu_qblocks, const int32_t* order_mask,
                                     const int32_t* mask_len, const uint8_t* membership, float budget2,
                                     void* out, float* lse, uint8_t* decisions, float* margins,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Row width a computation-order mask built by cosa_build_order_mask needs:
 * the longest |F_i| + ceil(budget1 * |R_i| - 1e-3) over blocks i < max_blocks_per_seq
 * (F_i: forced pages, R_i: the other causal pages).  Host-only.  Returns -1 for
 * max_blocks_per_seq < 1.  (max_blocks_per_seq: logical blocks per sequence, the
 * max_blocks of the dims.)
 */
int32_t cosa_order_mask_width(int32_t max_blocks_per_seq, float budget1, uint32_t flags);

/* Workspace bytes cosa_build_order_mask needs: the fp32 pooled query and key
 * proxies [total_qblocks, Hkv, 128] each and the fp32 score rows
 * [total_qblocks, Hkv, max_blocks] (used when proxy_scores is NULL),
 * each region padded to 256 bytes.  Host-only. */
size_t cosa_build_order_mask_workspace_bytes(const cosa_osk_dims_t* dims);

/*
 * Computation-order mask from the mean-pooled q.k proxy (CoSA section 4.2,
 * Eq. (14) for the mask format; the proxy is the dot product of mean-pooled
 * query-block and key-page representations, kept pages visited in descending
 * proxy order, as the paper's rewrite page describes it).  For every query
 * block i of sequence s and KV head g:
 *   qbar = sum over the group's q heads of the mean of q over the block's valid rows,
 *   kbar_j = mean of k over the tokens t < L_s of logical page j,
 *   score_j = qbar . kbar_j (fp32) for causal pages j <= i;
 *   kept = forced pages (flags) + the top ceil(budget1 * |R_i| - 1e-3) of the
 *   remaining causal pages R_i by (score descending, id ascending);
 *   the row lists the kept ids in (score descending, id ascending) order, -1 after.
 * order_mask [total_qblocks, Hkv, max_mask_len] and mask_len [total_qblocks, Hkv]
 * are written; dims->max_mask_len must be >= cosa_order_mask_width(...).
 * proxy_scores (nullable) fp32 [total_qblocks, Hkv, max_blocks]: score_j for
 * j <= i, NaN after.  budget1 in [0, 1].  k_pool uses the dims' KV strides.
 */
cosa_status_t cosa_build_order_mask(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                    const int32_t* page_table, const int32_t* cu_seqlens,
                                    const int32_t* cu_qblocks, float budget1, uint32_t flags,
                                    int32_t* order_mask, int32_t* mask_len, float* proxy_scores,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Row width a union mask of cosa_build_union_mask needs: the longest
 * min(i + 1, group * (|F_i| + ceil(budget1 * |R_i| - 1e-3))) over blocks
 * i < max_blocks_per_seq (group = Hq / Hkv).  Host-only.  -1 for
 * max_blocks_per_seq < 1 or group < 1. */
int32_t cosa_union_mask_width(int32_t max_blocks_per_seq, int32_t group, float budget1, uint32_t flags);

/* Workspace bytes cosa_build_union_mask needs: those of cosa_build_order_mask, then
 * each q head's fp32 block means [total_qblocks, Hq, 128] and score rows
 * [total_qblocks, Hq, max_blocks], each region padded to 256 bytes.  Host-only. */
size_t cosa_build_union_mask_workspace_bytes(const cosa_osk_dims_t* dims);

/*
 * Per-q-head page sets from the mean-pooled proxy, as a union row per KV head with a
 * membership mask (PageWeaver notes, section 2.2, union U_G and membership M; Eq. (3)
 * gives the reuse ratio sum head_len / sum mask_len).  Each q head h selects its own
 * set with the rule of cosa_build_order_mask applied to its own score
 * qbar_h . kbar_j (qbar_h: the mean of q_h over the block's valid rows): the forced
 * pages plus its top ceil(budget1 * |R_i| - 1e-3) by (score descending, id
 * ascending).  Row (qb, g) lists the union of the group's sets in the order of the
 * shared mask (group score descending, id ascending), -1 after; mask_len is the
 * union's size.  membership uint8 [total_qblocks, Hq, max_mask_len]: 1 where entry k
 * is in head h's set, 0 elsewhere (also past mask_len); head_len int32
 * [total_qblocks, Hq]: each head's set size.  dims->max_mask_len must be >=
 * cosa_union_mask_width(max_blocks, Hq / Hkv, budget1, flags); Hq / Hkv <= 32.
 * The output feeds cosa_osk_prefill_union.
 */
cosa_status_t cosa_build_union_mask(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                    const int32_t* page_table, const int32_t* cu_seqlens,
                                    const int32_t* cu_qblocks, float budget1, uint32_t flags,
                                    int32_t* order_mask, int32_t* mask_len, uint8_t* membership,
                                    int32_t* head_len, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Stage-1 selection modes of cosa_build_kap_mask. */
#define COSA_KAP_FRACTION 0 /* K_i = ceil(budget * (i + 1) - 1e-3), at least 1            */
#define COSA_KAP_TOP_P 1    /* smallest K_i whose leading scores reach budget of the total */

/* Row width a KAP mask needs: ceil(budget * max_blocks - 1e-3) clamped to
 * [1, max_blocks] for COSA_KAP_FRACTION, max_blocks for COSA_KAP_TOP_P (max_blocks:
 * logical blocks per sequence).  Host-only.  Returns -1 for max_blocks_per_seq < 1
 * or an unknown mode. */
int32_t cosa_kap_mask_width(int32_t max_blocks_per_seq, int32_t mode, float budget);

/* Workspace bytes cosa_build_kap_mask needs: fp32 block scores and uint8 HRM flags
 * [total_qblocks, Hkv, max_blocks] each (used where the caller passes no array of
 * its own), then the sampled rows' maxima, total_qblocks * Hq * 8 uint32, then a copy
 * of the sampled keys, Hkv * (total_qblocks / 4 + num_seqs) tiles of 8 KiB; each
 * region padded to 256 bytes.  Host-only. */
size_t cosa_build_kap_mask_workspace_bytes(const cosa_osk_dims_t* dims);

/*
 * Kernel-aware proxy (KAP) computation-order mask (CoSA section 4.2, Eq. (8)-(14);
 * Appendix C, Figure A and Algorithm A, pre-kernel proxy).  For every query block i
 * of sequence s and KV head g:
 *   Q~, K~ = every stride-th token of the sequence (token r*stride is sample r);
 *   S^ = row-wise softmax of Q~ K~^T * sm_scale with sample c visible to sample r
 *   iff c <= r (sm_scale = dims->sm_scale, 0 meaning 1/sqrt(128));
 *   P[r, j] = max of S^[r, c] over the sampled keys of page-sized block j (0 if none
 *   is visible); Pbar[r, j] = P[r, j] / max_j' P[r, j'];
 *   score s_ij = sum of Pbar[r, j] over the block's sampled rows r of all G q heads
 *   of the group; HRM flag h_ij = 1 if any of those rows has Pbar[r, j] = 1;
 *   the causal candidates j <= i sorted HRM blocks first, then by score descending,
 *   equal scores by block id ascending; the leading K_i of them (mode, budget:
 *   COSA_KAP_FRACTION with budget in (0, 1], or COSA_KAP_TOP_P with budget = p in
 *   [0, 1]) are the row, -1 after.
 * order_mask [total_qblocks, Hkv, max_mask_len] and mask_len [total_qblocks, Hkv]
 * are written; dims->max_mask_len must be >= cosa_kap_mask_width(...).
 * kap_scores (nullable) fp32 and hrm_flags (nullable) uint8, both
 * [total_qblocks, Hkv, max_blocks]: s_ij and h_ij for j <= i, NaN / 0 after.
 * Supported: b / stride = 4 or 8 samples per block (strides 16 or 8 at b = 64, 32 or
 * 16 at b = 128), and G * b / stride a power of two <= 32 (G = Hq / Hkv);
 * max_blocks <= 8192; otherwise COSA_ERR_UNSUPPORTED.  The page-table entries
 * of a sequence's pages must be valid physical pages.  k_pool uses the dims' KV
 * strides.  Asynchronous on `stream`; the workspace is overwritten.
 */
cosa_status_t cosa_build_kap_mask(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                  const int32_t* page_table, const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                                  int32_t stride, int32_t mode, float budget, int32_t* order_mask,
                                  int32_t* mask_len, float* kap_scores, uint8_t* hrm_flags, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Count malformed mask entries (PageWeaver notes section 2.1 conventions: such
 * entries add no interaction; the prefill treats them as not visited).
 * bad_counts: device int32[5], zeroed by the call, then incremented:
 *   [0] ids outside [0, ceil(L_s/b)) at positions < mask_len (includes -1),
 *   [1] non-causal ids (j > i), [2] repeated ids in a row,
 *   [3] mask_len outside [0, max_mask_len],
 *   [4] referenced page-table entries outside [0, num_phys_pages).
 */
cosa_status_t cosa_validate_order_mask(const cosa_osk_dims_t* dims, const int32_t* page_table,
                                       const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                                       const int32_t* order_mask, const int32_t* mask_len,
                                       int32_t* bad_counts, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* COSA_OSK_H */
