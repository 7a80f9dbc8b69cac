// C-ABI entry points of libcosa_osk: host-side argument checks, workspace
// sizing, and kernel launches on the caller's stream.  Declarations and the
// contract of every function are in include/cosa_osk.h.
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include "cosa_osk.h"
#include "osk_internal.h"

namespace {

using cosa_osk::kHeadDim;
using cosa_osk::kPage;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool stride_ok(int64_t s) { return s > 0 && (s % 8) == 0; }

// tokens per logical block (0 selects 64)
int32_t block_of(const cosa_osk_dims_t* d) { return d->block_size == 0 ? kPage : d->block_size; }

// logical blocks a page-table row can address
int32_t max_blocks(const cosa_osk_dims_t* d) {
  const int64_t b = block_of(d);
  return (int32_t)(((int64_t)d->max_pages_per_seq * d->page_size + b - 1) / b);
}

cosa_status_t check_dims(const cosa_osk_dims_t* d) {
  if (d == nullptr) return COSA_ERR_INVALID_ARG;
  if (d->block_size != 0 && d->block_size != 64 && d->block_size != 128) return COSA_ERR_UNSUPPORTED;
  // an empty batch (no query blocks) may come with a page table of no columns
  if (d->num_seqs < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->total_q_tokens < 0 ||
      d->total_qblocks < 0 || d->max_pages_per_seq < (d->total_qblocks > 0 ? 1 : 0) || d->num_phys_pages < 0 ||
      d->max_mask_len < 0)
    return COSA_ERR_INVALID_ARG;
  if (d->head_dim != kHeadDim) return COSA_ERR_UNSUPPORTED;
  // physical pages of 16, 32 or 64 tokens, or 128 under 128-token blocks: a page
  // size that divides the logical block
  const int32_t blk = block_of(d);
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64 && !(blk == 128 && d->page_size == 128))
    return COSA_ERR_UNSUPPORTED;
  if (d->num_q_heads % d->num_kv_heads != 0) return COSA_ERR_UNSUPPORTED;
  if (d->total_qblocks > cosa_osk::kMaxQBlocks || d->max_mask_len > cosa_osk::kMaxMaskLen ||
      max_blocks(d) > cosa_osk::kMaxPagesPerSeq)
    return COSA_ERR_UNSUPPORTED;
  // every query block holds 1..block tokens
  if ((int64_t)d->total_q_tokens > (int64_t)blk * d->total_qblocks || d->total_qblocks > d->total_q_tokens)
    return COSA_ERR_INVALID_ARG;
  // the strides of an empty Q / output (no tokens) or an empty pool (no pages) are never
  // used; array libraries give such tensors arbitrary (often zero) strides
  if (d->total_q_tokens > 0 && (!stride_ok(d->q_stride_tok) || !stride_ok(d->q_stride_head) ||
                                !stride_ok(d->o_stride_tok) || !stride_ok(d->o_stride_head)))
    return COSA_ERR_INVALID_ARG;
  if (d->num_phys_pages > 0 &&
      (!stride_ok(d->kv_stride_page) || !stride_ok(d->kv_stride_head) || !stride_ok(d->kv_stride_tok)))
    return COSA_ERR_INVALID_ARG;
  if (isnan(d->sm_scale) || isinf(d->sm_scale)) return COSA_ERR_INVALID_ARG;
  // page gathers address a page's tokens with 32-bit byte offsets
  if (d->kv_stride_tok > (int64_t)1 << 24) return COSA_ERR_UNSUPPORTED;
  return COSA_OK;
}

float resolved_scale(const cosa_osk_dims_t* d) {
  return d->sm_scale > 0.f ? d->sm_scale : (float)(1.0 / sqrt((double)d->head_dim));
}

int keep_count(float b1, int n) {
  if (n <= 0) return 0;
  const int k = (int)ceil((double)b1 * (double)n - 1e-3);
  return k < 0 ? 0 : (k > n ? n : k);
}

}  // namespace

extern "C" {

int cosa_abi_version(void) { return COSA_ABI_VERSION; }

const char* cosa_status_string(cosa_status_t status) {
  switch (status) {
    case COSA_OK: return "ok";
    case COSA_ERR_INVALID_ARG: return "invalid argument";
    case COSA_ERR_UNSUPPORTED: return "unsupported shape or limit";
    case COSA_ERR_WORKSPACE: return "workspace missing or too small";
    case COSA_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

// workspace layout: [schedule: total_qblocks int32, padded to 256 B][status: 256 B]
static size_t schedule_bytes(const cosa_osk_dims_t* dims) {
  return round_up((size_t)dims->total_qblocks * sizeof(int32_t) + 1);
}

size_t cosa_osk_workspace_bytes(const cosa_osk_dims_t* dims) {
  if (dims == nullptr || dims->total_qblocks < 0) return 0;
  return schedule_bytes(dims) + kAlign;
}

cosa_status_t cosa_osk_check_args(const cosa_osk_dims_t* dims, size_t workspace_bytes) {
  const cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  if (workspace_bytes < cosa_osk_workspace_bytes(dims)) return COSA_ERR_WORKSPACE;
  return COSA_OK;
}

}  // extern "C"

// The prefill with an optional membership mask (null: every q head takes every entry).
static cosa_status_t prefill_impl(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* page_table, const int32_t* cu_seqlens,
                                  const int32_t* cu_qblocks, const int32_t* order_mask, const int32_t* mask_len,
                                  const uint8_t* membership, float budget2, void* out, float* lse,
                                  uint8_t* decisions, float* margins, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  if (dims->total_qblocks == 0) {
    // an empty batch reads and writes nothing: its pointers and workspace are not checked
    if (isnan(budget2) || (margins != nullptr && decisions == nullptr)) return COSA_ERR_INVALID_ARG;
    return COSA_OK;
  }
  st = cosa_osk_check_args(dims, workspace_bytes);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || page_table == nullptr || cu_seqlens == nullptr ||
      cu_qblocks == nullptr || mask_len == nullptr || out == nullptr ||
      (order_mask == nullptr && dims->max_mask_len > 0))
    return COSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return COSA_ERR_INVALID_ARG;
  if (margins != nullptr && decisions == nullptr) return COSA_ERR_INVALID_ARG;
  if (isnan(budget2)) return COSA_ERR_INVALID_ARG;
  if (workspace == nullptr || !aligned16(workspace)) return COSA_ERR_WORKSPACE;
  cosa_osk::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pool);
  a.v = static_cast<const uint16_t*>(v_pool);
  a.page_table = page_table;
  a.cu_seqlens = cu_seqlens;
  a.cu_qblocks = cu_qblocks;
  a.order_mask = order_mask;
  a.mask_len = mask_len;
  a.membership = membership;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.decisions = decisions;
  a.margins = margins;
  a.sched = static_cast<int32_t*>(workspace);
  a.error_count = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + schedule_bytes(dims));
  a.q_st = dims->q_stride_tok;
  a.q_sh = dims->q_stride_head;
  a.o_st = dims->o_stride_tok;
  a.o_sh = dims->o_stride_head;
  a.kv_sp = dims->kv_stride_page;
  a.kv_sh = dims->kv_stride_head;
  a.kv_st = dims->kv_stride_tok;
  a.num_seqs = dims->num_seqs;
  a.hq = dims->num_q_heads;
  a.hkv = dims->num_kv_heads;
  a.total_qblocks = dims->total_qblocks;
  a.max_pages = max_blocks(dims);
  a.pt_stride = dims->max_pages_per_seq;
  a.page_len = dims->page_size;
  a.block = block_of(dims);
  a.num_phys = dims->num_phys_pages;
  a.max_mask_len = dims->max_mask_len;
  a.sm_scale = resolved_scale(dims);
  a.delta = budget2;
  return cosa_osk::launch_prefill(a, stream) == hipSuccess ? COSA_OK : COSA_ERR_HIP;
}

extern "C" {

cosa_status_t cosa_osk_prefill(const cosa_osk_dims_t* dims, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* page_table, const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                               const int32_t* order_mask, const int32_t* mask_len, float budget2, void* out,
                               float* lse, uint8_t* decisions, float* margins, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl(dims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask, mask_len, nullptr,
                      budget2, out, lse, decisions, margins, workspace, workspace_bytes, stream);
}

cosa_status_t cosa_osk_prefill_noalloc(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* page_table, const int32_t* cu_seqlens,
                                       const int32_t* cu_qblocks, const int32_t* order_mask,
                                       const int32_t* mask_len, float budget2, void* out, float* lse,
                                       uint8_t* decisions, float* margins, hipStream_t stream) {
  const cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  static_assert(cosa_osk::kNoAllocScratchBytes == COSA_OSK_NOALLOC_SCRATCH_BYTES, "scratch size");
  const size_t need = cosa_osk_workspace_bytes(dims);
  if (need > cosa_osk::kNoAllocScratchBytes) return COSA_ERR_WORKSPACE;
  if (dims->total_qblocks == 0)  // nothing to launch: the scratch is not looked up
    return prefill_impl(dims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask, mask_len, nullptr,
                        budget2, out, lse, decisions, margins, nullptr, 0, stream);
  void* scratch = nullptr;
  if (cosa_osk::noalloc_scratch(&scratch) != hipSuccess) return COSA_ERR_HIP;
  return prefill_impl(dims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask, mask_len, nullptr,
                      budget2, out, lse, decisions, margins, scratch, cosa_osk::kNoAllocScratchBytes, stream);
}

cosa_status_t cosa_osk_prefill_union(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* page_table, const int32_t* cu_seqlens,
                                     const int32_t* cu_qblocks, const int32_t* order_mask, const int32_t* mask_len,
                                     const uint8_t* membership, float budget2, void* out, float* lse,
                                     uint8_t* decisions, float* margins, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (membership == nullptr && dims != nullptr && dims->max_mask_len > 0 && dims->total_qblocks > 0)
    return COSA_ERR_INVALID_ARG;
  return prefill_impl(dims, q, k_pool, v_pool, page_table, cu_seqlens, cu_qblocks, order_mask, mask_len,
                      membership, budget2, out, lse, decisions, margins, workspace, workspace_bytes, stream);
}

int32_t cosa_order_mask_width(int32_t max_blocks_per_seq, float budget1, uint32_t flags) {
  if (max_blocks_per_seq < 1) return -1;
  int32_t width = 0;
  for (int32_t i = 0; i < max_blocks_per_seq; ++i) {
    int nf = 0;
    if (flags & COSA_FORCE_FIRST) ++nf;
    if ((flags & COSA_FORCE_DIAG) && !((flags & COSA_FORCE_FIRST) && i == 0)) ++nf;
    const int len = nf + keep_count(budget1, i + 1 - nf);
    if (len > width) width = len;
  }
  return width;
}

// builder workspace: pooled query and key proxies [total_qblocks, Hkv, 128] fp32 each,
// then the score rows [total_qblocks, Hkv, max_blocks] fp32 (max_blocks: logical blocks per sequence)
static size_t builder_pool_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * d->num_kv_heads * kHeadDim * sizeof(float) + 1);
}
static size_t builder_score_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * d->num_kv_heads * (size_t)(d->max_pages_per_seq > 0 ? max_blocks(d) : 0) *
                      sizeof(float) + 1);
}

size_t cosa_build_order_mask_workspace_bytes(const cosa_osk_dims_t* dims) {
  if (dims == nullptr || dims->total_qblocks < 0 || dims->num_kv_heads < 1) return 0;
  return 2 * builder_pool_bytes(dims) + builder_score_bytes(dims);
}

cosa_status_t cosa_build_order_mask(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                    const int32_t* page_table, const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                                    float budget1, uint32_t flags, int32_t* order_mask, int32_t* mask_len,
                                    float* proxy_scores, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  if (max_blocks(dims) > cosa_osk::kMaxPagesBuilder) return COSA_ERR_UNSUPPORTED;
  const bool empty = dims->total_qblocks == 0;  // reads and writes nothing: pointers unchecked
  if (!empty && (q == nullptr || k_pool == nullptr || page_table == nullptr || cu_seqlens == nullptr ||
                 cu_qblocks == nullptr || order_mask == nullptr || mask_len == nullptr))
    return COSA_ERR_INVALID_ARG;
  if (!(budget1 >= 0.f && budget1 <= 1.f)) return COSA_ERR_INVALID_ARG;
  if ((flags & ~(uint32_t)(COSA_FORCE_FIRST | COSA_FORCE_DIAG)) != 0u) return COSA_ERR_INVALID_ARG;
  if (dims->max_mask_len < cosa_order_mask_width(max_blocks(dims), budget1, flags)) return COSA_ERR_INVALID_ARG;
  if (empty) return COSA_OK;
  const size_t need = cosa_build_order_mask_workspace_bytes(dims);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return COSA_ERR_WORKSPACE;
  cosa_osk::BuilderArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pool);
  a.page_table = page_table;
  a.cu_seqlens = cu_seqlens;
  a.cu_qblocks = cu_qblocks;
  a.order_mask = order_mask;
  a.mask_len = mask_len;
  a.scores = proxy_scores;
  a.qbar = static_cast<float*>(workspace);
  a.kbar = reinterpret_cast<float*>(static_cast<char*>(workspace) + builder_pool_bytes(dims));
  a.score_rows = proxy_scores != nullptr
                     ? proxy_scores
                     : reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * builder_pool_bytes(dims));
  a.q_st = dims->q_stride_tok;
  a.q_sh = dims->q_stride_head;
  a.kv_sp = dims->kv_stride_page;
  a.kv_sh = dims->kv_stride_head;
  a.kv_st = dims->kv_stride_tok;
  a.num_seqs = dims->num_seqs;
  a.hq = dims->num_q_heads;
  a.hkv = dims->num_kv_heads;
  a.total_qblocks = dims->total_qblocks;
  a.max_pages = max_blocks(dims);
  a.pt_stride = dims->max_pages_per_seq;
  a.page_len = dims->page_size;
  a.block = block_of(dims);
  a.num_phys = dims->num_phys_pages;
  a.max_mask_len = dims->max_mask_len;
  a.budget1 = budget1;
  a.flags = flags;
  return cosa_osk::launch_build_order_mask(a, stream) == hipSuccess ? COSA_OK : COSA_ERR_HIP;
}

int32_t cosa_union_mask_width(int32_t max_blocks_per_seq, int32_t group, float budget1, uint32_t flags) {
  if (max_blocks_per_seq < 1 || group < 1) return -1;
  int64_t width = 0;
  for (int32_t i = 0; i < max_blocks_per_seq; ++i) {
    int nf = 0;
    if (flags & COSA_FORCE_FIRST) ++nf;
    if ((flags & COSA_FORCE_DIAG) && !((flags & COSA_FORCE_FIRST) && i == 0)) ++nf;
    const int64_t len = std::min<int64_t>((int64_t)i + 1, (int64_t)group * (nf + keep_count(budget1, i + 1 - nf)));
    if (len > width) width = len;
  }
  return (int32_t)width;
}

// union-builder workspace: the shared builder's regions, then each head's block means
// [total_qblocks, Hq, 128] fp32 and score rows [total_qblocks, Hq, max_blocks] fp32
static size_t union_head_pool_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * d->num_q_heads * kHeadDim * sizeof(float) + 1);
}
static size_t union_head_score_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * d->num_q_heads * (size_t)std::max(max_blocks(d), 0) * sizeof(float) +
                  1);
}

size_t cosa_build_union_mask_workspace_bytes(const cosa_osk_dims_t* dims) {
  if (dims == nullptr || dims->total_qblocks < 0 || dims->num_kv_heads < 1 || dims->num_q_heads < 1) return 0;
  return cosa_build_order_mask_workspace_bytes(dims) + union_head_pool_bytes(dims) + union_head_score_bytes(dims);
}

cosa_status_t cosa_build_union_mask(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                    const int32_t* page_table, const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                                    float budget1, uint32_t flags, int32_t* order_mask, int32_t* mask_len,
                                    uint8_t* membership, int32_t* head_len, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  if (max_blocks(dims) > cosa_osk::kMaxPagesBuilder) return COSA_ERR_UNSUPPORTED;
  const int32_t G = dims->num_q_heads / dims->num_kv_heads;
  if (G > 32) return COSA_ERR_UNSUPPORTED;  // a candidate's head bits are one 32-bit word
  const bool empty = dims->total_qblocks == 0;  // reads and writes nothing: pointers unchecked
  if (!empty && (q == nullptr || k_pool == nullptr || page_table == nullptr || cu_seqlens == nullptr ||
                 cu_qblocks == nullptr || order_mask == nullptr || mask_len == nullptr || membership == nullptr ||
                 head_len == nullptr))
    return COSA_ERR_INVALID_ARG;
  if (!(budget1 >= 0.f && budget1 <= 1.f)) return COSA_ERR_INVALID_ARG;
  if ((flags & ~(uint32_t)(COSA_FORCE_FIRST | COSA_FORCE_DIAG)) != 0u) return COSA_ERR_INVALID_ARG;
  if (dims->max_mask_len < cosa_union_mask_width(max_blocks(dims), G, budget1, flags)) return COSA_ERR_INVALID_ARG;
  if (empty) return COSA_OK;
  const size_t need = cosa_build_union_mask_workspace_bytes(dims);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return COSA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  cosa_osk::BuilderArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pool);
  a.page_table = page_table;
  a.cu_seqlens = cu_seqlens;
  a.cu_qblocks = cu_qblocks;
  a.order_mask = order_mask;
  a.mask_len = mask_len;
  a.scores = nullptr;
  a.qbar = reinterpret_cast<float*>(ws);
  a.kbar = reinterpret_cast<float*>(ws + builder_pool_bytes(dims));
  a.score_rows = reinterpret_cast<float*>(ws + 2 * builder_pool_bytes(dims));
  a.qbar_heads = reinterpret_cast<float*>(ws + cosa_build_order_mask_workspace_bytes(dims));
  a.head_score_rows =
      reinterpret_cast<float*>(ws + cosa_build_order_mask_workspace_bytes(dims) + union_head_pool_bytes(dims));
  a.membership = membership;
  a.head_len = head_len;
  a.q_st = dims->q_stride_tok;
  a.q_sh = dims->q_stride_head;
  a.kv_sp = dims->kv_stride_page;
  a.kv_sh = dims->kv_stride_head;
  a.kv_st = dims->kv_stride_tok;
  a.num_seqs = dims->num_seqs;
  a.hq = dims->num_q_heads;
  a.hkv = dims->num_kv_heads;
  a.total_qblocks = dims->total_qblocks;
  a.max_pages = max_blocks(dims);
  a.pt_stride = dims->max_pages_per_seq;
  a.page_len = dims->page_size;
  a.block = block_of(dims);
  a.num_phys = dims->num_phys_pages;
  a.max_mask_len = dims->max_mask_len;
  a.budget1 = budget1;
  a.flags = flags;
  return cosa_osk::launch_build_union_mask(a, stream) == hipSuccess ? COSA_OK : COSA_ERR_HIP;
}

int32_t cosa_kap_mask_width(int32_t max_blocks_per_seq, int32_t mode, float budget) {
  if (max_blocks_per_seq < 1) return -1;
  if (mode == COSA_KAP_TOP_P) return max_blocks_per_seq;
  if (mode != COSA_KAP_FRACTION) return -1;
  const int w = (int)ceil((double)budget * (double)max_blocks_per_seq - 1e-3);
  return std::max(1, std::min(max_blocks_per_seq, w));
}

// KAP workspace: fp32 score rows then uint8 flag rows, [total_qblocks, Hkv, max_pages] each
static size_t kap_score_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * d->num_kv_heads * (size_t)std::max(max_blocks(d), 0) *
                      sizeof(float) + 1);
}
static size_t kap_flag_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * d->num_kv_heads * (size_t)std::max(max_blocks(d), 0) + 1);
}

// then the row-maximum codes, [total_qblocks, Hkv, G * samples per block] uint32, sized
// for the largest sample count (8 per block)
static size_t kap_rowmax_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->total_qblocks * (size_t)std::max(d->num_q_heads, 0) * 8 * sizeof(uint32_t) + 1);
}

// then the packed sampled-key tiles, [Hkv, slots] x 8 KiB with slots = total_qblocks *
// samples per block / 32 + num_seqs, sized for 8 samples per block
static int64_t kap_tile_slots(const cosa_osk_dims_t* d, int per) {
  return (int64_t)d->total_qblocks * per / 32 + std::max(d->num_seqs, 0);
}
static size_t kap_tile_bytes(const cosa_osk_dims_t* d) {
  return round_up((size_t)d->num_kv_heads * (size_t)kap_tile_slots(d, 8) * 8 * 64 * 16 + 1);
}

size_t cosa_build_kap_mask_workspace_bytes(const cosa_osk_dims_t* dims) {
  if (dims == nullptr || dims->total_qblocks < 0 || dims->num_kv_heads < 1) return 0;
  return kap_score_bytes(dims) + kap_flag_bytes(dims) + kap_rowmax_bytes(dims) + kap_tile_bytes(dims);
}

cosa_status_t cosa_build_kap_mask(const cosa_osk_dims_t* dims, const void* q, const void* k_pool,
                                  const int32_t* page_table, const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                                  int32_t stride, int32_t mode, float budget, int32_t* order_mask,
                                  int32_t* mask_len, float* kap_scores, uint8_t* hrm_flags, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  if (max_blocks(dims) > cosa_osk::kMaxPagesBuilder) return COSA_ERR_UNSUPPORTED;
  const bool empty = dims->total_qblocks == 0;  // reads and writes nothing: pointers unchecked
  if (!empty && (q == nullptr || k_pool == nullptr || page_table == nullptr || cu_seqlens == nullptr ||
                 cu_qblocks == nullptr || order_mask == nullptr || mask_len == nullptr))
    return COSA_ERR_INVALID_ARG;
  if (mode != COSA_KAP_FRACTION && mode != COSA_KAP_TOP_P) return COSA_ERR_INVALID_ARG;
  if (mode == COSA_KAP_FRACTION ? !(budget > 0.f && budget <= 1.f) : !(budget >= 0.f && budget <= 1.f))
    return COSA_ERR_INVALID_ARG;
  // 4 or 8 samples per logical block: strides 16 and 8 for 64-token blocks, 32 and 16
  // for 128-token blocks
  const int blk = block_of(dims);
  if (stride <= 0 || (stride * 4 != blk && stride * 8 != blk)) return COSA_ERR_UNSUPPORTED;
  const int G = dims->num_q_heads / dims->num_kv_heads;
  // the sampled rows of a query block (all heads of the group) form a power-of-two group
  // of at most 32 MFMA columns
  const int rb = G * (blk / stride);
  if (rb > 32 || (rb & (rb - 1)) != 0) return COSA_ERR_UNSUPPORTED;
  if (dims->max_mask_len < cosa_kap_mask_width(max_blocks(dims), mode, budget)) return COSA_ERR_INVALID_ARG;
  if (empty) return COSA_OK;
  const size_t need = cosa_build_kap_mask_workspace_bytes(dims);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return COSA_ERR_WORKSPACE;
  cosa_osk::KapArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_pool);
  a.page_table = page_table;
  a.cu_seqlens = cu_seqlens;
  a.cu_qblocks = cu_qblocks;
  a.order_mask = order_mask;
  a.mask_len = mask_len;
  a.scores_out = kap_scores;
  a.flags_out = hrm_flags;
  a.score_rows = kap_scores != nullptr ? kap_scores : static_cast<float*>(workspace);
  a.flag_rows = hrm_flags != nullptr ? hrm_flags
                                     : reinterpret_cast<uint8_t*>(static_cast<char*>(workspace) + kap_score_bytes(dims));
  a.row_max = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kap_score_bytes(dims) + kap_flag_bytes(dims));
  a.k_tiles = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + kap_score_bytes(dims) + kap_flag_bytes(dims) +
                                          kap_rowmax_bytes(dims));
  if (kap_tile_slots(dims, blk / stride) > 0x7fffffff) return COSA_ERR_UNSUPPORTED;
  a.tile_slots = (int32_t)kap_tile_slots(dims, blk / stride);
  a.q_st = dims->q_stride_tok;
  a.q_sh = dims->q_stride_head;
  a.kv_sp = dims->kv_stride_page;
  a.kv_sh = dims->kv_stride_head;
  a.kv_st = dims->kv_stride_tok;
  a.num_seqs = dims->num_seqs;
  a.hq = dims->num_q_heads;
  a.hkv = dims->num_kv_heads;
  a.total_qblocks = dims->total_qblocks;
  a.max_pages = max_blocks(dims);
  a.pt_stride = dims->max_pages_per_seq;
  a.page_len = dims->page_size;
  a.block = block_of(dims);
  a.num_phys = dims->num_phys_pages;
  a.max_mask_len = dims->max_mask_len;
  a.stride = stride;
  a.mode = mode;
  a.budget = budget;
  a.sm_scale = resolved_scale(dims);
  return cosa_osk::launch_build_kap_mask(a, stream) == hipSuccess ? COSA_OK : COSA_ERR_HIP;
}

cosa_status_t cosa_validate_order_mask(const cosa_osk_dims_t* dims, const int32_t* page_table,
                                       const int32_t* cu_seqlens, const int32_t* cu_qblocks,
                                       const int32_t* order_mask, const int32_t* mask_len, int32_t* bad_counts,
                                       hipStream_t stream) {
  cosa_status_t st = check_dims(dims);
  if (st != COSA_OK) return st;
  if (page_table == nullptr || cu_seqlens == nullptr || cu_qblocks == nullptr || mask_len == nullptr ||
      bad_counts == nullptr || (order_mask == nullptr && dims->max_mask_len > 0))
    return COSA_ERR_INVALID_ARG;
  cosa_osk::ValidateArgs a{};
  a.page_table = page_table;
  a.cu_seqlens = cu_seqlens;
  a.cu_qblocks = cu_qblocks;
  a.order_mask = order_mask;
  a.mask_len = mask_len;
  a.bad = bad_counts;
  a.num_seqs = dims->num_seqs;
  a.hkv = dims->num_kv_heads;
  a.total_qblocks = dims->total_qblocks;
  a.max_pages = max_blocks(dims);
  a.pt_stride = dims->max_pages_per_seq;
  a.page_len = dims->page_size;
  a.block = block_of(dims);
  a.num_phys = dims->num_phys_pages;
  a.max_mask_len = dims->max_mask_len;
  return cosa_osk::launch_validate(a, stream) == hipSuccess ? COSA_OK : COSA_ERR_HIP;
}

}  // extern "C"
