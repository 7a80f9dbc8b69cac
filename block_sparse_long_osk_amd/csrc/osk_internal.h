// Launch interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cosa_osk {

// Blocks, tiles and pages.  The logical block (query block, key block, unit of a skip
// vote) holds `block` = 64 or 128 tokens; the KV cache's physical pages hold page_len =
// 16, 32, 64 (or 128, for 128-token blocks) tokens.  Logical block j of a sequence is
// its tokens block*j .. block*j + block - 1, token t stored in the physical page of
// page-table entry t / page_len at row t % page_len.  kPage is the height of one K or
// V tile in LDS, 64 tokens: a 64-token block is one tile, a 128-token block two.
// max_pages in the argument blocks below counts logical blocks per sequence; pt_stride
// is the page-table row length.
constexpr int kPage = 64;
constexpr int kMaxBlockPages = 8;        // physical pages of one logical block (128 / 16)
constexpr int kHeadDim = 128;
constexpr int kMaxQBlocks = 16384;       // schedule keys live in LDS
constexpr int kMaxMaskLen = 8191;        // schedule histogram lives in LDS
constexpr int kMaxPagesPerSeq = 16384;   // visited-page bitmap lives in LDS
constexpr int kMaxPagesBuilder = 8192;   // builder sort keys live in LDS

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  const int32_t* cu_seqlens;
  const int32_t* cu_qblocks;
  const int32_t* order_mask;
  const int32_t* mask_len;
  const uint8_t* membership;  // nullable: [total_qblocks, hq, max_mask_len], entry k belongs to q head h
  uint16_t* out;
  float* lse;
  uint8_t* decisions;
  float* margins;
  int32_t* sched;        // workspace: query-block visit order, [total_qblocks]
  int32_t* error_count;  // workspace health word (zeroed by the schedule kernel; 0 after every call)
  int64_t q_st, q_sh, o_st, o_sh, kv_sp, kv_sh, kv_st;
  int32_t num_seqs, hq, hkv, total_qblocks, max_pages, num_phys, max_mask_len;
  int32_t pt_stride, page_len;  // page-table row length; tokens per physical page
  int32_t block;                // tokens per logical block (64 or 128)
  int32_t heads_per_phase;      // KV heads the grid walks together (a divisor of hkv; set by the launcher)
  float sm_scale;
  float delta;
};

struct BuilderArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* page_table;
  const int32_t* cu_seqlens;
  const int32_t* cu_qblocks;
  int32_t* order_mask;
  int32_t* mask_len;
  float* scores;      // nullable (the caller's proxy_scores)
  float* qbar;        // workspace [total_qblocks, hkv, 128]
  float* kbar;        // workspace [hkv, 128, total_qblocks] (dims-major)
  float* score_rows;  // [total_qblocks, hkv, max_pages]: scores, or workspace when scores is null
  // per-q-head sets (union builder only; null otherwise)
  float* qbar_heads;       // workspace [total_qblocks, hq, 128]: each head's block mean
  float* head_score_rows;  // workspace [total_qblocks, hq, max_pages]
  uint8_t* membership;     // [total_qblocks, hq, max_mask_len]
  int32_t* head_len;       // [total_qblocks, hq]
  int64_t q_st, q_sh, kv_sp, kv_sh, kv_st;
  int32_t num_seqs, hq, hkv, total_qblocks, max_pages, num_phys, max_mask_len;
  int32_t pt_stride, page_len, block;
  float budget1;
  uint32_t flags;
};

struct ValidateArgs {
  const int32_t* page_table;
  const int32_t* cu_seqlens;
  const int32_t* cu_qblocks;
  const int32_t* order_mask;
  const int32_t* mask_len;
  int32_t* bad;
  int32_t num_seqs, hkv, total_qblocks, max_pages, num_phys, max_mask_len;
  int32_t pt_stride, page_len, block;
};

struct KapArgs {
  const uint16_t* q;
  const uint16_t* k;
  const int32_t* page_table;
  const int32_t* cu_seqlens;
  const int32_t* cu_qblocks;
  int32_t* order_mask;
  int32_t* mask_len;
  float* scores_out;    // nullable: the caller's copy of the block scores
  uint8_t* flags_out;   // nullable: the caller's copy of the HRM flags
  float* score_rows;    // [total_qblocks, hkv, max_pages]: scores_out, or workspace
  uint8_t* flag_rows;   // [total_qblocks, hkv, max_pages]: flags_out, or workspace
  uint32_t* row_max;    // workspace: [total_qblocks, hkv, G * block / stride] row-maximum codes
  uint16_t* k_tiles;    // workspace: [hkv, tile_slots] packed key tiles (8 KiB each)
  int32_t tile_slots;   // total_qblocks * (block / stride) / 32 + num_seqs
  int64_t q_st, q_sh, kv_sp, kv_sh, kv_st;
  int32_t num_seqs, hq, hkv, total_qblocks, max_pages, num_phys, max_mask_len;
  int32_t pt_stride, page_len, block;
  int32_t stride, mode;
  float budget, sm_scale;
};

// Checked build (compiled with COSA_OSK_CHECKED): the prefill kernels test the index
// invariants they rely on -- schedule positions, mask columns, page-table columns, physical
// page ids, output rows -- and count each violation in the workspace health word, which the
// host reads back after the call (0 when healthy).  The default build compiles the tests away.
#ifdef COSA_OSK_CHECKED
#define COSA_CHECK(args, cond)                              \
  do {                                                      \
    if (!(cond)) atomicAdd((args).error_count, 1);          \
  } while (0)
#else
#define COSA_CHECK(args, cond) \
  do {                         \
  } while (0)
#endif

// Physical pages of logical block j of a sequence (pt_row: its page-table row, n_pt
// entries): the block is usable iff every page holding one of its tokens t < L is a
// valid page id; then ph[0 .. block / page_len - 1] are set (pages past L repeat ph[0]).
__device__ __forceinline__ bool block_phys(const int32_t* pt_row, int n_pt, int j, int L, int page_len, int block,
                                           int num_phys, int* ph) {
  const int sub = block / page_len;
  bool ok = true;
  for (int s = 0; s < sub; ++s) {
    const int t0 = j * block + s * page_len;
    int p = -1;
    if (t0 < L) {
      const int e = j * sub + s;
      p = e < n_pt ? pt_row[e] : -1;
      if (p < 0 || p >= num_phys) ok = false;
    } else {
      p = ph[0];
    }
    ph[s] = p;
  }
  return ok;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Bytes of the library-held prefill scratch (one copy per device): the prefill
// workspace of kMaxQBlocks query blocks (schedule padded to 256 B, then the 256-byte
// status block); and the address of the current device's copy (looked up on the
// first call on each device).
constexpr size_t kNoAllocScratchBytes = ((size_t)kMaxQBlocks * 4 + 1 + 255) / 256 * 256 + 256;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_build_kap_mask(const KapArgs& a, hipStream_t stream);
hipError_t launch_build_order_mask(const BuilderArgs& a, hipStream_t stream);
hipError_t launch_build_union_mask(const BuilderArgs& a, hipStream_t stream);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream);

}  // namespace cosa_osk
