// Computation-order mask from the mean-pooled q.k proxy, for gfx950.
//
// Mask format: CoSA section 4.2, Eq. (14) -- row i lists the kept logical page
// ids in visit order, -1 after them.  Proxy: the dot product of mean-pooled
// query-block and key-page representations, kept pages visited in descending
// proxy order (the CoSA rewrite page, section 4.2 "Implementation").  Grouped
// q heads share one page set per KV head (PageWeaver notes, section 2), so the
// query representation of KV head g sums the group's per-head block means.
//
// Kernels:
//   pool   one workgroup per (query block, KV head):
//          qbar = sum_h mean_r q, kbar = mean_t k of the same-index logical block
//          (64 or 128 tokens);
//          Q and K are each read once in 16-byte chunks along the head dimension.
//   score  one workgroup per 8 consecutive query blocks of a sequence and a KV
//          head: fp32 scores of the causal pages, each pooled key row read once
//          for the 8 blocks; rows go to the caller's proxy_scores or workspace.
//   select one workgroup per (query block, KV head): a radix select finds the
//          n_keep-th key of the non-forced candidates by (score desc, id asc); the
//          kept and forced keys are then bitonic-sorted in LDS.
//
// Per-q-head sets (PageWeaver notes, section 2.2: the heads of a group traverse the
// union of their sets, a membership mask keeping each head to its own): each q head
// selects its own set by the same rule from its own score qbar_h . kbar (qbar_h its
// block mean); the KV head's row is the union, visited in the group-score order of
// the shared mask, with membership[qb, h, k] = 1 iff entry k is in head h's set.
//   pool_heads  one workgroup per (query block, KV head): the G per-head means;
//   score       the score kernel above over per-head rows;
//   union       one workgroup per (query block, KV head): a radix select over the
//               G heads' candidates (their own scores; the heads share the digit
//               passes) marks each head's top n_keep, then one sort of the union's
//               members by the group score writes the row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "osk_internal.h"
#include "block_select.h"

namespace cosa_osk {

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ int seq_of_qblock(const int32_t* cu_qblocks, int num_seqs, int qb) {
  int lo = 0, hi = num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_qblocks[mid] <= qb) lo = mid; else hi = mid;
  }
  return lo;
}

// Thread t handles dims 8*(t%16) .. +8 (one 16-byte load per row) of rows
// t/16, t/16 + 16, ...; the 16 row groups' partial sums are combined in LDS.
__global__ __launch_bounds__(256) void mask_pool_kernel(const BuilderArgs a) {
  __shared__ float red[16][kHeadDim];
  const int qb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int chunk = tid & 15, rg = tid >> 4;
  const int s = seq_of_qblock(a.cu_qblocks, a.num_seqs, qb);
  const int i = qb - a.cu_qblocks[s];
  const int tok0 = a.cu_seqlens[s];
  const int L = a.cu_seqlens[s + 1] - tok0;
  const int rows = min(a.block, L - i * a.block);
  const int G = a.hq / a.hkv;
  auto add8 = [](float (&acc)[8], const uint16_t* p) {
    const uint4 w = *(const uint4*)p;
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(u[e] << 16);
      acc[2 * e + 1] += __uint_as_float(u[e] & 0xffff0000u);
    }
  };
  // ---- qbar: sum over the group's heads of the block mean
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < G; ++hh) {
    const uint16_t* qh = a.q + (int64_t)tok0 * a.q_st + (int64_t)(g * G + hh) * a.q_sh + chunk * 8;
    for (int r = rg; r < rows; r += 16) add8(acc, qh + (int64_t)(i * a.block + r) * a.q_st);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][chunk * 8 + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float t = 0.f;
    for (int x = 0; x < 16; ++x) t += red[x][tid];
    a.qbar[((int64_t)qb * a.hkv + g) * kHeadDim + tid] = t / (float)rows;
  }
  __syncthreads();
  // ---- kbar: mean of the same-index logical block's keys (through its physical pages)
  const int32_t* pt_row = a.page_table + (int64_t)s * a.pt_stride;
  int ph[kMaxBlockPages];
  const bool has_page = i < a.max_pages && block_phys(pt_row, a.pt_stride, i, L, a.page_len, a.block, a.num_phys, ph);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (has_page) {
    for (int t = rg; t < rows; t += 16) {
      const uint16_t* kp = a.k + (int64_t)ph[t / a.page_len] * a.kv_sp + (int64_t)g * a.kv_sh + chunk * 8;
      add8(acc, kp + (int64_t)(t % a.page_len) * a.kv_st);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][chunk * 8 + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float t = 0.f;
    for (int x = 0; x < 16; ++x) t += red[x][tid];
    a.kbar[((int64_t)g * kHeadDim + tid) * a.total_qblocks + qb] = has_page ? t / (float)rows : 0.f;
  }
}

// Each q head's block mean: thread t handles dims 8*(t%16) .. +8 of rows t/16, +16, ...
__global__ __launch_bounds__(256) void mask_pool_heads_kernel(const BuilderArgs a) {
  __shared__ float red[16][kHeadDim];
  const int qb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int chunk = tid & 15, rg = tid >> 4;
  const int s = seq_of_qblock(a.cu_qblocks, a.num_seqs, qb);
  const int i = qb - a.cu_qblocks[s];
  const int tok0 = a.cu_seqlens[s];
  const int L = a.cu_seqlens[s + 1] - tok0;
  const int rows = min(a.block, L - i * a.block);
  const int G = a.hq / a.hkv;
  for (int hh = 0; hh < G; ++hh) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* qh = a.q + (int64_t)tok0 * a.q_st + (int64_t)(g * G + hh) * a.q_sh + chunk * 8;
    for (int r = rg; r < rows; r += 16) {
      const uint4 w = *(const uint4*)(qh + (int64_t)(i * a.block + r) * a.q_st);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(u[e] << 16);
        acc[2 * e + 1] += __uint_as_float(u[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][chunk * 8 + e] = acc[e];
    __syncthreads();
    if (tid < kHeadDim) {
      float t = 0.f;
      for (int x = 0; x < 16; ++x) t += red[x][tid];
      a.qbar_heads[((int64_t)qb * a.hq + g * G + hh) * kHeadDim + tid] = t / (float)rows;
    }
    __syncthreads();
  }
}

// Query blocks per score workgroup: each pooled key row is read once for the group.
constexpr int kScoreGroup = 8;

// score_j = qbar . kbar_j (fp32, dims in order) for the causal pages j <= i of
// kScoreGroup consecutive query blocks of one sequence and score row r; rows are
// written for j <= i only.  HEADS = false: r = KV head g (the group's pooled query,
// score_rows); HEADS = true: r = q head h of KV head h / G (qbar_heads, head_score_rows).
template <bool HEADS>
__global__ __launch_bounds__(256) void mask_score_kernel(const BuilderArgs a) {
  __shared__ float qs[kScoreGroup][kHeadDim];
  const int gi = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int nr = HEADS ? a.hq : a.hkv;                 // score rows per query block
  const int g = HEADS ? r / (a.hq / a.hkv) : r;        // the KV head of row r
  const float* qsrc = HEADS ? a.qbar_heads : a.qbar;
  float* dst = HEADS ? a.head_score_rows : a.score_rows;
  // the sequence of group gi (groups do not straddle sequences)
  int s = 0, base = 0;
  for (; s < a.num_seqs; ++s) {
    const int ng = (a.cu_qblocks[s + 1] - a.cu_qblocks[s] + kScoreGroup - 1) / kScoreGroup;
    if (gi < base + ng) break;
    base += ng;
  }
  if (s >= a.num_seqs) return;  // the grid is an upper bound on the group count
  const int qb0 = a.cu_qblocks[s];
  const int i0 = (gi - base) * kScoreGroup;
  const int ng = min(kScoreGroup, a.cu_qblocks[s + 1] - qb0 - i0);
  for (int x = tid; x < kScoreGroup * kHeadDim; x += 256) {
    const int q = x / kHeadDim, d = x % kHeadDim;
    qs[q][d] = q < ng ? qsrc[((int64_t)(qb0 + i0 + q) * nr + r) * kHeadDim + d] : 0.f;
  }
  __syncthreads();
  // block indices are clamped to the page-table width as in the select kernel
  const int jmax = min(i0 + ng - 1, a.max_pages - 1);
  // kbar is stored dims-major ([hkv, 128, total_qblocks]): for each dim, consecutive
  // threads read consecutive blocks' values
  const float* kcol = a.kbar + (int64_t)g * kHeadDim * a.total_qblocks + qb0;
  for (int j = tid; j <= jmax; j += 256) {
    float acc[kScoreGroup];
#pragma unroll
    for (int q = 0; q < kScoreGroup; ++q) acc[q] = 0.f;
#pragma unroll 8
    for (int d = 0; d < kHeadDim; ++d) {
      const float kv = kcol[(int64_t)d * a.total_qblocks + j];
#pragma unroll
      for (int q = 0; q < kScoreGroup; ++q) acc[q] = fmaf(qs[q][d], kv, acc[q]);
    }
#pragma unroll
    for (int q = 0; q < kScoreGroup; ++q)
      if (q < ng && j <= min(i0 + q, a.max_pages - 1))
        dst[((int64_t)(qb0 + i0 + q) * nr + r) * a.max_pages + j] = acc[q];
  }
}

// ceil(b1 * n - 1e-3) clamped to [0, n]
__device__ __forceinline__ int keep_count(float b1, int n) {
  if (n <= 0) return 0;
  const int k = (int)ceil((double)b1 * (double)n - 1e-3);
  return max(0, min(n, k));
}

// ascending key == (score descending, id ascending)
__device__ __forceinline__ uint64_t sort_key(float score, int id) {
  const uint32_t b = __float_as_uint(score);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);  // increasing in score
  return ((uint64_t)(~ord) << 32) | (uint32_t)id;
}

// One workgroup per (query block, KV head): the top n_keep of the non-forced candidates by
// (score descending, id ascending) are found by a radix select on their keys, then the
// kept and forced candidates -- n_keep + |F| keys -- are sorted by the same key.
// dynamic LDS: [cap uint64: the kept keys][cap uint32: high key words of the candidates];
// cap a power of two >= max_pages
constexpr int kSelectThreads = 256;
__global__ __launch_bounds__(kSelectThreads) void mask_select_kernel(const BuilderArgs a, int cap) {
  extern __shared__ uint64_t keys[];
  uint32_t* hkey = reinterpret_cast<uint32_t*>(keys + cap);
  __shared__ int hist[1][256];
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_k[1];
  __shared__ int s_count;
  const int qb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int s = seq_of_qblock(a.cu_qblocks, a.num_seqs, qb);
  // block index within the sequence; the clamp keeps the candidate list inside the
  // LDS key array even for a cu_qblocks inconsistent with max_pages_per_seq
  const int i = min(qb - a.cu_qblocks[s], a.max_pages - 1);
  const bool f_first = (a.flags & 1u) != 0u;
  const bool f_diag = (a.flags & 2u) != 0u && !(f_first && i == 0);
  const int nf = (f_first ? 1 : 0) + (f_diag ? 1 : 0);
  const int nrest = i + 1 - nf;
  const int nkeep = keep_count(a.budget1, nrest);
  const int r0 = f_first ? 1 : 0;  // rest index r is candidate id r + r0 (the diagonal is last)
  const float* srow = a.score_rows + ((int64_t)qb * a.hkv + g) * a.max_pages;
  for (int r = tid; r < nrest; r += kSelectThreads) hkey[r] = (uint32_t)(sort_key(srow[r + r0], 0) >> 32);
  if (a.scores)
    for (int j = i + 1 + tid; j < a.max_pages; j += kSelectThreads)
      a.scores[((int64_t)qb * a.hkv + g) * a.max_pages + j] = __builtin_nanf("");
  if (tid == 0) s_count = 0;
  __syncthreads();
  if (nkeep > 0 && nkeep < nrest) radix_select<kSelectThreads>(hkey, cap, 1, nrest, r0, nkeep, hist, s_prefix, s_k, tid);
  // the kept keys and the forced ones, compacted (any order) and sorted
  if (nkeep > 0)
    for (int r = tid; r < nrest; r += kSelectThreads) {
      const uint64_t key = ((uint64_t)hkey[r] << 32) | (uint32_t)(r + r0);
      if (nkeep == nrest || key <= s_prefix[0]) keys[atomicAdd(&s_count, 1)] = key;
    }
  if (tid == 0 && f_first) keys[atomicAdd(&s_count, 1)] = sort_key(srow[0], 0);
  if (tid == 1 && f_diag) keys[atomicAdd(&s_count, 1)] = sort_key(srow[i], i);
  __syncthreads();
  const int n = nf + nkeep;
  int N = 1;
  while (N < n) N <<= 1;
  for (int x = n + tid; x < N; x += kSelectThreads) keys[x] = ~0ull;
  __syncthreads();
  bitonic_block<kSelectThreads>(keys, N, tid);
  int32_t* row = a.order_mask + ((int64_t)qb * a.hkv + g) * a.max_mask_len;
  for (int x = tid; x < a.max_mask_len; x += kSelectThreads) row[x] = x < n ? (int32_t)(keys[x] & 0xffffffffu) : -1;
  if (tid == 0) a.mask_len[(int64_t)qb * a.hkv + g] = n;
}

hipError_t launch_build_order_mask(const BuilderArgs& a, hipStream_t stream) {
  if (a.total_qblocks == 0) return hipSuccess;
  const dim3 grid((unsigned)a.total_qblocks, (unsigned)a.hkv);
  hipLaunchKernelGGL(mask_pool_kernel, grid, dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // groups of kScoreGroup blocks per sequence: at most total_qblocks / kScoreGroup + num_seqs
  const dim3 sgrid((unsigned)(a.total_qblocks / kScoreGroup + a.num_seqs), (unsigned)a.hkv);
  hipLaunchKernelGGL(mask_score_kernel<false>, sgrid, dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // sort keys in LDS sized for the longest row (fewer workgroups per CU otherwise)
  int cap = 1;
  while (cap < a.max_pages) cap <<= 1;
  hipLaunchKernelGGL(mask_select_kernel, grid, dim3(kSelectThreads), (size_t)cap * (sizeof(uint64_t) + sizeof(uint32_t)),
                     stream, a, cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// union of per-q-head sets with membership
// ---------------------------------------------------------------------------
constexpr int kUnionThreads = 512;
constexpr int kUnionMaxHeadsPerPass = kSelectMaxSegments;

// One workgroup per (query block, KV head).  A head's set is its forced blocks plus the
// n_keep smallest keys (score descending, id ascending) of its other candidates: the
// n_keep-th smallest key is found exactly by a radix select over the 64-bit keys (eight
// 8-bit passes, the heads of a pass sharing them), so no head's candidates are sorted;
// only the union is sorted, by the group score.
// dynamic LDS: [max(cap * 8, hpp * cap * 4) bytes: the heads' high key words, later the
// union's sort keys][cap uint32: each candidate's head bits]; cap a power of two >= max_pages
__global__ __launch_bounds__(kUnionThreads) void union_select_kernel(const BuilderArgs a, int cap, int hpp) {
  extern __shared__ uint64_t dyn[];
  const size_t region = max((size_t)cap, ((size_t)hpp * cap + 1) / 2);  // uint64 words
  uint64_t* keys = dyn;                                        // union sort keys [cap]
  uint32_t* hkey = reinterpret_cast<uint32_t*>(dyn);           // high key words [hpp][cap]
  uint32_t* bits = reinterpret_cast<uint32_t*>(dyn + region);  // [cap]
  __shared__ int hist[kUnionMaxHeadsPerPass][256];
  __shared__ uint64_t s_prefix[kUnionMaxHeadsPerPass];
  __shared__ int s_k[kUnionMaxHeadsPerPass];
  __shared__ int s_count;
  const int qb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int G = a.hq / a.hkv;
  const int s = seq_of_qblock(a.cu_qblocks, a.num_seqs, qb);
  const int i = min(qb - a.cu_qblocks[s], a.max_pages - 1);
  const bool f_first = (a.flags & 1u) != 0u;
  const bool f_diag = (a.flags & 2u) != 0u && !(f_first && i == 0);
  const int nf = (f_first ? 1 : 0) + (f_diag ? 1 : 0);
  const int nrest = i + 1 - nf;
  const int nkeep = keep_count(a.budget1, nrest);
  const int r0 = f_first ? 1 : 0;  // rest index r is candidate id r + r0 (the diagonal is last)
  const uint32_t all = G >= 32 ? 0xffffffffu : ((1u << G) - 1u);
  for (int j = tid; j <= i; j += kUnionThreads)
    bits[j] = ((f_first && j == 0) || (f_diag && j == i)) ? all : 0u;
  if (tid == 0) s_count = 0;
  for (int h0 = 0; h0 < G; h0 += hpp) {
    const int nh = min(hpp, G - h0);
    __syncthreads();
    for (int x = tid; x < nh * nrest; x += kUnionThreads) {
      const int seg = x / nrest, r = x - seg * nrest;
      const float sc = a.head_score_rows[((int64_t)qb * a.hq + g * G + h0 + seg) * a.max_pages + r + r0];
      hkey[seg * cap + r] = (uint32_t)(sort_key(sc, 0) >> 32);
    }
    __syncthreads();
    if (nkeep > 0 && nkeep < nrest)
      radix_select<kUnionThreads>(hkey, cap, nh, nrest, r0, nkeep, hist, s_prefix, s_k, tid);
    // members: the keys up to the n_keep-th smallest (all of them when n_keep == |R|)
    if (nkeep > 0) {
      for (int x = tid; x < nh * nrest; x += kUnionThreads) {
        const int seg = x / nrest, r = x - seg * nrest;
        const uint64_t key = ((uint64_t)hkey[seg * cap + r] << 32) | (uint32_t)(r + r0);
        if (nkeep == nrest || key <= s_prefix[seg]) atomicOr(&bits[r + r0], 1u << (h0 + seg));
      }
    }
  }
  __syncthreads();
  // the union's members, compacted, then sorted by the group score (descending, id ascending)
  const float* grow = a.score_rows + ((int64_t)qb * a.hkv + g) * a.max_pages;
  for (int j = tid; j <= i; j += kUnionThreads)
    if (bits[j] != 0u) keys[atomicAdd(&s_count, 1)] = sort_key(grow[j], j);
  __syncthreads();
  const int nu = s_count;
  int N2 = 1;
  while (N2 < nu) N2 <<= 1;
  for (int x = nu + tid; x < N2; x += kUnionThreads) keys[x] = ~0ull;
  __syncthreads();
  bitonic_block<kUnionThreads>(keys, N2, tid);
  const int nw = min(nu, a.max_mask_len);
  int32_t* row = a.order_mask + ((int64_t)qb * a.hkv + g) * a.max_mask_len;
  for (int x = tid; x < a.max_mask_len; x += kUnionThreads) {
    const int id = x < nw ? (int)(keys[x] & 0xffffffffu) : -1;
    row[x] = id;
    const uint32_t b = id >= 0 ? bits[id] : 0u;
    for (int hh = 0; hh < G; ++hh)
      a.membership[((int64_t)qb * a.hq + g * G + hh) * a.max_mask_len + x] = (uint8_t)((b >> hh) & 1u);
  }
  if (tid == 0) a.mask_len[(int64_t)qb * a.hkv + g] = nw;
  if (tid < G) a.head_len[(int64_t)qb * a.hq + g * G + tid] = nf + nkeep;
}

hipError_t launch_build_union_mask(const BuilderArgs& a, hipStream_t stream) {
  if (a.total_qblocks == 0) return hipSuccess;
  const dim3 grid((unsigned)a.total_qblocks, (unsigned)a.hkv);
  hipLaunchKernelGGL(mask_pool_kernel, grid, dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mask_pool_heads_kernel, grid, dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned ngroups = (unsigned)(a.total_qblocks / kScoreGroup + a.num_seqs);
  hipLaunchKernelGGL(mask_score_kernel<false>, dim3(ngroups, (unsigned)a.hkv), dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(mask_score_kernel<true>, dim3(ngroups, (unsigned)a.hq), dim3(256), 0, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  int cap = 1;
  while (cap < a.max_pages) cap <<= 1;
  // heads selected together per pass: as many as fit their high key words in 32 KiB
  const int G = a.hq / a.hkv;
  const int hpp = max(1, min(min(G, kUnionMaxHeadsPerPass), (int)((32u << 10) / ((size_t)cap * 4))));
  const size_t region = std::max((size_t)cap, ((size_t)hpp * cap + 1) / 2) * sizeof(uint64_t);
  hipLaunchKernelGGL(union_select_kernel, grid, dim3(kUnionThreads), region + (size_t)cap * sizeof(uint32_t), stream,
                     a, cap, hpp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// validator: counts malformed mask entries (they are not visited by the prefill)
// ---------------------------------------------------------------------------
__global__ void zero_counts_kernel(int32_t* c, int n) {
  if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}

__global__ __launch_bounds__(64) void validate_kernel(const ValidateArgs a) {
  __shared__ uint32_t seen[kMaxPagesPerSeq / 32];
  const int qb = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  const int s = seq_of_qblock(a.cu_qblocks, a.num_seqs, qb);
  const int i = qb - a.cu_qblocks[s];
  const int L = a.cu_seqlens[s + 1] - a.cu_seqlens[s];
  const int n_pages = min((L + a.block - 1) / a.block, a.max_pages);
  int len = a.mask_len[(int64_t)qb * a.hkv + g];
  int c_range = 0, c_causal = 0, c_dup = 0, c_len = 0, c_phys = 0;
  if (len < 0 || len > a.max_mask_len) {
    c_len = lane == 0 ? 1 : 0;
    len = min(max(len, 0), a.max_mask_len);
  }
  for (int x = lane; x < (n_pages + 31) / 32; x += 64) seen[x] = 0u;
  __syncthreads();
  const int32_t* row = a.order_mask + ((int64_t)qb * a.hkv + g) * a.max_mask_len;
  for (int k = lane; k < len; k += 64) {
    const int id = row[k];
    if (id < 0 || id >= n_pages) { ++c_range; continue; }
    if (id > i) ++c_causal;
    const uint32_t bit = 1u << (id & 31);
    if (atomicOr(&seen[id >> 5], bit) & bit) ++c_dup;
    int ph[kMaxBlockPages];
    if (!block_phys(a.page_table + (int64_t)s * a.pt_stride, a.pt_stride, id, L, a.page_len, a.block, a.num_phys,
                    ph))
      ++c_phys;
  }
  // reduce over the wave, one atomic per counter
  const int vals[5] = {c_range, c_causal, c_dup, c_len, c_phys};
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    int v = vals[c];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&a.bad[c], v);
  }
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, stream, a.bad, 5);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.total_qblocks == 0) return err;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)a.total_qblocks, (unsigned)a.hkv), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace cosa_osk
