// Kernel-aware proxy (KAP) computation-order mask for gfx950.
//
// Method: CoSA section 4.2 ("Block ranking", Eq. (8)-(12); "Flag-grouped
// sorting", Eq. (13)-(14)) and Appendix C (Figure A; Algorithm A, the pre-kernel
// proxy): stride-downsampled queries and keys, causal softmax scores, MaxPool over
// each key block's sampled keys, MaxNorm per sampled query row, block score and
// HRM flag per (query block, key block), HRM-first sort, stage-1 selection.
//
// The softmax normaliser of Eq. (8) cancels in the MaxNorm of Eq. (10): with m_rj
// the largest visible sampled logit of key block j for sampled row r and M_r the
// row's largest overall, Pbar[r, j] = exp(m_rj - M_r), and the row's MaxNorm is 1
// exactly in the block(s) where m_rj == M_r.  So two passes over the sampled
// logits suffice: the row maxima, then the block maxima against them.
//
// Kernels:
//   kap_score  one wave per KV head and BPW consecutive query blocks of a
//              sequence; their G heads x (64/stride) sampled rows per block fill
//              the 32 columns of S^T = K~ Q~^T tiles (v_mfma_f32_32x32x16_bf16,
//              32 sampled keys per tile, read through the page table).  Pass 1:
//              row maxima; pass 2: the same logits again (bitwise the same), block
//              maxima, Pbar, the block sums over rows and heads, the HRM flags.
//   kap_select one workgroup per (query block, KV head): the causal candidates'
//              keys (HRM flag, score descending, id ascending) sorted bitonically
//              in LDS; a fixed fraction or Top-p count; the mask row.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "osk_internal.h"

namespace cosa_osk {

typedef __attribute__((ext_vector_type(8))) __bf16 kbf16x8_t;
typedef __attribute__((ext_vector_type(16))) float kf32x16_t;
typedef __attribute__((ext_vector_type(4))) int ki32x4_t;

constexpr float kKapLog2e = 1.442695040888963407f;

__device__ __forceinline__ float kap_partner_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One wave: query blocks i0 .. i0+BPW-1 of sequence `seq` (fewer at its end) and KV
// head g.  Lane l holds query column n = l % 32 of the S^T tiles: block i0 + n / RB,
// head n % RB / PER of the group, sampled row n % PER of the block; its 16
// accumulator entries are the keys m = 8 (e / 4) + 4 (l / 32) + e % 4 of the tile.
template <int PER>
__global__ __launch_bounds__(64) void kap_score_kernel(const KapArgs a, int G) {
  const int RB = G * PER;  // sampled rows per query block (all heads of the group)
  const int BPW = 32 / RB;
  const int gi = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  int seq = 0, base = 0;
  for (; seq < a.num_seqs; ++seq) {
    const int nb = a.cu_qblocks[seq + 1] - a.cu_qblocks[seq];
    const int ng = (nb + BPW - 1) / BPW;
    if (gi < base + ng) break;
    base += ng;
  }
  if (seq >= a.num_seqs) return;  // the grid is an upper bound on the group count
  const int qb_seq = a.cu_qblocks[seq];
  const int nqb = a.cu_qblocks[seq + 1] - qb_seq;
  const int i0 = (gi - base) * BPW;
  const int tok0 = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - tok0;
  const int R = (L + a.stride - 1) / a.stride;  // sampled positions of the sequence
  const int32_t* pt = a.page_table + (int64_t)seq * a.max_pages;

  const int n = lane & 31, hi = lane >> 5;
  const int blk = n / RB, within = n % RB;
  const int hh = within / PER, sr = within % PER;
  const int i = i0 + blk;
  const int r = i * PER + sr;  // this column's sampled query position
  const bool row_ok = blk < BPW && i < nqb && i < a.max_pages && r < R;

  kbf16x8_t qf[8];
  {
    const uint16_t* qrow =
        a.q + (int64_t)(tok0 + (int64_t)r * a.stride) * a.q_st + (int64_t)(g * G + hh) * a.q_sh + hi * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      ki32x4_t x = {0, 0, 0, 0};
      if (row_ok) x = *(const ki32x4_t*)(qrow + c * 16);
      qf[c] = __builtin_bit_cast(kbf16x8_t, x);
    }
  }
  const int i_last = min(min(i0 + BPW, nqb), a.max_pages) - 1;
  const int c_end = min(R, (i_last + 1) * PER);  // sampled keys any column may see
  const int n_tiles = (c_end + 31) / 32;

  // S^T tile kt: keys 32 kt + m for the lane's 16 entries, in scaled-logit units
  auto tile = [&](int kt, kf32x16_t& acc) {
    const int c = 32 * kt + n;  // the key this lane loads (A operand row)
    bool k_ok = c < R;
    int64_t off = 0;
    if (k_ok) {
      const int t = c * a.stride;
      const int page = t / kPage;
      const int ph = page < a.max_pages ? pt[page] : -1;
      k_ok = ph >= 0 && ph < a.num_phys;
      off = (int64_t)ph * a.kv_sp + (int64_t)g * a.kv_sh + (int64_t)(t % kPage) * a.kv_st + hi * 8;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      ki32x4_t x = {0, 0, 0, 0};
      if (k_ok) x = *(const ki32x4_t*)(a.k + off + cc * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(kbf16x8_t, x), qf[cc], acc, 0, 0, 0);
    }
  };
  // visibility of entry e of tile kt for this lane's column: sample c <= r (for a valid
  // column r < R, so the key is a sample of the sequence)
  auto visible = [&](int kt, int e) { return 32 * kt + 8 * (e >> 2) + 4 * hi + (e & 3) <= r; };

  // ---- pass 1: row maxima over the causal sampled keys
  float M = -INFINITY;
  for (int kt = 0; kt < n_tiles; ++kt) {
    kf32x16_t acc;
    tile(kt, acc);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (visible(kt, e)) M = fmaxf(M, acc[e] * a.sm_scale);
  }
  M = kap_partner_max(M);

  // ---- pass 2: block maxima, Pbar = exp(m_rj - M_r), sums over the block's rows, flags
  float* srow = a.score_rows + ((int64_t)(qb_seq + i) * a.hkv + g) * a.max_pages;
  uint8_t* frow = a.flag_rows + ((int64_t)(qb_seq + i) * a.hkv + g) * a.max_pages;
  for (int kt = 0; kt < n_tiles; ++kt) {
    kf32x16_t acc;
    tile(kt, acc);
    // the lane's key blocks in this tile: PER = 4: block 8 kt + 2 q + hi from entries
    // 4q .. 4q+3; PER = 8: block 4 kt + q from entries 4q .. 4q+3 of both lanes l, l^32
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      float mb = -INFINITY;
#pragma unroll
      for (int e = 4 * qq; e < 4 * qq + 4; ++e)
        if (visible(kt, e)) mb = fmaxf(mb, acc[e] * a.sm_scale);
      if (PER == 8) mb = kap_partner_max(mb);
      const int j = PER == 4 ? 8 * kt + 2 * qq + hi : 4 * kt + qq;
      const bool owner = row_ok && (PER == 4 || hi == 0);
      float pbar = 0.f;
      int hrm = 0;
      if (owner && mb != -INFINITY) {
        pbar = exp2f((mb - M) * kKapLog2e);
        hrm = (mb == M) ? 1 : 0;
      }
      // sum and OR over the RB columns of the query block (consecutive lanes)
#pragma unroll
      for (int w = 1; w < 32; w <<= 1) {
        if (w < RB) {
          pbar += __shfl_xor(pbar, w, 64);
          hrm |= __shfl_xor(hrm, w, 64);
        }
      }
      if (row_ok && within == 0 && (PER == 4 || hi == 0) && j <= i) {
        srow[j] = pbar;
        frow[j] = (uint8_t)hrm;
      }
    }
  }
}

// ascending key == (HRM flag set first, score descending, id ascending); scores are >= 0
__device__ __forceinline__ uint64_t kap_key(float s, int hrm, int id) {
  const uint32_t b = __float_as_uint(s) & 0x7fffffffu;
  const uint32_t hw = (hrm ? 0u : 0x80000000u) | (~b & 0x7fffffffu);
  return ((uint64_t)hw << 32) | (uint32_t)id;
}
__device__ __forceinline__ float kap_key_score(uint64_t k) {
  return __uint_as_float(~(uint32_t)(k >> 32) & 0x7fffffffu);
}

// dynamic LDS: keys [cap] uint64, then csum [cap] float (cap a power of two >= max_pages)
__global__ __launch_bounds__(256) void kap_select_kernel(const KapArgs a, int cap) {
  extern __shared__ uint64_t keys[];
  float* csum = reinterpret_cast<float*>(keys + cap);
  __shared__ float part[256];
  __shared__ int s_below;
  const int qb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  int lo = 0, hi_s = a.num_seqs;
  while (hi_s - lo > 1) {
    const int mid = (lo + hi_s) >> 1;
    if (a.cu_qblocks[mid] <= qb) lo = mid; else hi_s = mid;
  }
  const int i = min(qb - a.cu_qblocks[lo], a.max_pages - 1);
  const int n = i + 1;  // causal candidates
  int N = 1;
  while (N < n) N <<= 1;
  const int64_t rowoff = ((int64_t)qb * a.hkv + g) * a.max_pages;
  for (int j = tid; j < N; j += 256) keys[j] = j < n ? kap_key(a.score_rows[rowoff + j], a.flag_rows[rowoff + j], j) : ~0ull;
  if (tid == 0) s_below = 0;
  __syncthreads();
  for (int kk = 2; kk <= N; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int x = tid; x < N; x += 256) {
        const int y = x ^ jj;
        if (y > x) {
          const uint64_t p = keys[x], q = keys[y];
          const bool up = (x & kk) == 0;
          if ((p > q) == up) { keys[x] = q; keys[y] = p; }
        }
      }
      __syncthreads();
    }
  }
  int kcount;
  if (a.mode == 0) {
    kcount = max(1, min(n, (int)ceil((double)a.budget * (double)n - 1e-3)));
  } else {
    // inclusive prefix sums of the sorted scores: each thread sums a contiguous run,
    // a scan over the 256 run totals, then the runs again with their offsets
    const int per = (n + 255) / 256;
    const int x0 = tid * per, x1 = min(n, x0 + per);
    float run = 0.f;
    for (int x = x0; x < x1; ++x) run += kap_key_score(keys[x]);
    part[tid] = run;
    __syncthreads();
    for (int w = 1; w < 256; w <<= 1) {
      const float v = tid >= w ? part[tid - w] : 0.f;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    float acc = tid > 0 ? part[tid - 1] : 0.f;
    for (int x = x0; x < x1; ++x) {
      acc += kap_key_score(keys[x]);
      csum[x] = acc;
    }
    __syncthreads();
    const float thr = a.budget * part[255];
    int below = 0;
    for (int x = x0; x < x1; ++x) below += csum[x] < thr ? 1 : 0;
    if (below) atomicAdd(&s_below, below);
    __syncthreads();
    kcount = max(1, min(n, s_below + 1));
  }
  int32_t* row = a.order_mask + ((int64_t)qb * a.hkv + g) * a.max_mask_len;
  const int kw = min(kcount, a.max_mask_len);
  for (int x = tid; x < a.max_mask_len; x += 256) row[x] = x < kw ? (int32_t)(keys[x] & 0xffffffffu) : -1;
  if (tid == 0) a.mask_len[(int64_t)qb * a.hkv + g] = kw;
  // the caller's copies: nothing past the causal candidates
  if (a.scores_out)
    for (int j = n + tid; j < a.max_pages; j += 256) a.scores_out[rowoff + j] = __builtin_nanf("");
  if (a.flags_out)
    for (int j = n + tid; j < a.max_pages; j += 256) a.flags_out[rowoff + j] = 0;
}

hipError_t launch_build_kap_mask(const KapArgs& a, hipStream_t stream) {
  if (a.total_qblocks == 0) return hipSuccess;
  const int G = a.hq / a.hkv;
  const int per = kPage / a.stride;
  const int bpw = 32 / (G * per);
  const dim3 sgrid((unsigned)(a.total_qblocks / bpw + a.num_seqs), (unsigned)a.hkv);
  if (per == 4)
    hipLaunchKernelGGL(kap_score_kernel<4>, sgrid, dim3(64), 0, stream, a, G);
  else
    hipLaunchKernelGGL(kap_score_kernel<8>, sgrid, dim3(64), 0, stream, a, G);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int cap = 1;
  while (cap < a.max_pages) cap <<= 1;
  hipLaunchKernelGGL(kap_select_kernel, dim3((unsigned)a.total_qblocks, (unsigned)a.hkv), dim3(256),
                     (size_t)cap * (sizeof(uint64_t) + sizeof(float)), stream, a, cap);
  return hipGetLastError();
}

}  // namespace cosa_osk
