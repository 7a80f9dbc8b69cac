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
//              sequence; their G heads x (block/stride) sampled rows per block fill
//              the 32 columns of S^T = K~ Q~^T tiles (v_mfma_f32_32x32x16_bf16,
//              32 sampled keys per tile, read through the page table).  Pass 1:
//              row maxima; pass 2: the same logits again (bitwise the same), block
//              maxima, Pbar, the block sums over rows and heads (DPP row sums),
//              the HRM flags.
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
#ifndef KAP_COLUMN_TILES
#define KAP_COLUMN_TILES 2
#endif
constexpr int kKapColumnTiles = KAP_COLUMN_TILES;  // column tiles of 32 query rows per wave

__device__ __forceinline__ float kap_partner_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Windowed sums over lane groups of rb = 2^k consecutive lanes with DPP row shifts
// (bound_ctrl: lanes shifted in from outside the row read 0): the last lane of each
// group ends with the group's total.  For rb = 32 a group is one half of the wave (two
// 16-lane rows): the last lanes of its two rows are added, per half.
__device__ __forceinline__ float group_sum(float v, int rb, int hi) {
  if (rb > 1) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
  if (rb > 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
  if (rb > 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
  if (rb > 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
  if (rb > 16) {
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float up = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    v = hi ? up : lo;
  }
  return v;
}
__device__ __forceinline__ int group_or(int v, int rb, int hi) {
  if (rb > 1) v |= __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  if (rb > 2) v |= __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  if (rb > 4) v |= __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  if (rb > 8) v |= __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  if (rb > 16) {
    const int lo = __builtin_amdgcn_readlane(v, 15) | __builtin_amdgcn_readlane(v, 31);
    const int up = __builtin_amdgcn_readlane(v, 47) | __builtin_amdgcn_readlane(v, 63);
    v = hi ? up : lo;
  }
  return v;
}

// One wave: query blocks i0 .. i0 + CT*BPW - 1 of sequence `seq` (fewer at its end)
// and KV head g, as CT column tiles of 32.  In tile ct, lane l holds query column
// n = l % 32: block i0 + ct*BPW + n / RB, head n % RB / PER of the group, sampled row
// n % PER of the block; its 16 accumulator entries are the keys
// m = 8 (e / 4) + 4 (l / 32) + e % 4 of the key tile.  Each key tile's operands are
// read once and feed the CT column tiles.
template <int PER, int CT>
__global__ __launch_bounds__(64) void kap_score_kernel(const KapArgs a, int G) {
  const int RB = G * PER;  // sampled rows per query block (all heads of the group)
  const int BPW = 32 / RB;
  const int gi = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  int seq = 0, base = 0;
  for (; seq < a.num_seqs; ++seq) {
    const int nb = a.cu_qblocks[seq + 1] - a.cu_qblocks[seq];
    const int ng = (nb + CT * BPW - 1) / (CT * BPW);
    if (gi < base + ng) break;
    base += ng;
  }
  if (seq >= a.num_seqs) return;  // the grid is an upper bound on the group count
  const int qb_seq = a.cu_qblocks[seq];
  const int nqb = a.cu_qblocks[seq + 1] - qb_seq;
  const int i0 = (gi - base) * CT * BPW;
  const int tok0 = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - tok0;
  const int R = (L + a.stride - 1) / a.stride;  // sampled positions of the sequence
  const int32_t* pt = a.page_table + (int64_t)seq * a.pt_stride;

  const int n = lane & 31, hi = lane >> 5;
  const int within = n % RB;
  const int hh = within / PER, sr = within % PER;
  int i[CT], r[CT];
  bool row_ok[CT], blk_ok[CT];
  kbf16x8_t qf[CT][8];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    i[ct] = i0 + ct * BPW + n / RB;
    r[ct] = i[ct] * PER + sr;  // this column's sampled query position
    blk_ok[ct] = n / RB < BPW && i[ct] < nqb && i[ct] < a.max_pages;  // the column's query block exists
    row_ok[ct] = blk_ok[ct] && r[ct] < R;                               // and so does its sampled row
    const uint16_t* qrow =
        a.q + (int64_t)(tok0 + (int64_t)r[ct] * a.stride) * a.q_st + (int64_t)(g * G + hh) * a.q_sh + hi * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      ki32x4_t x = {0, 0, 0, 0};
      if (row_ok[ct]) x = *(const ki32x4_t*)(qrow + c * 16);
      qf[ct][c] = __builtin_bit_cast(kbf16x8_t, x);
    }
  }
  const int i_last = min(min(i0 + CT * BPW, nqb), a.max_pages) - 1;
  const int c_end = min(R, (i_last + 1) * PER);  // sampled keys any column may see
  const int n_tiles = (c_end + 31) / 32;

  // S^T tiles kt (keys 32 kt + m of the lane's 16 entries) for the CT column tiles
  auto tile = [&](int kt, kf32x16_t (&acc)[CT]) {
    const int c = 32 * kt + n;  // the key this lane loads (A operand row)
    bool k_ok = c < R;
    int64_t off = 0;
    if (k_ok) {
      const int t = c * a.stride;
      const int page = t / a.page_len;  // physical page of token t
      const int ph = page < a.pt_stride ? pt[page] : -1;
      k_ok = ph >= 0 && ph < a.num_phys;
      off = (int64_t)ph * a.kv_sp + (int64_t)g * a.kv_sh + (int64_t)(t % a.page_len) * a.kv_st + hi * 8;
    }
    kbf16x8_t ka[8];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      ki32x4_t x = {0, 0, 0, 0};
      if (k_ok) x = *(const ki32x4_t*)(a.k + off + cc * 16);
      ka[cc] = __builtin_bit_cast(kbf16x8_t, x);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][e] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cc], qf[ct][cc], acc[ct], 0, 0, 0);
    }
  };
  // entry e of tile kt is visible to column r iff its key sample c <= r (for a valid
  // column r < R, so the key is a sample of the sequence)
  auto key_of = [&](int kt, int e) { return 32 * kt + 8 * (e >> 2) + 4 * hi + (e & 3); };

  // ---- pass 1: row maxima over the causal sampled keys
  float M[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) M[ct] = -INFINITY;
  for (int kt = 0; kt < n_tiles; ++kt) {
    kf32x16_t acc[CT];
    tile(kt, acc);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (key_of(kt, e) <= r[ct]) M[ct] = fmaxf(M[ct], acc[ct][e] * a.sm_scale);
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) M[ct] = kap_partner_max(M[ct]);

  // ---- pass 2: block maxima, Pbar = exp(m_rj - M_r), sums over the block's rows, flags
  for (int kt = 0; kt < n_tiles; ++kt) {
    kf32x16_t acc[CT];
    tile(kt, acc);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float* srow = a.score_rows + ((int64_t)(qb_seq + i[ct]) * a.hkv + g) * a.max_pages;
      uint8_t* frow = a.flag_rows + ((int64_t)(qb_seq + i[ct]) * a.hkv + g) * a.max_pages;
      // the lane's key blocks in this tile: PER = 4: block 8 kt + 2 q + hi from entries
      // 4q .. 4q+3; PER = 8: block 4 kt + q from entries 4q .. 4q+3 of both lanes l, l^32
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        float mb = -INFINITY;
#pragma unroll
        for (int e = 4 * qq; e < 4 * qq + 4; ++e)
          if (key_of(kt, e) <= r[ct]) mb = fmaxf(mb, acc[ct][e] * a.sm_scale);
        if (PER == 8) mb = kap_partner_max(mb);
        const int j = PER == 4 ? 8 * kt + 2 * qq + hi : 4 * kt + qq;
        const bool owner = row_ok[ct] && (PER == 4 || hi == 0);
        float pbar = 0.f;
        int hrm = 0;
        if (owner && mb != -INFINITY) {
          pbar = exp2f((mb - M[ct]) * kKapLog2e);
          hrm = (mb == M[ct]) ? 1 : 0;
        }
        // sum and OR over the RB columns of the query block: consecutive lanes, an
        // aligned group inside a 16-lane DPP row (RB <= 16) or two such rows (RB = 32)
        pbar = group_sum(pbar, RB, hi);
        hrm = group_or(hrm, RB, hi);
        // the group's last lane writes (its own sampled row may lie past the sequence end)
        if (blk_ok[ct] && within == RB - 1 && (PER == 4 || hi == 0) && j <= i[ct]) {
          srow[j] = pbar;
          frow[j] = (uint8_t)hrm;
        }
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
  const int per = a.block / a.stride;  // sampled rows and keys per logical block: 4 or 8
  const int bpw = 32 / (G * per) * kKapColumnTiles;  // query blocks per wave
  const dim3 sgrid((unsigned)(a.total_qblocks / bpw + a.num_seqs), (unsigned)a.hkv);
  if (per == 4)
    hipLaunchKernelGGL((kap_score_kernel<4, kKapColumnTiles>), sgrid, dim3(64), 0, stream, a, G);
  else
    hipLaunchKernelGGL((kap_score_kernel<8, kKapColumnTiles>), sgrid, dim3(64), 0, stream, a, G);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int cap = 1;
  while (cap < a.max_pages) cap <<= 1;
  hipLaunchKernelGGL(kap_select_kernel, dim3((unsigned)a.total_qblocks, (unsigned)a.hkv), dim3(256),
                     (size_t)cap * (sizeof(uint64_t) + sizeof(float)), stream, a, cap);
  return hipGetLastError();
}

}  // namespace cosa_osk
