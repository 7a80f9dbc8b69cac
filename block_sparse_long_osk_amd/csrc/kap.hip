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
//   kap_pack   the sampled keys of every sequence and KV head, read once through the
//              page table into 8 KiB tiles of 32 keys in MFMA operand order.
//   kap_rowmax one wave per (KV head, BPW consecutive query blocks of a sequence, chunk
//              of up to 32 key tiles): their G heads x (block/stride) sampled rows per
//              block fill the 32 columns of S^T = K~ Q~^T tiles
//              (v_mfma_f32_32x32x16_bf16, 32 sampled keys per tile); the chunk's
//              partial row maxima, combined over the chunks by an integer atomic max.
//   kap_score  the same units and the same logits again (bitwise the same): block
//              maxima, Pbar, the block sums over rows and heads (DPP row sums), the
//              HRM flags.
//   kap_select one workgroup per (query block, KV head): keys (HRM flag, score
//              descending, id ascending); a fixed fraction by radix select of the kept
//              keys, which alone are sorted; Top-p by a bitonic sort of every candidate
//              and the prefix sums of the sorted scores; the mask row.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "osk_internal.h"
#include "block_select.h"

namespace cosa_osk {

typedef __attribute__((ext_vector_type(8))) __bf16 kbf16x8_t;
typedef __attribute__((ext_vector_type(16))) float kf32x16_t;
typedef __attribute__((ext_vector_type(4))) int ki32x4_t;

constexpr float kKapLog2e = 1.442695040888963407f;
#ifndef KAP_COLUMN_TILES
#define KAP_COLUMN_TILES 2
#endif
constexpr int kKapColumnTiles = KAP_COLUMN_TILES;  // column tiles of 32 query rows per wave

// x * y rounded by itself (never contracted into a following add or subtract)
__device__ __forceinline__ float kap_mul_unfused(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}
__device__ __forceinline__ float kap_partner_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Windowed sums over lane groups of RB = 2^k consecutive lanes with DPP row shifts
// (bound_ctrl: lanes shifted in from outside the row read 0): the last lane of each
// group ends with the group's total.  For RB = 32 a group is one half of the wave (two
// 16-lane rows): the last lanes of its two rows are added, per half.
template <int RB>
__device__ __forceinline__ float group_sum(float v, int hi) {
  if constexpr (RB > 1) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true));
  if constexpr (RB > 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true));
  if constexpr (RB > 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true));
  if constexpr (RB > 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true));
  if constexpr (RB > 16) {
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float up = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47)) +
                     __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    v = hi ? up : lo;
  }
  return v;
}
template <int RB>
__device__ __forceinline__ int group_or(int v, int hi) {
  if constexpr (RB > 1) v |= __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  if constexpr (RB > 2) v |= __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  if constexpr (RB > 4) v |= __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  if constexpr (RB > 8) v |= __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  if constexpr (RB > 16) {
    const int lo = __builtin_amdgcn_readlane(v, 15) | __builtin_amdgcn_readlane(v, 31);
    const int up = __builtin_amdgcn_readlane(v, 47) | __builtin_amdgcn_readlane(v, 63);
    v = hi ? up : lo;
  }
  return v;
}

// Row maxima travel between the two passes as order-preserving unsigned codes (a
// larger float has a larger code), so partial maxima of one row from several key
// ranges combine with an integer atomic max; code 0 lies below every float.
__device__ __forceinline__ uint32_t ord_code(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float ord_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

constexpr int kKapChunkTiles = 32;  // key tiles of 32 sampled keys per work unit

// Packed key tiles.  Tile kt of a sequence holds its sampled keys 32 kt .. 32 kt + 31 in
// MFMA A-operand order: dim chunk cc (16 dims), lane l: key 32 kt + l % 32, dims
// 16 cc + 8 (l / 32) .. +8 -- 8 x 64 x 16 bytes, so each operand load of a wave reads one
// contiguous KiB.  Keys past the sequence's samples, or on a page that is not a valid
// physical page, are zero.  Sequence s owns the tile slots from
// cu_qblocks[s] * PER / 32 + s on (its ceil(R / 32) <= ceil(n_qblocks * PER / 32) tiles
// end before the next sequence's first slot).
constexpr int kKapTileElems = 8 * 64 * 8;  // bf16 elements per packed tile
__device__ __forceinline__ int kap_tile_base(int qb_seq, int per, int seq) { return qb_seq * per / 32 + seq; }

// One wave per (tile slot, KV head): 32 keys x 256 bytes, read as 4 rows per 16-byte
// load round, written to their operand positions.
__global__ __launch_bounds__(64) void kap_pack_kernel(const KapArgs a, int per) {
  const int slot = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  int seq = 0;
  while (seq + 1 < a.num_seqs && kap_tile_base(a.cu_qblocks[seq + 1], per, seq + 1) <= slot) ++seq;
  const int kt = slot - kap_tile_base(a.cu_qblocks[seq], per, seq);
  const int tok0 = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - tok0;
  const int R = (L + a.stride - 1) / a.stride;
  if (kt < 0 || 32 * kt >= R) return;  // a slot past the sequence's tiles: never read
  const int32_t* pt = a.page_table + (int64_t)seq * a.pt_stride;
  uint16_t* dst = a.k_tiles + ((int64_t)g * a.tile_slots + slot) * kKapTileElems;
  const int gran = lane & 15;  // 16-byte granule of the key row: dims 8 gran .. +8
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int m = 4 * x + (lane >> 4);  // key row within the tile
    const int c = 32 * kt + m;
    ki32x4_t v = {0, 0, 0, 0};
    if (c < R) {
      // a key is read only if its logical block is usable (every physical page
      // holding one of the block's tokens is in the pool), as for the mean-pooled
      // proxy and the prefill; otherwise the block has no stored keys and packs zero
      const int t = c * a.stride;
      const int j = t / a.block, sub = a.block / a.page_len;
      bool ok = true;
      for (int x2 = 0; x2 < sub; ++x2) {
        const int t0 = j * a.block + x2 * a.page_len;
        const int e = j * sub + x2;
        const int p = (t0 < L && e < a.pt_stride) ? pt[e] : (t0 < L ? -1 : 0);
        ok = ok && p >= 0 && p < a.num_phys;
      }
      if (ok) {  // then t's own page entry was among those checked, inside the row
        const int ph = pt[t / a.page_len];
        v = *(const ki32x4_t*)(a.k + (int64_t)ph * a.kv_sp + (int64_t)g * a.kv_sh +
                                (int64_t)(t % a.page_len) * a.kv_st + gran * 8);
      }
    }
    // dims 8 gran .. +8 = chunk gran / 2, lane half gran % 2
    *(ki32x4_t*)(dst + ((gran >> 1) * 64 + (gran & 1) * 32 + m) * 8) = v;
  }
}

// One wave's work unit: query blocks i0 .. i0 + CT*BPW - 1 of sequence `seq` (fewer at
// its end), KV head g, and one chunk of at most kKapChunkTiles key tiles of them; the
// KV head is the fastest index of the grid, so that with eight KV heads each XCD's
// L2 serves one head's sampled keys.  In column tile ct, lane l holds query column
// n = l % 32: block i0 + ct*BPW + n / RB, head n % RB / PER of the group, sampled row
// n % PER of the block (RB = G * PER sampled rows per query block); its 16 accumulator
// entries are the keys m = 8 (e / 4) + 4 (l / 32) + e % 4 of the key tile.  Each key
// tile's operands are read once and feed the CT column tiles.
//
// Maxima are taken over the raw dot products and scaled once: for a scale s > 0,
// rounding is monotone, so round(s * max x) equals max round(s * x) bit for bit.  A
// key tile whose last key precedes the unit's first sampled row is visible to every
// column in full, so only the tiles on the diagonal test causality per entry.
template <int PER, int RB, int CT>
struct KapUnit {
  static constexpr int BPW = 32 / RB;
  int g, n, hi, within, qb_seq, R, r_min, t_begin, t_end;
  const uint16_t* ktiles;  // this sequence's packed key tiles of KV head g, this lane's granule
  int i[CT], r[CT];
  bool row_ok[CT], blk_ok[CT];
  kbf16x8_t qf[CT][8];

  // false: no work (past the last query group, or the chunk lies past the group's keys)
  __device__ __forceinline__ bool init(const KapArgs& a, int chunks) {
    const int u = blockIdx.x / a.hkv;
    g = blockIdx.x % a.hkv;
    const int gi = u / chunks, chunk = u % chunks;
    const int lane = threadIdx.x;
    int seq = 0, base = 0;
    for (; seq < a.num_seqs; ++seq) {
      const int nb = a.cu_qblocks[seq + 1] - a.cu_qblocks[seq];
      const int ng = (nb + CT * BPW - 1) / (CT * BPW);
      if (gi < base + ng) break;
      base += ng;
    }
    if (seq >= a.num_seqs) return false;  // the grid is an upper bound on the unit count
    qb_seq = a.cu_qblocks[seq];
    const int nqb = a.cu_qblocks[seq + 1] - qb_seq;
    const int i0 = (gi - base) * CT * BPW;
    const int tok0 = a.cu_seqlens[seq];
    const int L = a.cu_seqlens[seq + 1] - tok0;
    R = (L + a.stride - 1) / a.stride;  // sampled positions of the sequence
    const int i_last = min(min(i0 + CT * BPW, nqb), a.max_pages) - 1;
    const int c_end = min(R, (i_last + 1) * PER);  // sampled keys any column may see
    const int n_tiles = (c_end + 31) / 32;
    t_begin = chunk * kKapChunkTiles;
    if (t_begin >= n_tiles) return false;
    t_end = min(n_tiles, t_begin + kKapChunkTiles);
    r_min = i0 * PER;  // no column of the unit has a smaller row
    ktiles = a.k_tiles + ((int64_t)g * a.tile_slots + kap_tile_base(qb_seq, PER, seq)) * kKapTileElems + lane * 8;

    n = lane & 31;
    hi = lane >> 5;
    within = n % RB;
    const int hh = within / PER, sr = within % PER;
    const int G = RB / PER;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      i[ct] = i0 + ct * BPW + n / RB;
      r[ct] = i[ct] * PER + sr;  // this column's sampled query position
      blk_ok[ct] = i[ct] < nqb && i[ct] < a.max_pages;  // the column's query block exists
      row_ok[ct] = blk_ok[ct] && r[ct] < R;             // and so does its sampled row
#pragma unroll
      for (int c = 0; c < 8; ++c) qf[ct][c] = kbf16x8_t{};
      if (row_ok[ct]) {
        const uint16_t* qrow = a.q + (int64_t)(tok0 + (int64_t)r[ct] * a.stride) * a.q_st +
                               (int64_t)(g * G + hh) * a.q_sh + hi * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) qf[ct][c] = __builtin_bit_cast(kbf16x8_t, *(const ki32x4_t*)(qrow + c * 16));
      }
    }
    return true;
  }
  // S^T tile kt (keys 32 kt + m of the lane's 16 entries) for the CT column tiles; the
  // packed tile holds each lane's A operands in order, one contiguous KiB per dim chunk
  __device__ __forceinline__ void tile(const KapArgs& a, int kt, kf32x16_t (&acc)[CT]) const {
    kbf16x8_t ka[8];
    const uint16_t* src = ktiles + (int64_t)kt * kKapTileElems;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) ka[cc] = __builtin_bit_cast(kbf16x8_t, *(const ki32x4_t*)(src + cc * 512));
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[ct][e] = 0.f;
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cc], qf[ct][cc], acc[ct], 0, 0, 0);
    }
  }
  // entry e of tile kt is visible to column r iff its key sample c <= r (for a valid
  // column r < R, so the key is a sample of the sequence)
  __device__ __forceinline__ int key_of(int kt, int e) const { return 32 * kt + 8 * (e >> 2) + 4 * hi + (e & 3); }
  __device__ __forceinline__ bool whole(int kt) const { return 32 * kt + 31 <= r_min; }  // wave-uniform
  // index of column ct's row in the row-maxima array [total_qblocks, Hkv, RB]
  __device__ __forceinline__ int64_t row_index(const KapArgs& a, int ct) const {
    return ((int64_t)(qb_seq + i[ct]) * a.hkv + g) * RB + within;
  }
};

// Pass 1: the unit's partial row maxima over the causal sampled keys (raw dot products),
// combined over the units of the query group with an atomic max of the codes.
template <int PER, int RB, int CT>
__global__ __launch_bounds__(64) void kap_rowmax_kernel(const KapArgs a, int chunks) {
  KapUnit<PER, RB, CT> w;
  if (!w.init(a, chunks)) return;
  float M[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) M[ct] = -INFINITY;
  for (int kt = w.t_begin; kt < w.t_end; ++kt) {
    kf32x16_t acc[CT];
    w.tile(a, kt, acc);
    if (w.whole(kt)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) M[ct] = fmaxf(M[ct], acc[ct][e]);
    } else {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (w.key_of(kt, e) <= w.r[ct]) M[ct] = fmaxf(M[ct], acc[ct][e]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const float m = kap_partner_max(M[ct]);
    if (w.row_ok[ct] && w.hi == 0) atomicMax(a.row_max + w.row_index(a, ct), ord_code(m));
  }
}

// Pass 2: block maxima, Pbar = exp(m_rj - M_r), sums over the block's rows, flags.  A
// valid row always has its maximum: its own sample is a key of the unit holding the
// diagonal tile.
template <int PER, int RB, int CT>
__global__ __launch_bounds__(64) void kap_score_kernel(const KapArgs a, int chunks) {
  KapUnit<PER, RB, CT> w;
  if (!w.init(a, chunks)) return;
  const float scale = a.sm_scale;  // > 0
  float M[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    M[ct] = w.row_ok[ct] ? kap_mul_unfused(ord_float(a.row_max[w.row_index(a, ct)]), scale) : -INFINITY;
  for (int kt = w.t_begin; kt < w.t_end; ++kt) {
    kf32x16_t acc[CT];
    w.tile(a, kt, acc);
    const bool full = w.whole(kt);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float* srow = a.score_rows + ((int64_t)(w.qb_seq + w.i[ct]) * a.hkv + w.g) * a.max_pages;
      uint8_t* frow = a.flag_rows + ((int64_t)(w.qb_seq + w.i[ct]) * a.hkv + w.g) * a.max_pages;
      // the lane's key blocks in this tile: PER = 4: block 8 kt + 2 q + hi from entries
      // 4q .. 4q+3; PER = 8: block 4 kt + q from entries 4q .. 4q+3 of both lanes l, l^32
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        float mb = -INFINITY;
        if (full) {
          mb = fmaxf(fmaxf(acc[ct][4 * qq], acc[ct][4 * qq + 1]), fmaxf(acc[ct][4 * qq + 2], acc[ct][4 * qq + 3]));
        } else {
#pragma unroll
          for (int e = 4 * qq; e < 4 * qq + 4; ++e)
            if (w.key_of(kt, e) <= w.r[ct]) mb = fmaxf(mb, acc[ct][e]);
        }
        if (PER == 8) mb = kap_partner_max(mb);
        mb = kap_mul_unfused(mb, scale);  // rounded as M was: Pbar is exactly 1 at the row maximum
        const int j = PER == 4 ? 8 * kt + 2 * qq + w.hi : 4 * kt + qq;
        const bool use = w.row_ok[ct] && (PER == 4 || w.hi == 0) && mb != -INFINITY;
        const float e2 = exp2f((mb - M[ct]) * kKapLog2e);
        float pbar = use ? e2 : 0.f;
        int hrm = (use && mb == M[ct]) ? 1 : 0;
        // sum and OR over the RB columns of the query block: consecutive lanes, an
        // aligned group inside a 16-lane DPP row (RB <= 16) or two such rows (RB = 32)
        pbar = group_sum<RB>(pbar, w.hi);
        hrm = group_or<RB>(hrm, w.hi);
        // the group's last lane writes (its own sampled row may lie past the sequence end)
        if (w.blk_ok[ct] && w.within == RB - 1 && (PER == 4 || w.hi == 0) && j <= w.i[ct]) {
          srow[j] = pbar;
          frow[j] = (uint8_t)hrm;
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void kap_clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = 0u;
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

// One workgroup per (query block, KV head).  Fixed fraction: the K_i-th smallest key
// (keys are distinct: the block id is their low word) is found by a radix select on the
// candidates' keys, and only the K_i kept keys are sorted.  Top-p: every candidate is
// sorted, then the prefix sums of the sorted scores give the count.
// dynamic LDS: keys [cap] uint64, then [cap] 32-bit words (the candidates' high key
// words, or the prefix sums); cap a power of two >= max_pages
__global__ __launch_bounds__(256) void kap_select_kernel(const KapArgs a, int cap) {
  extern __shared__ uint64_t keys[];
  float* csum = reinterpret_cast<float*>(keys + cap);
  uint32_t* hkey = reinterpret_cast<uint32_t*>(keys + cap);
  __shared__ float part[256];
  __shared__ int s_below, s_count;
  __shared__ int hist[1][256];
  __shared__ uint64_t s_prefix[1];
  __shared__ int s_k[1];
  const int qb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  int lo = 0, hi_s = a.num_seqs;
  while (hi_s - lo > 1) {
    const int mid = (lo + hi_s) >> 1;
    if (a.cu_qblocks[mid] <= qb) lo = mid; else hi_s = mid;
  }
  const int i = min(qb - a.cu_qblocks[lo], a.max_pages - 1);
  const int n = i + 1;  // causal candidates
  const int64_t rowoff = ((int64_t)qb * a.hkv + g) * a.max_pages;
  if (tid == 0) {
    s_below = 0;
    s_count = 0;
  }
  int kcount, nsort;
  if (a.mode == 0) {
    kcount = max(1, min(n, (int)ceil((double)a.budget * (double)n - 1e-3)));
    for (int j = tid; j < n; j += 256) hkey[j] = (uint32_t)(kap_key(a.score_rows[rowoff + j], a.flag_rows[rowoff + j], j) >> 32);
    __syncthreads();
    if (kcount < n) radix_select<256>(hkey, cap, 1, n, 0, kcount, hist, s_prefix, s_k, tid);
    // the kept keys, compacted in any order (kcount of them: the keys are distinct)
    for (int j = tid; j < n; j += 256) {
      const uint64_t key = ((uint64_t)hkey[j] << 32) | (uint32_t)j;
      if (kcount == n || key <= s_prefix[0]) keys[atomicAdd(&s_count, 1)] = key;
    }
    nsort = kcount;
  } else {
    for (int j = tid; j < n; j += 256) keys[j] = kap_key(a.score_rows[rowoff + j], a.flag_rows[rowoff + j], j);
    nsort = n;
  }
  int N = 1;
  while (N < nsort) N <<= 1;
  __syncthreads();
  for (int x = nsort + tid; x < N; x += 256) keys[x] = ~0ull;
  __syncthreads();
  bitonic_block<256>(keys, N, tid);
  if (a.mode != 0) {
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

template <int PER, int RB>
static void launch_kap_passes(const KapArgs& a, dim3 grid, int chunks, hipStream_t stream) {
  constexpr int CT = kKapColumnTiles;
  hipLaunchKernelGGL((kap_rowmax_kernel<PER, RB, CT>), grid, dim3(64), 0, stream, a, chunks);
  hipLaunchKernelGGL((kap_score_kernel<PER, RB, CT>), grid, dim3(64), 0, stream, a, chunks);
}

hipError_t launch_build_kap_mask(const KapArgs& a, hipStream_t stream) {
  if (a.total_qblocks == 0) return hipSuccess;
  const int G = a.hq / a.hkv;
  const int per = a.block / a.stride;  // sampled rows and keys per logical block: 4 or 8
  const int rb = G * per;              // a power of two <= 32, checked by the caller
  const int bpw = 32 / rb * kKapColumnTiles;  // query blocks per unit
  // units: (query group, key chunk) x KV head; a group's keys span at most
  // max_pages * per samples
  const int max_tiles = (a.max_pages * per + 31) / 32;
  const int chunks = (max_tiles + kKapChunkTiles - 1) / kKapChunkTiles;
  const int64_t units = (int64_t)(a.total_qblocks / bpw + a.num_seqs) * chunks * a.hkv;
  if (units > 0x7fffffff) return hipErrorInvalidValue;
  if (a.tile_slots > 0)
    hipLaunchKernelGGL(kap_pack_kernel, dim3((unsigned)a.tile_slots, (unsigned)a.hkv), dim3(64), 0, stream, a, per);
  const int64_t n_rows = (int64_t)a.total_qblocks * a.hkv * rb;
  hipLaunchKernelGGL(kap_clear_kernel, dim3((unsigned)std::min<int64_t>((n_rows + 255) / 256, 4096)), dim3(256), 0,
                     stream, a.row_max, n_rows);
  const dim3 grid((unsigned)units);
  switch (rb) {
    case 4: launch_kap_passes<4, 4>(a, grid, chunks, stream); break;
    case 8: per == 4 ? launch_kap_passes<4, 8>(a, grid, chunks, stream) : launch_kap_passes<8, 8>(a, grid, chunks, stream); break;
    case 16: per == 4 ? launch_kap_passes<4, 16>(a, grid, chunks, stream) : launch_kap_passes<8, 16>(a, grid, chunks, stream); break;
    case 32: per == 4 ? launch_kap_passes<4, 32>(a, grid, chunks, stream) : launch_kap_passes<8, 32>(a, grid, chunks, stream); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int cap = 1;
  while (cap < a.max_pages) cap <<= 1;
  hipLaunchKernelGGL(kap_select_kernel, dim3((unsigned)a.total_qblocks, (unsigned)a.hkv), dim3(256),
                     (size_t)cap * (sizeof(uint64_t) + sizeof(float)), stream, a, cap);
  return hipGetLastError();
}

}  // namespace cosa_osk
