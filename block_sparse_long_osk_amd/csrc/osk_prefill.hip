// Ordered-skipping block-sparse prefill attention for gfx950 (MI355X).
//
// Method: CoSA section 4.3 and Appendix C, Algorithm A (attention loop): each
// 64-row query block walks the logical pages of its computation-order mask in
// mask order through the page table, keeps the tiled online softmax of section
// 3.1 Eq. (1)-(2), and skips the value side of a page when Delta > 0 and
// max_r(m_loc[r] - m[r]) < ln(Delta / N) (section 3.3, Eq. (5)), with the
// running max m updated before the test.  Query/key visibility follows the
// PageWeaver notes, section 2.1, Eq. (1): t < L and t <= c.
//
// Organisation on the chip:
// * one workgroup = one (query block, KV head[, head subgroup]) unit, W waves,
//   one wave per q head of the KV head's group: the W heads share every K/V
//   page tile staged in LDS (grouped-query packing) and vote independently;
// * a wave owns its q head's 64 query rows; it computes S^T = K Q^T with
//   v_mfma_f32_32x32x16_bf16 so that each lane holds one query row (lane%32)
//   and half of that row's 64 logits: the row max and row sum need one
//   permlane32 swap, the 64-row skip vote one 32-lane butterfly;
// * O^T = V^T P^T: the probabilities go from the S^T accumulators straight
//   into the B operand (bf16) with no data movement; V^T comes from the
//   row-major V tile through ds_read_b64_tr_b16 (transposing LDS read);
// * K and V page tiles are gathered with global_load_lds_dwordx4 (direct to
//   LDS, no VGPR staging) into a double buffer: the page of visit v+1 is in
//   flight while visit v computes; XOR swizzles keep LDS reads conflict-free;
// * the visit list of a unit (mask row -> validity -> page table -> physical
//   page, first occurrence of a repeated id only) is resolved in LDS windows
//   of 512 entries before the visits, so the hot loop does no dependent
//   global index loads;
// * a one-workgroup schedule kernel orders query blocks by mask length
//   (longest first; stable), and the grid walks that order with the KV head
//   minor, so consecutive workgroups (which the dispatcher spreads over the 8
//   XCDs round-robin) put each KV head's pages on its own XCD's L2.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "osk_internal.h"

namespace cosa_osk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kTileBytes = kPage * kHeadDim * 2;  // one K or V page of one KV head: 16 KiB
constexpr int kWindow = 512;                      // mask entries resolved per window
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kRebase = 8.f;  // log2 headroom of the lazily moved exponent base

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float permlane32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float permlane32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// value of lane (l ^ 32) as seen by lane l
__device__ __forceinline__ uint32_t permlane32_partner(uint32_t x, int lane) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return lane < 32 ? r[1] : r[0];
}
// max over the 32 lanes of each wave half (both halves hold the same rows)
__device__ __forceinline__ float half_wave_max(float x) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// XOR swizzle of the 16-byte granule index inside a 256-byte K row (t = key row):
// the 32 lanes of an MFMA A-operand read hit 16 distinct granules per 16 rows.
__device__ __forceinline__ int swz_k(int t, int granule) { return granule ^ (t & 15); }
// V rows: granule pairs (32-byte chunks) XORed by {0,3,5,6}[t%4] so that the
// four rows each ds_read_b64_tr_b16 lane group touches fall in distinct banks.
__device__ __forceinline__ int swz_v(int t, int granule) { return granule ^ (2 * ((0x6530 >> (4 * (t & 3))) & 0xF)); }

// Gather one page's K and V tile (64 tokens x 128 dims of one KV head) into
// LDS with direct-to-LDS 16-byte loads.  Granule p of the tile lands at LDS
// byte 16*p; it holds token t = p/16 and the (swizzled) source granule.
template <int W>
__device__ __forceinline__ void issue_page_loads(const uint16_t* kpage, const uint16_t* vpage, int64_t kv_st,
                                                 LDS_PTR(uint8_t) kdst, LDS_PTR(uint8_t) vdst, int wave, int lane) {
#pragma unroll
  for (int x = 0; x < 16 / W; ++x) {
    const int m = x * W + wave;
    const int p = m * 64 + lane;
    const int t = p >> 4, gs = p & 15;
    const uint16_t* ks = kpage + t * kv_st + swz_k(t, gs) * 8;
    const uint16_t* vs = vpage + t * kv_st + swz_v(t, gs) * 8;
    __builtin_amdgcn_global_load_lds((const void*)ks, (LDS_PTR(void))(kdst + m * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)vs, (LDS_PTR(void))(vdst + m * 1024), 16, 0, 0);
  }
}

// A operand of O^T = V^T P^T for n-tile nt (32 output dims) and key chunk tc
// (16 keys): lane l holds V[t][n] for n = 32 nt + l%32 and the 8 keys
// t = 16 tc + 8 (kk/4) + 4 (l/32) + kk%4, kk = 0..7 -- the same key order in
// which the lane's S^T accumulator entries feed the B operand.
__device__ __forceinline__ bf16x8_t read_vt(LDS_PTR(const uint8_t) vb, int nt, int tc, int lane) {
  const int hi = lane >> 5, nhalf = (lane >> 4) & 1, e = (lane & 15) >> 2, qq = lane & 3;
  const int n = nt * 32 + nhalf * 16 + qq * 4;
  const int t0 = tc * 16 + hi * 4 + e;
  const int t1 = t0 + 8;
  const int off0 = t0 * 256 + swz_v(t0, n >> 3) * 16 + (n & 7) * 2;
  const int off1 = t1 * 256 + swz_v(t1, n >> 3) * 16 + (n & 7) * 2;
  s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4_t))(vb + off0));
  s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4_t))(vb + off1));
  typedef __attribute__((ext_vector_type(8))) short s16x8_t;
  s16x8_t c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, c);
}

// ---------------------------------------------------------------------------
// schedule: query blocks ordered by mask length, longest first (stable)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void osk_schedule_kernel(const int32_t* __restrict__ mask_len, int n_qb, int hkv,
                                                             int max_len, int32_t* __restrict__ order) {
  __shared__ uint16_t key[kMaxQBlocks];
  __shared__ int hist[kMaxMaskLen + 1];
  __shared__ int partial[1024];
  const int tid = threadIdx.x;
  const int nbins = max_len + 1;
  for (int b = tid; b < nbins; b += 1024) hist[b] = 0;
  __syncthreads();
  for (int qb = tid; qb < n_qb; qb += 1024) {
    int c = 0;
    for (int g = 0; g < hkv; ++g) c = max(c, min(max(mask_len[(int64_t)qb * hkv + g], 0), max_len));
    key[qb] = (uint16_t)(max_len - c);  // ascending key == descending cost
    atomicAdd(&hist[max_len - c], 1);
  }
  __syncthreads();
  // exclusive scan of hist: each thread scans a contiguous segment
  const int seg = (nbins + 1023) / 1024;
  const int b0 = tid * seg, b1 = min(nbins, b0 + seg);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += hist[b];
  partial[tid] = s;
  __syncthreads();
  if (tid < 64) {  // wave 0 scans the 1024 partials
    int run = 0;
    for (int c0 = 0; c0 < 1024; c0 += 64) {
      int x = partial[c0 + tid];
      int incl = x;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(incl, off, 64);
        if (tid >= off) incl += y;
      }
      partial[c0 + tid] = run + incl - x;
      run += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
  int base = partial[tid];
  for (int b = b0; b < b1; ++b) {
    int x = hist[b];
    hist[b] = base;
    base += x;
  }
  __syncthreads();
  if (tid < 64) {  // stable scatter, 64 query blocks at a time, in index order
    const int lane = tid;
    for (int c0 = 0; c0 < n_qb; c0 += 64) {
      const int qb = c0 + lane;
      const bool valid = qb < n_qb;
      const int k = valid ? (int)key[qb] : -1;
      uint64_t todo = __ballot(valid);
      while (todo) {
        const int leader = __builtin_ctzll(todo);
        const int lk = __shfl(k, leader, 64);
        const uint64_t same = __ballot(valid && k == lk);
        const int pos0 = hist[lk];
        if (valid && k == lk) {
          const int rank = __popcll(same & ((1ull << lane) - 1ull));
          order[pos0 + rank] = qb;
        }
        if (lane == leader) hist[lk] = pos0 + __popcll(same);
        todo &= ~same;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// the ordered-skipping prefill kernel
// ---------------------------------------------------------------------------
template <int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(1, 1)))
void osk_prefill_kernel(const PrefillArgs a, int heads_per_group, int nsub) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[4 * kTileBytes];  // K0 K1 V0 V1
  __shared__ int raw_id[kWindow];
  __shared__ int raw_phys[kWindow];
  __shared__ int vis_phys[kWindow];
  __shared__ int vis_j[kWindow];
  __shared__ int vis_k[kWindow];
  __shared__ uint32_t seen_bits[kMaxPagesPerSeq / 32];
  __shared__ int s_count;
  __shared__ uint8_t dec_lds[W][kWindow];
  __shared__ float mar_lds[W][kWindow];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5;
  const int nthreads = 64 * W;

  // ---- which unit: schedule position (block order), KV head (minor), head subgroup
  const int per_qb = a.hkv * nsub;
  const int pos = blockIdx.x / per_qb;
  const int rem = blockIdx.x - pos * per_qb;
  const int g = rem / nsub;
  const int sub = rem - g * nsub;
  const int qb = a.sched[pos];
  const int h = g * heads_per_group + sub * W + wave;
  int lo = 0, hi_s = a.num_seqs;
  while (hi_s - lo > 1) {
    const int mid = (lo + hi_s) >> 1;
    if (a.cu_qblocks[mid] <= qb) lo = mid; else hi_s = mid;
  }
  const int s = lo;
  const int i = qb - a.cu_qblocks[s];
  const int tok0 = a.cu_seqlens[s];
  const int L = a.cu_seqlens[s + 1] - tok0;
  // pages addressable through the page table (cu_seqlens and max_pages_per_seq agree
  // for well-formed inputs; the clamp keeps every table and bitmap access in bounds)
  const int n_pages = min((L + kPage - 1) / kPage, a.max_pages);
  const bool skip_on = a.delta > 0.f;
  const float scale_log2 = a.sm_scale * kLog2e;
  const float tau2 = skip_on ? (float)(log2((double)a.delta) - log2((double)L)) : 0.f;
  const bool logging = a.decisions != nullptr;
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))kv_lds;

  // ---- this wave's 64 query rows as MFMA B operands: lane holds row 32 rt + lane%32,
  //      dims 16 c + 8 hi .. +8
  bf16x8_t qf[2][8];
  bool row_ok[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = rt * 32 + (lane & 31);
    row_ok[rt] = (i * kPage + r) < L;
    const uint16_t* qrow = a.q + (int64_t)(tok0 + i * kPage + r) * a.q_st + (int64_t)h * a.q_sh + hi * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      i32x4_t x = {0, 0, 0, 0};
      if (row_ok[rt]) x = *(const i32x4_t*)(qrow + c * 16);
      qf[rt][c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- online-softmax state (log2 domain, scaled).  m2: the running row max of Eq. (2),
  //      which the skip vote uses.  b2: the exponent base of l2 and O; it follows m2 lazily
  //      (moved only when m2 exceeds it by more than kRebase, so p = 2^(s - b2) <= 2^kRebase)
  //      -- O / l is unchanged by the choice of base, and the rescale of O becomes rare.
  float m2[2] = {-INFINITY, -INFINITY};
  float b2[2] = {-INFINITY, -INFINITY};
  float l2[2] = {0.f, 0.f};
  f32x16_t o[4][2];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nt][rt][e] = 0.f;

  for (int x = threadIdx.x; x < (n_pages + 31) / 32; x += nthreads) seen_bits[x] = 0u;

  const int len = min(max(a.mask_len[(int64_t)qb * a.hkv + g], 0), a.max_mask_len);
  const int32_t* mrow = a.order_mask + ((int64_t)qb * a.hkv + g) * a.max_mask_len;
  const int32_t* pt_row = a.page_table + (int64_t)s * a.max_pages;
  const int64_t kv_head_off = (int64_t)g * a.kv_sh;
  int buf = 0;

  for (int k0 = 0; k0 < len; k0 += kWindow) {
    const int wl = min(kWindow, len - k0);
    // (A) resolve the window's entries in parallel: validity and page table
    for (int e = threadIdx.x; e < wl; e += nthreads) {
      const int id = mrow[k0 + e];
      int ph = -1;
      if (id >= 0 && id < n_pages && id <= i) {
        ph = pt_row[id];
        if (ph < 0 || ph >= a.num_phys) ph = -1;
      }
      raw_id[e] = ph >= 0 ? id : -1;
      raw_phys[e] = ph;
    }
    if (logging)
      for (int x = lane; x < wl; x += 64) { dec_lds[wave][x] = 2; mar_lds[wave][x] = __builtin_nanf(""); }
    __syncthreads();
    // (B) wave 0 compacts the visited entries in mask order; a repeated id keeps
    //     only its first occurrence (bitmap over the sequence's pages)
    if (wave == 0) {
      int count = 0;
      for (int c0 = 0; c0 < wl; c0 += 64) {
        const int e = c0 + lane;
        const int id = e < wl ? raw_id[e] : -1;
        bool keep = id >= 0;
        const uint32_t bit = 1u << (id & 31);
        bool coll = false;
        if (keep && (seen_bits[id >> 5] & bit)) keep = false;
        if (keep) coll = (atomicOr(&seen_bits[id >> 5], bit) & bit) != 0u;
        if (__ballot(coll)) {
          bool dup = false;
          for (int jl = 0; jl < 64; ++jl) {
            const int idj = __shfl(id, jl, 64);
            const int kj = __shfl((int)keep, jl, 64);
            if (jl < lane && kj && idj == id) dup = true;
          }
          keep = keep && !dup;
        }
        const uint64_t km = __ballot(keep);
        if (keep) {
          const int p = count + __popcll(km & ((1ull << lane) - 1ull));
          vis_phys[p] = raw_phys[e];
          vis_j[p] = id;
          vis_k[p] = k0 + e;
        }
        count += __popcll(km);
      }
      if (lane == 0) s_count = count;
    }
    __syncthreads();
    const int nv = s_count;

    if (nv > 0) {
      {
        const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(vis_phys[0]) * a.kv_sp + kv_head_off;
        issue_page_loads<W>(a.k + off, a.v + off, a.kv_st, lds + buf * kTileBytes,
                            lds + (2 + buf) * kTileBytes, wave, lane);
      }
      for (int v = 0; v < nv; ++v) {
        wait_vmem_all();
        __syncthreads();  // page v resident; every wave is done with the other buffer
        const int j = __builtin_amdgcn_readfirstlane(vis_j[v]);
        LDS_PTR(uint8_t) kb = lds + buf * kTileBytes;
        LDS_PTR(uint8_t) vb = lds + (2 + buf) * kTileBytes;
        const int tail_rows = min(kPage, L - j * kPage);  // valid tokens on page j
        if (tail_rows < kPage) {
          // tokens past L on the tail page: zero their V rows (their logits are masked,
          // and a zero probability must not meet a non-finite value)
          for (int x = threadIdx.x; x < (kPage - tail_rows) * 16; x += nthreads)
            *(LDS_PTR(i32x4_t))(vb + tail_rows * 256 + x * 16) = i32x4_t{0, 0, 0, 0};
          __syncthreads();
        }
        if (v + 1 < nv) {
          const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(vis_phys[v + 1]) * a.kv_sp + kv_head_off;
          issue_page_loads<W>(a.k + off, a.v + off, a.kv_st, lds + (buf ^ 1) * kTileBytes,
                              lds + (2 + (buf ^ 1)) * kTileBytes, wave, lane);
        }

        // ---- S^T = K Q^T for 64 keys x 64 query rows (fp32 accumulate)
        f32x16_t acc[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[tt][rt][e] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int t = tt * 32 + (lane & 31);
            const bf16x8_t ka = *(LDS_PTR(const bf16x8_t))(kb + t * 256 + swz_k(t, 2 * c + hi) * 16);
            acc[tt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0][c], acc[tt][0], 0, 0, 0);
            acc[tt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[1][c], acc[tt][1], 0, 0, 0);
          }
        }
        // ---- visibility on the diagonal and tail pages: t <= c and t < L
        if (j == i || tail_rows < kPage) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int t = j * kPage + tt * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
                const int c = i * kPage + rt * 32 + (lane & 31);
                if (t > c || t >= L) acc[tt][rt][e] = -INFINITY;
              }
        }
        // ---- local row max, running-max update, block vote (Eq. (1), (2), (5))
        float mnew2[2], alpha[2];
        float dmax = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          float mx = -INFINITY;
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[tt][rt][e]);
          mx = permlane32_max(mx);
          const float mloc2 = mx * scale_log2;
          mnew2[rt] = fmaxf(m2[rt], mloc2);
          const float dd = (row_ok[rt] && mloc2 != -INFINITY) ? (mloc2 - mnew2[rt]) : -INFINITY;
          dmax = fmaxf(dmax, dd);
        }
        const float margin2 = uniform_f(half_wave_max(dmax));
        const bool skip = skip_on && (margin2 < tau2);
        if (logging && lane == 0) {
          dec_lds[wave][vis_k[v] - k0] = skip ? 1 : 0;
          mar_lds[wave][vis_k[v] - k0] = margin2 * kLn2;
        }
        m2[0] = mnew2[0];
        m2[1] = mnew2[1];
        if (!skip) {
          // ---- move the exponent base if some row's max passed it by more than kRebase
          if (__ballot(m2[0] > b2[0] + kRebase || m2[1] > b2[1] + kRebase)) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
              alpha[rt] = (m2[rt] == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(b2[rt] - m2[rt]);
              b2[rt] = m2[rt];
              l2[rt] *= alpha[rt];
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
              for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[nt][rt][e] *= alpha[rt];
          }
          // ---- P = 2^(S' - b) as bf16 B operands; row sums; O^T += V^T P^T
          bf16x8_t pb[2][4];
          float rs[2] = {0.f, 0.f};
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const float msub = (b2[rt] == -INFINITY) ? 0.f : b2[rt];
#pragma unroll
            for (int tc = 0; tc < 4; ++tc) {
              bf16x8_t pv;
#pragma unroll
              for (int kk = 0; kk < 8; ++kk) {
                const float p = __builtin_amdgcn_exp2f(fmaf(acc[tc >> 1][rt][8 * (tc & 1) + kk], scale_log2, -msub));
                rs[rt] += p;
                pv[kk] = (__bf16)p;
              }
              pb[rt][tc] = pv;
            }
          }
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) l2[rt] += permlane32_sum(rs[rt]);
#pragma unroll
          for (int tc = 0; tc < 4; ++tc) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
              const bf16x8_t va = read_vt(vb, nt, tc, lane);
              o[nt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[0][tc], o[nt][0], 0, 0, 0);
              o[nt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[1][tc], o[nt][1], 0, 0, 0);
            }
          }
        }
        buf ^= 1;
      }
    }
    if (logging) {
      uint8_t* drow = a.decisions + ((int64_t)qb * a.hq + h) * a.max_mask_len + k0;
      float* mrw = a.margins ? a.margins + ((int64_t)qb * a.hq + h) * a.max_mask_len + k0 : nullptr;
      for (int x = lane; x < wl; x += 64) {
        drow[x] = dec_lds[wave][x];
        if (mrw) mrw[x] = mar_lds[wave][x];
      }
    }
    __syncthreads();  // window LDS (visit list, log) is reused by the next window
  }
  if (logging) {
    uint8_t* drow = a.decisions + ((int64_t)qb * a.hq + h) * a.max_mask_len;
    float* mrw = a.margins ? a.margins + ((int64_t)qb * a.hq + h) * a.max_mask_len : nullptr;
    for (int x = len + lane; x < a.max_mask_len; x += 64) {
      drow[x] = 2;
      if (mrw) mrw[x] = __builtin_nanf("");
    }
  }

  // ---- epilogue: O <- O / l (0 when nothing was computed), bf16 out, natural-log LSE
  float inv_l[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) inv_l[rt] = l2[rt] > 0.f ? 1.f / l2[rt] : 0.f;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = rt * 32 + (lane & 31);
    uint16_t* orow = a.out + (int64_t)(tok0 + i * kPage + r) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        // lane (hi=0) holds dims 32nt+16mm+{0..3, 8..11}; its partner (hi=1) {4..7, 12..15}
        const f32x16_t ov = o[nt][rt] * inv_l[rt];
        const uint32_t r0a = pack_bf16x2(ov[8 * mm + 0], ov[8 * mm + 1]);
        const uint32_t r0b = pack_bf16x2(ov[8 * mm + 2], ov[8 * mm + 3]);
        const uint32_t r1a = pack_bf16x2(ov[8 * mm + 4], ov[8 * mm + 5]);
        const uint32_t r1b = pack_bf16x2(ov[8 * mm + 6], ov[8 * mm + 7]);
        const uint32_t sa = hi ? r0a : r1a, sb = hi ? r0b : r1b;
        const uint32_t ra = permlane32_partner(sa, lane), rb = permlane32_partner(sb, lane);
        i32x4_t st;
        if (hi == 0) st = i32x4_t{(int)r0a, (int)r0b, (int)ra, (int)rb};
        else st = i32x4_t{(int)ra, (int)rb, (int)r1a, (int)r1b};
        if (row_ok[rt]) *(i32x4_t*)(orow + nt * 32 + mm * 16 + hi * 8) = st;
      }
    }
    if (a.lse != nullptr && hi == 0 && row_ok[rt]) {
      a.lse[(int64_t)(tok0 + i * kPage + r) * a.hq + h] =
          l2[rt] > 0.f ? (b2[rt] + log2f(l2[rt])) * kLn2 : -INFINITY;
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.total_qblocks == 0) return hipSuccess;
  const int G = a.hq / a.hkv;
  const int W = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int nsub = G / W;
  hipLaunchKernelGGL(osk_schedule_kernel, dim3(1), dim3(1024), 0, stream, a.mask_len, a.total_qblocks, a.hkv,
                     a.max_mask_len, a.sched);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)a.total_qblocks * (unsigned)a.hkv * (unsigned)nsub);
  if (W == 4)
    hipLaunchKernelGGL(osk_prefill_kernel<4>, grid, dim3(256), 0, stream, a, G, nsub);
  else if (W == 2)
    hipLaunchKernelGGL(osk_prefill_kernel<2>, grid, dim3(128), 0, stream, a, G, nsub);
  else
    hipLaunchKernelGGL(osk_prefill_kernel<1>, grid, dim3(64), 0, stream, a, G, nsub);
  return hipGetLastError();
}

}  // namespace cosa_osk
