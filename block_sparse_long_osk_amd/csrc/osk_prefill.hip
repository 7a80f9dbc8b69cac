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
// * one workgroup = one (query block, KV head[, head subgroup]) unit with HW q
//   heads of the KV head's group; two waves per head, each owning 32 of the
//   block's 64 query rows (2*HW waves, two waves per SIMD at HW = 4, so one
//   wave's softmax VALU work runs under another wave's MFMAs).  The two halves
//   of a head combine their partial vote margins through LDS: one vote per
//   (q head, 64-row block);
// * a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so each lane holds
//   one query row (lane%32) and half of that row's 64 logits: row max and row
//   sum need one permlane32 swap, the 32-row partial vote one DPP reduction;
// * O^T = V^T P^T: the probabilities go from the S^T accumulators straight into
//   the B operand (bf16); V^T comes from the row-major V tile through
//   ds_read_b64_tr_b16 (transposing LDS read);
// * K and V page tiles are gathered with global_load_lds_dwordx4 (direct to LDS,
//   no VGPR staging) into a ring of kRing page slots; every wave gathers its
//   share of each page kRing-1 visits ahead.  LDS counters say when a slot's
//   page has landed (ready) and when every wave is done with it (used), so the
//   heads of a group are not held in lock step by a per-visit barrier: a head
//   that skips a page runs ahead of one that computes it;
// * the visit list of a unit (mask row -> validity -> page table -> physical
//   page, first occurrence of a repeated id only) is resolved in LDS windows of
//   512 entries before the visits, so the hot loop does no dependent global loads;
// * a one-workgroup schedule kernel orders query blocks by mask length (longest
//   first; stable), and the grid walks that order with the KV head minor, so
//   consecutive workgroups (which the dispatcher spreads over the 8 XCDs round-
//   robin) keep each KV head's pages in one XCD's L2.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "osk_internal.h"

namespace cosa_osk {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(8))) short s16x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kTileBytes = kPage * kHeadDim * 2;  // one K or V page of one KV head: 16 KiB
constexpr int kPageBytes = 2 * kTileBytes;        // K then V
constexpr int kWindow = 512;                      // mask entries resolved per window
constexpr int kRing = 4;                          // page slots in flight per workgroup
constexpr int kSpinLimit = 1 << 22;               // bound of every inter-wave wait
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
// max over lanes 0..31 (lanes 32..63 hold the same rows), returned wave-uniform
__device__ __forceinline__ float max_lanes32(float x) {
  const int ninf = __float_as_int(-INFINITY);
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x111, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x112, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x114, 0xF, 0xF, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(x), 0x118, 0xF, 0xF, false)));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  return fmaxf(a, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// The page gathers are issued from inline assembly: the compiler does not see
// them as LDS writes, so it does not wait for them before unrelated LDS reads;
// their completion is tracked explicitly with vmcnt (the visit loop issues no
// other vector-memory instruction).
__device__ __forceinline__ void dma_16B(const void* gsrc, uint32_t lds_byte_addr) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "s"(lds_byte_addr)
      : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// wait until at most `pages` pages' worth of this wave's gather instructions are outstanding
template <int PW>
__device__ __forceinline__ void wait_pages_outstanding(int pages) {
  if (pages <= 0) wait_vmcnt<0>();
  else if (pages == 1) wait_vmcnt<PW>();
  else if (pages == 2) wait_vmcnt<2 * PW>();
  else wait_vmcnt<3 * PW>();
}

__device__ __forceinline__ int lds_load_acquire(int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_add_release(int* p, int v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Bounded wait until *ctr >= target.  Every wave of the workgroup is resident,
// and each counter is advanced by waves that never wait on a later visit, so
// the wait ends; the bound turns a broken protocol into an abort, never a hang.
__device__ __forceinline__ bool wait_at_least(int* ctr, int target, int* abort_flag) {
  for (int it = 0; it < kSpinLimit; ++it) {
    if (__builtin_amdgcn_readfirstlane(lds_load_acquire(ctr)) >= target) return true;
    if (__builtin_amdgcn_readfirstlane(lds_load_acquire(abort_flag)) != 0) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(abort_flag, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  return false;
}

// XOR swizzle of the 16-byte granule index inside a 256-byte K row (t = key row):
// the 32 lanes of an MFMA A-operand read hit 16 distinct granules per 16 rows.
__device__ __forceinline__ int swz_k(int t, int granule) { return granule ^ (t & 15); }
// V rows: granule pairs (32-byte chunks) XORed by {0,3,5,6}[t%4] so that the
// four rows each ds_read_b64_tr_b16 lane group touches fall in distinct banks.
__device__ __forceinline__ int swz_v(int t, int granule) { return granule ^ (2 * ((0x6530 >> (4 * (t & 3))) & 0xF)); }

// This wave's share (PW of the page's 32 one-KiB blocks: 16 of K, 16 of V) of
// one page's gather into the ring slot at LDS byte address slot_addr.  Granule
// p of a tile lands at byte 16*p and holds token t = p/16; on the tail page,
// tokens at or past the valid count read row 0 instead (their logits are masked;
// their values then stay finite, so a zero probability never meets a non-finite
// value).
template <int NW, int PW>
__device__ __forceinline__ void gather_page_share(const uint16_t* kpage, const uint16_t* vpage, int64_t kv_st,
                                                  uint32_t slot_addr, int valid_rows, int wave, int lane) {
#pragma unroll
  for (int x = 0; x < PW; ++x) {
    const int m = x * NW + wave;  // block 0..31
    const int blk = m & 15;
    const int p = blk * 64 + lane;
    const int t = p >> 4, gs = p & 15;
    const int ts = t < valid_rows ? t : 0;
    const uint16_t* src = (m < 16) ? kpage + ts * kv_st + swz_k(t, gs) * 8 : vpage + ts * kv_st + swz_v(t, gs) * 8;
    // the LDS base goes to M0 and must be wave-uniform (it is: m depends on the wave only)
    dma_16B(src, __builtin_amdgcn_readfirstlane(slot_addr + (m < 16 ? 0u : (uint32_t)kTileBytes) +
                                                (uint32_t)blk * 1024u));
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
  s16x8_t c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, c);
}

// ---------------------------------------------------------------------------
// schedule: query blocks ordered by mask length, longest first (stable)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void osk_schedule_kernel(const int32_t* __restrict__ mask_len, int n_qb, int hkv,
                                                             int max_len, int32_t* __restrict__ order,
                                                             int32_t* __restrict__ error_count) {
  __shared__ uint16_t key[kMaxQBlocks];
  __shared__ int hist[kMaxMaskLen + 1];
  __shared__ int partial[1024];
  const int tid = threadIdx.x;
  const int nbins = max_len + 1;
  if (tid == 0) *error_count = 0;
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
template <int HW>
__global__ __launch_bounds__(128 * HW) void osk_prefill_kernel(const PrefillArgs a, int heads_per_group, int nsub) {
  constexpr int NW = 2 * HW;   // waves
  constexpr int NT = 64 * NW;  // threads
  constexpr int PW = 32 / NW;  // page-gather instructions per wave per page
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kPageBytes];
  __shared__ int raw_id[kWindow];
  __shared__ int raw_phys[kWindow];
  __shared__ int vis_phys[kWindow];
  __shared__ int vis_j[kWindow];
  __shared__ int vis_k[kWindow];
  __shared__ uint32_t seen_bits[kMaxPagesPerSeq / 32];
  __shared__ uint8_t dec_lds[HW][kWindow];
  __shared__ float mar_lds[HW][kWindow];
  __shared__ int ready_ctr[kRing];
  __shared__ int used_ctr[kRing];
  __shared__ int vote_seq[HW][2][2];
  __shared__ float vote_val[HW][2][2];
  __shared__ int s_count;
  __shared__ int s_abort;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hi = lane >> 5;
  const int half = wave & 1;  // rows 32*half .. +31 of the block; the halves of a head sit on different SIMDs
  const int hl = wave >> 1;   // head within the workgroup

  // ---- which unit: schedule position (block order), KV head (minor), head subgroup
  const int per_qb = a.hkv * nsub;
  const int pos = blockIdx.x / per_qb;
  const int rem = blockIdx.x - pos * per_qb;
  const int g = rem / nsub;
  const int sub = rem - g * nsub;
  const int qb = a.sched[pos];
  const int h = g * heads_per_group + sub * HW + hl;
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
  LDS_PTR(uint8_t) ring_lds = (LDS_PTR(uint8_t))ring;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring_lds;

  // ---- this wave's 32 query rows as MFMA B operands: lane holds row 32*half + lane%32,
  //      dims 16 c + 8 hi .. +8
  const int r_blk = half * 32 + (lane & 31);
  const bool row_ok = (i * kPage + r_blk) < L;
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = a.q + (int64_t)(tok0 + i * kPage + r_blk) * a.q_st + (int64_t)h * a.q_sh + hi * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      i32x4_t x = {0, 0, 0, 0};
      if (row_ok) x = *(const i32x4_t*)(qrow + c * 16);
      qf[c] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- online-softmax state (log2 domain, scaled).  m2: the running row max of Eq. (2),
  //      which the skip vote uses.  b2: the exponent base of l2 and O; it follows m2 lazily
  //      (moved only when m2 exceeds it by more than kRebase, so p = 2^(s - b2) <= 2^kRebase)
  //      -- O / l is unchanged by the choice of base, and the rescale of O becomes rare.
  float m2 = -INFINITY, b2 = -INFINITY, l2 = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[nt][e] = 0.f;

  for (int x = threadIdx.x; x < (n_pages + 31) / 32; x += NT) seen_bits[x] = 0u;
  if (threadIdx.x == 0) s_abort = 0;

  const int len = min(max(a.mask_len[(int64_t)qb * a.hkv + g], 0), a.max_mask_len);
  const int32_t* mrow = a.order_mask + ((int64_t)qb * a.hkv + g) * a.max_mask_len;
  const int32_t* pt_row = a.page_table + (int64_t)s * a.max_pages;
  const uint16_t* kbase = a.k + (int64_t)g * a.kv_sh;
  const uint16_t* vbase = a.v + (int64_t)g * a.kv_sh;

  for (int k0 = 0; k0 < len; k0 += kWindow) {
    const int wl = min(kWindow, len - k0);
    // (A) resolve the window's entries in parallel: validity and page table
    for (int e = threadIdx.x; e < wl; e += NT) {
      const int id = mrow[k0 + e];
      int ph = -1;
      if (id >= 0 && id < n_pages && id <= i) {
        ph = pt_row[id];
        if (ph < 0 || ph >= a.num_phys) ph = -1;
      }
      raw_id[e] = ph >= 0 ? id : -1;
      raw_phys[e] = ph;
    }
    if (logging && half == 0)
      for (int x = lane; x < wl; x += 64) { dec_lds[hl][x] = 2; mar_lds[hl][x] = __builtin_nanf(""); }
    if (threadIdx.x < kRing) { ready_ctr[threadIdx.x] = 0; used_ctr[threadIdx.x] = 0; }
    if (threadIdx.x < 4 * HW) (&vote_seq[0][0][0])[threadIdx.x] = 0;
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

    // ---- ring prologue: gather pages 0 .. kRing-2, announce 0 .. kRing-3
    const int pro = min(kRing - 1, nv);
    for (int p = 0; p < pro; ++p) {
      const int jp = __builtin_amdgcn_readfirstlane(vis_j[p]);
      const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(vis_phys[p]) * a.kv_sp;
      gather_page_share<NW, PW>(kbase + off, vbase + off, a.kv_st, ring_addr + (uint32_t)(p % kRing) * kPageBytes,
                                min(kPage, L - jp * kPage), wave, lane);
    }
    for (int p = 0; p < min(kRing - 2, nv); ++p) {
      wait_pages_outstanding<PW>(pro - 1 - p);
      if (lane == 0) lds_add_release(&ready_ctr[p % kRing], 1);
    }

    for (int v = 0; v < nv; ++v) {
      const int slot = v % kRing;
      // ---- keep kRing-1 pages in flight: gather page v+kRing-1 once every wave is done
      //      with the page that held its slot, then announce page v+kRing-2
      const int u = v + kRing - 1;
      const int issued = min(u, nv - 1);
      if (u < nv) {
        if (!wait_at_least(&used_ctr[u % kRing], NW * (u / kRing), &s_abort)) break;
        const int ju = __builtin_amdgcn_readfirstlane(vis_j[u]);
        const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(vis_phys[u]) * a.kv_sp;
        gather_page_share<NW, PW>(kbase + off, vbase + off, a.kv_st, ring_addr + (uint32_t)(u % kRing) * kPageBytes,
                                  min(kPage, L - ju * kPage), wave, lane);
      }
      const int sgn = v + kRing - 2;
      if (sgn < nv) {
        wait_pages_outstanding<PW>(issued - sgn);
        if (lane == 0) lds_add_release(&ready_ctr[sgn % kRing], 1);
      }
      // ---- page v resident in its slot (every wave's share has landed)
      if (!wait_at_least(&ready_ctr[slot], NW * (v / kRing + 1), &s_abort)) break;
      const int j = __builtin_amdgcn_readfirstlane(vis_j[v]);
      LDS_PTR(const uint8_t) kb = ring_lds + slot * kPageBytes;
      LDS_PTR(const uint8_t) vb = kb + kTileBytes;
      const int tail_rows = min(kPage, L - j * kPage);  // valid tokens on page j

      // ---- S^T = K Q^T for 64 keys x 32 query rows (fp32 accumulate)
      f32x16_t acc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[tt][e] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = tt * 32 + (lane & 31);
          const bf16x8_t ka = *(LDS_PTR(const bf16x8_t))(kb + t * 256 + swz_k(t, 2 * c + hi) * 16);
          acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[c], acc[tt], 0, 0, 0);
        }
      }
      // ---- visibility on the diagonal and tail pages: t <= c and t < L
      if (j == i || tail_rows < kPage) {
        const int c_tok = i * kPage + r_blk;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int t = j * kPage + tt * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
            if (t > c_tok || t >= L) acc[tt][e] = -INFINITY;
          }
      }
      // ---- local row max, running-max update, block vote (Eq. (1), (2), (5))
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[tt][e]);
      mx = permlane32_max(mx);
      const float mloc2 = mx * scale_log2;
      const float mnew2 = fmaxf(m2, mloc2);
      const float dd = (row_ok && mloc2 != -INFINITY) ? (mloc2 - mnew2) : -INFINITY;
      const float my_margin = max_lanes32(dd);
      // exchange the 32-row partial margin with the other half of this head
      const int par = v & 1;
      if (lane == 0) {
        vote_val[hl][half][par] = my_margin;
        __hip_atomic_store(&vote_seq[hl][half][par], v + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (!wait_at_least(&vote_seq[hl][half ^ 1][par], v + 1, &s_abort)) break;
      const float margin2 = fmaxf(my_margin, __int_as_float(__builtin_amdgcn_readfirstlane(
                                                  __float_as_int(vote_val[hl][half ^ 1][par]))));
      const bool skip = skip_on && (margin2 < tau2);
      if (logging && half == 0 && lane == 0) {
        dec_lds[hl][vis_k[v] - k0] = skip ? 1 : 0;
        mar_lds[hl][vis_k[v] - k0] = margin2 * kLn2;
      }
      m2 = mnew2;
      if (!skip) {
        // ---- move the exponent base if some row's max passed it by more than kRebase
        if (__ballot(m2 > b2 + kRebase)) {
          const float alpha = (m2 == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(b2 - m2);
          b2 = m2;
          l2 *= alpha;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[nt][e] *= alpha;
        }
        // ---- P = 2^(S' - b) as bf16 B operands; row sums; O^T += V^T P^T
        const float msub = (b2 == -INFINITY) ? 0.f : b2;
        bf16x8_t pb[4];
        float rs = 0.f;
#pragma unroll
        for (int tc = 0; tc < 4; ++tc) {
          bf16x8_t pv;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const float p = __builtin_amdgcn_exp2f(fmaf(acc[tc >> 1][8 * (tc & 1) + kk], scale_log2, -msub));
            rs += p;
            pv[kk] = (__bf16)p;
          }
          pb[tc] = pv;
        }
        l2 += permlane32_sum(rs);
#pragma unroll
        for (int tc = 0; tc < 4; ++tc) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const bf16x8_t va = read_vt(vb, nt, tc, lane);
            o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[tc], o[nt], 0, 0, 0);
          }
        }
      }
      // every LDS read of this slot has returned (the release waits for the wave's
      // outstanding LDS reads before the count moves)
      if (lane == 0) lds_add_release(&used_ctr[slot], 1);
    }
    wait_vmcnt<0>();  // no page gather may still be writing LDS past this point
    __syncthreads();  // the window's LDS (visit list, ring, log) is reused next
    if (logging && half == 0) {
      uint8_t* drow = a.decisions + ((int64_t)qb * a.hq + h) * a.max_mask_len + k0;
      float* mrw = a.margins ? a.margins + ((int64_t)qb * a.hq + h) * a.max_mask_len + k0 : nullptr;
      for (int x = lane; x < wl; x += 64) {
        drow[x] = dec_lds[hl][x];
        if (mrw) mrw[x] = mar_lds[hl][x];
      }
    }
    if (s_abort != 0) break;
    __syncthreads();
  }
  if (logging && half == 0) {
    uint8_t* drow = a.decisions + ((int64_t)qb * a.hq + h) * a.max_mask_len;
    float* mrw = a.margins ? a.margins + ((int64_t)qb * a.hq + h) * a.max_mask_len : nullptr;
    for (int x = len + lane; x < a.max_mask_len; x += 64) {
      drow[x] = 2;
      if (mrw) mrw[x] = __builtin_nanf("");
    }
  }
  if (threadIdx.x == 0 && s_abort != 0) atomicAdd(a.error_count, 1);

  // ---- epilogue: O <- O / l (0 when nothing was computed), bf16 out, natural-log LSE
  const float inv_l = l2 > 0.f ? 1.f / l2 : 0.f;
  uint16_t* orow = a.out + (int64_t)(tok0 + i * kPage + r_blk) * a.o_st + (int64_t)h * a.o_sh;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const f32x16_t ov = o[nt] * inv_l;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      // lane (hi=0) holds dims 32nt+16mm+{0..3, 8..11}; its partner (hi=1) {4..7, 12..15}
      const uint32_t r0a = pack_bf16x2(ov[8 * mm + 0], ov[8 * mm + 1]);
      const uint32_t r0b = pack_bf16x2(ov[8 * mm + 2], ov[8 * mm + 3]);
      const uint32_t r1a = pack_bf16x2(ov[8 * mm + 4], ov[8 * mm + 5]);
      const uint32_t r1b = pack_bf16x2(ov[8 * mm + 6], ov[8 * mm + 7]);
      const uint32_t sa = hi ? r0a : r1a, sb = hi ? r0b : r1b;
      const uint32_t ra = permlane32_partner(sa, lane), rb = permlane32_partner(sb, lane);
      i32x4_t st;
      if (hi == 0) st = i32x4_t{(int)r0a, (int)r0b, (int)ra, (int)rb};
      else st = i32x4_t{(int)ra, (int)rb, (int)r1a, (int)r1b};
      if (row_ok) *(i32x4_t*)(orow + nt * 32 + mm * 16 + hi * 8) = st;
    }
  }
  if (a.lse != nullptr && hi == 0 && row_ok)
    a.lse[(int64_t)(tok0 + i * kPage + r_blk) * a.hq + h] = l2 > 0.f ? (b2 + log2f(l2)) * kLn2 : -INFINITY;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.total_qblocks == 0) return hipSuccess;
  const int G = a.hq / a.hkv;
  const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int nsub = G / HW;
  hipLaunchKernelGGL(osk_schedule_kernel, dim3(1), dim3(1024), 0, stream, a.mask_len, a.total_qblocks, a.hkv,
                     a.max_mask_len, a.sched, a.error_count);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)a.total_qblocks * (unsigned)a.hkv * (unsigned)nsub);
  if (HW == 4)
    hipLaunchKernelGGL(osk_prefill_kernel<4>, grid, dim3(512), 0, stream, a, G, nsub);
  else if (HW == 2)
    hipLaunchKernelGGL(osk_prefill_kernel<2>, grid, dim3(256), 0, stream, a, G, nsub);
  else
    hipLaunchKernelGGL(osk_prefill_kernel<1>, grid, dim3(128), 0, stream, a, G, nsub);
  return hipGetLastError();
}

}  // namespace cosa_osk
