// Ordered-skipping block-sparse prefill attention for gfx950 (MI355X).
//
// Method: CoSA section 4.3 and Appendix C, Algorithm A (attention loop): each
// query block walks the logical blocks of its computation-order mask in mask order
// through the page table, keeps the tiled online softmax of section 3.1 Eq. (1)-(2),
// and skips the value side of a block when Delta > 0 and max_r(m_loc[r] - m[r]) <
// ln(Delta / N) (section 3.3, Eq. (5)), with the running max m updated before the
// test.  Query/key visibility follows the PageWeaver notes, section 2.1, Eq. (1):
// t < L and t <= c.  Logical blocks hold 64 tokens (osk_prefill_ring_kernel) or 128
// (osk_prefill_b128_kernel; CoSA Appendix D.1: one vote per 128-row query tile), each
// resolved through the physical pages of the KV cache; with a membership mask the
// q heads of a KV group keep their own block sets inside the union row (PageWeaver
// notes, section 2.2).
//
// Organisation on the chip (64-token blocks; the 128-token kernel below differs as
// its own comment says):
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
//   no VGPR staging) into separate rings of kRing tile slots each;
// * the pages are taken two at a time: the key sides of pages 2k and 2k+1 (S^T,
//   row max, partial vote), one workgroup barrier, then their value sides.  The
//   barrier is the only inter-wave synchronisation: it publishes both halves'
//   vote margins, certifies that every wave is done with the K tiles of pages 2k,
//   2k+1 and the V tiles of pages 2k-2, 2k-1 (so those slots can be refilled)
//   and, with each wave's wait for its own gathers before it, that the K tiles of
//   pages 2k+2, 2k+3 and the V tiles of pages 2k, 2k+1 are resident;
// * the visit list of a unit (mask row -> validity -> page table -> physical
//   page, first occurrence of a repeated id only) is resolved in LDS windows of
//   512 entries before the visits, so the hot loop does no dependent global loads;
// * a one-workgroup schedule kernel orders query blocks by mask length (longest
//   first; stable), and the grid walks that order with the KV head minor, so
//   consecutive workgroups (which the dispatcher spreads over the 8 XCDs round-
//   robin) keep each KV head's pages on the same XCDs' L2s (8 / heads_per_phase
//   XCDs per head); the KV heads are taken in phases of as many heads as have
//   their K and V pool slices fit in 192 MiB, so the pages in flight at any time
//   stay within the 256 MB last-level cache.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

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
// mask entries resolved per window: 512, or fewer when a logical block spans several
// physical pages (NPB ids per entry take LDS)
template <int NPB>
constexpr int window_len() { return NPB == 1 ? 512 : NPB <= 4 ? 256 : 128; }
constexpr int kRing = 4;                          // page slots in flight per workgroup
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
// x * y rounded by itself: never fused into a later add or subtract, so that
// m_loc - max(m, m_loc) is exactly 0 for a row whose running max moves to m_loc.
__device__ __forceinline__ float mul_unfused(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// The page gathers are issued from inline assembly: the compiler does not see
// them as LDS writes, so it does not wait for them before unrelated LDS reads;
// their completion is tracked explicitly with vmcnt (the visit loop issues no
// other vector-memory instruction).  One 16-byte granule per lane, from a
// wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane byte offset, to LDS
// byte address lds_byte_addr + 16 * lane.
__device__ __forceinline__ void dma_16B_saddr(const void* sbase, uint32_t voff, uint32_t lds_byte_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_byte_addr)
      : "memory", "m0");
}
// vmcnt holds at most 63; waiting for fewer outstanding instructions is always safe
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N > 63 ? 63 : N) : "memory");
}

// Workgroup barrier for LDS hand-offs: this wave's LDS accesses complete first;
// the page gathers (vmcnt) are left in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}
// XOR swizzle of the 16-byte granule index inside a 256-byte K row (t = key row):
// the 32 lanes of an MFMA A-operand read hit 16 distinct granules per 16 rows.
__device__ __forceinline__ int swz_k(int t, int granule) { return granule ^ (t & 15); }
// V rows: granule pairs (32-byte chunks) XORed by {0,3,5,6}[t%4] so that the
// four rows each ds_read_b64_tr_b16 lane group touches fall in distinct banks.
__device__ __forceinline__ int swz_v(int t, int granule) { return granule ^ (2 * ((0x6530 >> (4 * (t & 3))) & 0xF)); }

// Hides a value from the optimiser (empty asm), e.g. to keep a cheap per-lane term
// from being hoisted out of a loop into a long-lived register.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

// Gather of K and V page tiles into LDS.  A tile is 16 one-KiB blocks; with NW
// waves, wave w issues blocks b = x*NW + w (x < 16/NW), and lane l of block b
// fills row 4b + l/16, granule l%16 (the granule order of the swizzles above).
// The swizzle terms depend on the row only through its low 4 (K) or 2 (V) bits,
// so a per-lane byte offset (row within the block + swizzled granule) serves
// every block of the wave -- two for K when NW = 2, where odd blocks are 8 rows
// off -- and the block's row base goes into the scalar address.  On a tail page
// (fewer than 64 valid tokens) rows at or past the valid count read row 0: their
// logits are masked and their values stay finite, so a zero probability never
// meets a non-finite value.
template <int NW>
struct TileGather {
  static constexpr int kBlocks = 16 / NW;  // blocks per wave per tile
  uint32_t lane_k[2], lane_v;
  int kv_st;  // token stride in elements (the host bounds it so offsets fit in 32 bits)

  __device__ __forceinline__ void init(int64_t kv_stride_tok, int wave, int lane) {
    kv_st = (int)kv_stride_tok;
    const int trow = lane >> 4;
#pragma unroll
    for (int x = 0; x < 2; ++x)
      lane_k[x] = (uint32_t)(trow * kv_st + swz_k(4 * (x * NW + wave) + trow, lane & 15) * 8) * 2u;
    lane_v = (uint32_t)(trow * kv_st + swz_v(trow, lane & 15) * 8) * 2u;
  }
  // This wave's share of one tile (valid_rows rows hold data) into the slot at LDS byte
  // address slot.  sub_base[s] is the tile's base in physical page s of the logical
  // block (page_len tokens each, SUB = 64 / page_len pages); the 4 rows of a 1-KiB
  // block always lie in one physical page.
  template <int SUB>
  __device__ __forceinline__ void issue(const uint16_t* const (&sub_base)[SUB], int page_len, uint32_t slot,
                                        int valid_rows, bool is_v, int wave, int lane) const {
    if (valid_rows >= kPage) {
#pragma unroll
      for (int x = 0; x < kBlocks; ++x) {
        const int b = x * NW + wave;
        const int row = 4 * b;
        const uint16_t* base = SUB == 1 ? sub_base[0] + row * kv_st
                                        : sub_base[row / page_len] + (row % page_len) * kv_st;
        dma_16B_saddr(base, is_v ? lane_v : lane_k[x & 1], slot + (uint32_t)b * 1024u);
      }
    } else {
      // Tail block: rows at or past the valid count read a valid row instead -- the
      // block's own first row when the block straddles the end, row 0 of the logical
      // block when it lies wholly past it -- so their (masked) values stay finite.  Rare:
      // the lane terms are recomputed here rather than kept in registers.
      const int ln = (int)opaque((uint32_t)lane);
#pragma unroll
      for (int x = 0; x < kBlocks; ++x) {
        const int b = x * NW + wave;
        const int row = 4 * b;
        const bool past = row >= valid_rows;
        const uint16_t* base = past ? sub_base[0]
                                    : (SUB == 1 ? sub_base[0] + row * kv_st
                                                : sub_base[row / page_len] + (row % page_len) * kv_st);
        const int t = row + (ln >> 4);
        const int ts = (past || t >= valid_rows) ? 0 : t - row;  // row within the addressed group
        const uint32_t voff = (uint32_t)(ts * kv_st + (is_v ? swz_v(t, ln & 15) : swz_k(t, ln & 15)) * 8) * 2u;
        dma_16B_saddr(base, voff, slot + (uint32_t)b * 1024u);
      }
    }
  }
};


// LDS operand addressing.  The swizzles above only touch address bits 4..7, so an
// operand address is a per-lane base XOR a per-chunk constant, plus an immediate
// offset.  The per-lane base of a tile is formed once per tile and hidden from the
// optimiser (empty asm), so that the chunk addresses are not hoisted out of the
// visit loop into a dozen loop-invariant registers.
template <class T>
__device__ __forceinline__ LDS_PTR(const T) lds_at(uint32_t byte_addr) {
  return (LDS_PTR(const T))(uintptr_t)byte_addr;
}
// K tile: A operand of S^T = K Q^T for key tile tt (32 keys) and dim chunk c
// (16 dims): lane l reads key t = 32 tt + l%32, dims 16 c + 8 (l/32) .. +8, at
// t*256 + swz_k(t, 2c + l/32)*16 = (base ^ (c << 5)) + 8192 tt.
__device__ __forceinline__ uint32_t k_lane_base(uint32_t kb, int lane) {
  return opaque(kb + (uint32_t)((lane & 31) * 256 + (((lane >> 5) ^ (lane & 15)) << 4)));
}
// V tile: A operand of O^T = V^T P^T for n-tile nt (32 output dims) and key chunk
// tc (16 keys): lane l holds V[t][n] for n = 32 nt + l%32 and the 8 keys
// t = 16 tc + 8 (kk/4) + 4 (l/32) + kk%4, kk = 0..7 -- the same key order in which
// the lane's S^T accumulator entries feed the B operand.  Two ds_read_b64_tr_b16
// (keys kk < 4 and kk >= 4, 8 rows apart) at (base ^ (nt << 6)) + 4096 tc (+2048).
__device__ __forceinline__ uint32_t v_lane_base(uint32_t vb, int lane) {
  const int hi = lane >> 5, nhalf = (lane >> 4) & 1, e = (lane & 15) >> 2, qq = lane & 3;
  const int sw = 2 * ((0x6530 >> (4 * e)) & 0xF);  // swz_v's row term for rows t = e mod 4
  return opaque(vb + (uint32_t)((hi * 4 + e) * 256 + (((2 * nhalf + (qq >> 1)) ^ sw) << 4) + (qq & 1) * 8));
}
__device__ __forceinline__ bf16x8_t read_vt(uint32_t vbase_lane, int nt, int tc) {
  const uint32_t a0 = (vbase_lane ^ (uint32_t)(nt << 6)) + (uint32_t)tc * 4096u;
  s16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4_t))lds_at<s16x4_t>(a0));
  s16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4_t))lds_at<s16x4_t>(a0 + 2048u));
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
  {  // stable scatter: wave w fills the bins [w * per, (w + 1) * per) and walks every
     // query block in index order, 64 at a time, so each bin is filled in index order
    const int lane = tid & 63, wv = tid >> 6;
    const int per = (nbins + 15) / 16;
    const int lo = wv * per, hi = min(nbins, lo + per);
    for (int c0 = 0; c0 < n_qb; c0 += 64) {
      const int qb = c0 + lane;
      const int k = qb < n_qb ? (int)key[qb] : -1;
      const bool mine = k >= lo && k < hi;
      uint64_t todo = __ballot(mine);
      while (todo) {
        const int leader = __builtin_ctzll(todo);
        const int lk = __shfl(k, leader, 64);
        const uint64_t same = __ballot(mine && k == lk);
        const int pos0 = hist[lk];
        if (mine && k == lk) {
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
// pieces shared by the two prefill kernels
// ---------------------------------------------------------------------------
// One workgroup's unit: a query block (by schedule position), a KV head, and the
// HW q heads hl = 0..HW-1 of subgroup `sub` of that KV head's group.
struct Unit {
  int qb, g, h, i, tok0, L, n_pages, len;
  const int32_t* pt_row;
};

template <int HW, int B>
__device__ __forceinline__ Unit decode_unit(const PrefillArgs& a, int heads_per_group, int nsub, int hl) {
  Unit u;
  // The grid takes the KV heads in phases of heads_per_phase: every query block (in the
  // longest-first order) for the first heads, then for the next ones.  Within a phase the
  // KV head is minor, so consecutive workgroups, which the dispatcher deals out to the 8
  // XCDs in turn, keep each KV head on the same XCDs.
  const int hp = a.heads_per_phase;
  const int per_phase = a.total_qblocks * hp * nsub;
  const int phase = blockIdx.x / per_phase;
  const int idx = blockIdx.x - phase * per_phase;
  const int per_qb = hp * nsub;
  const int pos = idx / per_qb;
  const int rem = idx - pos * per_qb;
  u.g = phase * hp + rem / nsub;
  const int sub = rem - (rem / nsub) * nsub;
  COSA_CHECK(a, pos >= 0 && pos < a.total_qblocks && u.g < a.hkv);
  u.qb = a.sched[pos];
  COSA_CHECK(a, u.qb >= 0 && u.qb < a.total_qblocks);
  u.h = u.g * heads_per_group + sub * HW + hl;
  COSA_CHECK(a, u.h < a.hq);
  int lo = 0, hi_s = a.num_seqs;
  while (hi_s - lo > 1) {
    const int mid = (lo + hi_s) >> 1;
    if (a.cu_qblocks[mid] <= u.qb) lo = mid; else hi_s = mid;
  }
  u.i = u.qb - a.cu_qblocks[lo];
  u.tok0 = a.cu_seqlens[lo];
  u.L = a.cu_seqlens[lo + 1] - u.tok0;
  // pages addressable through the page table (cu_seqlens and max_pages_per_seq agree
  // for well-formed inputs; the clamp keeps every table and bitmap access in bounds)
  u.n_pages = min((u.L + B - 1) / B, a.max_pages);
  u.len = min(max(a.mask_len[(int64_t)u.qb * a.hkv + u.g], 0), a.max_mask_len);
  u.pt_row = a.page_table + (int64_t)lo * a.pt_stride;
  return u;
}

// The wave's 32 query rows as MFMA B operands: lane holds row r_blk of the B-token
// query block, dims 16 c + 8 hi .. +8 (zero for rows past the sequence end).
template <int B>
__device__ __forceinline__ void load_q(const PrefillArgs& a, const Unit& u, int r_blk, bool row_ok, int hi,
                                       bf16x8_t (&qf)[8]) {
  const uint16_t* qrow = a.q + (int64_t)(u.tok0 + u.i * B + r_blk) * a.q_st + (int64_t)u.h * a.q_sh + hi * 8;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    i32x4_t x = {0, 0, 0, 0};
    if (row_ok) x = *(const i32x4_t*)(qrow + c * 16);
    qf[c] = __builtin_bit_cast(bf16x8_t, x);
  }
}
// Q must have landed before the visit loop: otherwise the compiler places its vmcnt
// wait inside the loop, where it would also drain the in-flight page gathers.  Called
// after the window's visit list is resolved, so that Q's loads overlap the mask-row
// and page-table loads.
__device__ __forceinline__ void wait_q_landed() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt unconstrained
}

// Visit list of one window of the mask row, in LDS (NPB physical page ids per block).
// raw_id and vis_j hold the block id in bits 0..15 and, in bits 16 + hl, whether the
// entry belongs to the workgroup's head hl (all set without a membership mask).
template <int NPB>
struct WindowLds {
  static constexpr int kWin = window_len<NPB>();
  int raw_id[kWin];
  int raw_phys[kWin * NPB];  // physical pages of each entry's logical block
  int vis_phys[kWin * NPB];
  int vis_j[kWin];
  int vis_k[kWin];
  uint32_t seen_bits[kMaxPagesPerSeq / 32];
  int count;
};

// Resolve mask entries k0 .. k0+wl-1 into the window's visit list: an entry is
// visited when its id is a causal logical block of the sequence (0 <= id <= i, id
// below the block count) whose physical pages are valid, only at its first
// occurrence in the row (bitmap over the sequence's blocks, kept across windows),
// and only if it belongs to one of the workgroup's HW heads h_first .. h_first+HW-1
// (membership mask; a repeated id is not visited by any head).
// B: tokens per logical block; NPB = B / page_len physical pages per block.
// Returns the number of visits.  Called by every thread of the workgroup; ends with
// a barrier.
template <int NT, int NPB, int B, int HW>
__device__ __forceinline__ int resolve_window(const PrefillArgs& a, const Unit& u, const int32_t* mrow, int k0,
                                              int wl, WindowLds<NPB>& w, int wave, int lane, int h_first) {
  for (int e = threadIdx.x; e < wl; e += NT) {
    COSA_CHECK(a, k0 + e < a.max_mask_len);
    const int id = mrow[k0 + e];
    int mbits = (1 << HW) - 1;
    if (a.membership != nullptr) {
      mbits = 0;
      const uint8_t* mem = a.membership + ((int64_t)u.qb * a.hq + h_first) * a.max_mask_len + k0 + e;
#pragma unroll
      for (int x = 0; x < HW; ++x) mbits |= mem[(int64_t)x * a.max_mask_len] != 0 ? (1 << x) : 0;
    }
    int ph[NPB];
    bool ok = false;
    if (id >= 0 && id < u.n_pages && id <= u.i) {
      if (NPB == 1) {
        COSA_CHECK(a, id < a.pt_stride);
        ph[0] = u.pt_row[id];
        ok = ph[0] >= 0 && ph[0] < a.num_phys;
      } else {
        ok = block_phys(u.pt_row, a.pt_stride, id, u.L, a.page_len, B, a.num_phys, ph);
      }
    }
    w.raw_id[e] = ok ? (id | (mbits << 16)) : -1;
#pragma unroll
    for (int x = 0; x < NPB; ++x) w.raw_phys[e * NPB + x] = ok ? ph[x] : -1;
  }
  __syncthreads();
  // wave 0 compacts the visited entries in mask order
  if (wave == 0) {
    int count = 0;
    for (int c0 = 0; c0 < wl; c0 += 64) {
      const int e = c0 + lane;
      const int raw = e < wl ? w.raw_id[e] : -1;
      const int id = raw >= 0 ? (raw & 0xFFFF) : -1;
      bool keep = id >= 0;
      const uint32_t bit = 1u << (id & 31);
      bool coll = false;
      if (keep && (w.seen_bits[id >> 5] & bit)) keep = false;
      if (keep) coll = (atomicOr(&w.seen_bits[id >> 5], bit) & bit) != 0u;
      if (__ballot(coll)) {
        // a repeated id inside these 64 entries: the lowest entry keeps it
        bool dup = false;
        for (int jl = 0; jl < 64; ++jl) {
          const int idj = __shfl(id, jl, 64);
          const int kj = __shfl((int)keep, jl, 64);
          if (jl < lane && kj && idj == id) dup = true;
        }
        keep = keep && !dup;
      }
      // first occurrences are marked seen whether or not one of this workgroup's heads
      // takes them; the workgroup visits those that belong to one of its heads
      const bool visit = keep && (raw >> 16) != 0;
      const uint64_t km = __ballot(visit);
      if (visit) {
        const int p = count + __popcll(km & ((1ull << lane) - 1ull));
#pragma unroll
        for (int x = 0; x < NPB; ++x) w.vis_phys[p * NPB + x] = w.raw_phys[e * NPB + x];
        w.vis_j[p] = raw;
        w.vis_k[p] = k0 + e;
      }
      count += __popcll(km);
    }
    if (lane == 0) w.count = count;
  }
  __syncthreads();
  return w.count;
}

// S^T = K Q^T for the 64 keys of the K tile at kb and the wave's 32 query rows.
// All 16 K operands are requested ahead of the MFMAs, so LDS latency is paid
// once per tile rather than once per MFMA.
__device__ __forceinline__ void qk_tile(uint32_t kb, const bf16x8_t (&qf)[8], int lane,
                                        f32x16_t (&acc)[2]) {
  const uint32_t kl = k_lane_base(kb, lane);
  bf16x8_t ka[8][2];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) ka[c][tt] = *lds_at<bf16x8_t>((kl ^ (uint32_t)(c << 5)) + (uint32_t)tt * 8192u);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[tt][e] = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c][tt], qf[c], acc[tt], 0, 0, 0);
  // keep the scheduler from sinking each read next to its MFMA: 8 reads ahead
#pragma unroll
  for (int x = 0; x < 8; ++x) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int x = 0; x < 8; ++x) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// Visibility t <= c and t < L for the 64-key tile whose first key is token key0 of the
// sequence, the lane's query row being token c_tok; `need` (wave-uniform) is false
// when the tile is known to be wholly visible.
__device__ __forceinline__ void mask_tile_at(f32x16_t (&acc)[2], int key0, int c_tok, int L, int hi, bool need) {
  if (need) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = key0 + tt * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
        if (t > c_tok || t >= L) acc[tt][e] = -INFINITY;
      }
  }
}
// 64-token blocks: masking is needed on the diagonal block and on the tail block.
__device__ __forceinline__ void mask_tile(f32x16_t (&acc)[2], int j, int i, int r_blk, int L, int hi) {
  mask_tile_at(acc, j * kPage, i * kPage + r_blk, L, hi, j == i || L - j * kPage < kPage);
}
// The page's local row max in the scaled log2 domain; lanes l and l^32 hold the
// same row.
__device__ __forceinline__ float rowmax2(const f32x16_t (&acc)[2], float scale_log2) {
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[tt][e]);
  return mul_unfused(permlane32_max(mx), scale_log2);
}
__device__ __forceinline__ float mask_rowmax2(f32x16_t (&acc)[2], int j, int i, int r_blk, int L, int hi,
                                              float scale_log2) {
  mask_tile(acc, j, i, r_blk, L, hi);
  return rowmax2(acc, scale_log2);
}

// P = 2^(S' - b) as bf16 B operands (lane's 32 logits of its row, key order of
// the S^T accumulator), returning the lane's partial row sum.
__device__ __forceinline__ float probs_tile(const f32x16_t (&acc)[2], float scale_log2, float b2,
                                            bf16x8_t (&pb)[4]) {
  const float msub = (b2 == -INFINITY) ? 0.f : b2;
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
  return rs;
}

// The 16 V^T A operands of the V tile at vb.
__device__ __forceinline__ void load_vt_tile(uint32_t vb, int lane, bf16x8_t (&va)[4][4]) {
  const uint32_t vl = v_lane_base(vb, lane);
#pragma unroll
  for (int tc = 0; tc < 4; ++tc)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) va[tc][nt] = read_vt(vl, nt, tc);
}
// O^T += V^T P^T from operands in registers.
__device__ __forceinline__ void pv_mfma(const bf16x8_t (&va)[4][4], const bf16x8_t (&pb)[4], f32x16_t (&o)[4]) {
#pragma unroll
  for (int tc = 0; tc < 4; ++tc)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[tc][nt], pb[tc], o[nt], 0, 0, 0);
}
// O^T += V^T P^T for the V tile at vb.
__device__ __forceinline__ void pv_tile(uint32_t vb, const bf16x8_t (&pb)[4], int lane,
                                        f32x16_t (&o)[4]) {
  bf16x8_t va[4][4];
  load_vt_tile(vb, lane, va);
  pv_mfma(va, pb, o);
}

// Move the exponent base when some row's running max passed it by more than
// kRebase (O / l does not depend on the base), rescaling l and O.
__device__ __forceinline__ void maybe_rebase(float m2, float& b2, float& l2, f32x16_t (&o)[4]) {
  if (__ballot(m2 > b2 + kRebase)) {
    const float alpha = (m2 == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(b2 - m2);
    b2 = m2;
    l2 *= alpha;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[nt][e] *= alpha;
  }
}

// Decision and margin log of one head for mask entries k0 .. k0+wl-1.
__device__ __forceinline__ void flush_log(const PrefillArgs& a, const Unit& u, int k0, int wl, const uint8_t* dec,
                                          const float* mar, int lane) {
  COSA_CHECK(a, k0 >= 0 && k0 + wl <= a.max_mask_len);
  uint8_t* drow = a.decisions + ((int64_t)u.qb * a.hq + u.h) * a.max_mask_len + k0;
  float* mrw = a.margins ? a.margins + ((int64_t)u.qb * a.hq + u.h) * a.max_mask_len + k0 : nullptr;
  for (int x = lane; x < wl; x += 64) {
    drow[x] = dec[x];
    if (mrw) mrw[x] = mar[x];
  }
}
// Entries past the mask length: code 2 (not visited), margin NaN.
__device__ __forceinline__ void fill_log_tail(const PrefillArgs& a, const Unit& u, int lane) {
  uint8_t* drow = a.decisions + ((int64_t)u.qb * a.hq + u.h) * a.max_mask_len;
  float* mrw = a.margins ? a.margins + ((int64_t)u.qb * a.hq + u.h) * a.max_mask_len : nullptr;
  for (int x = u.len + lane; x < a.max_mask_len; x += 64) {
    drow[x] = 2;
    if (mrw) mrw[x] = __builtin_nanf("");
  }
}

// O <- O / l (0 when nothing was computed), bf16 out, natural-log LSE; row r_blk of a
// B-token query block.
template <int B>
__device__ __forceinline__ void store_output(const PrefillArgs& a, const Unit& u, const f32x16_t (&o)[4], float l2,
                                             float b2, int r_blk, bool row_ok, int lane) {
  const int hi = lane >> 5;
  const float inv_l = l2 > 0.f ? 1.f / l2 : 0.f;
  COSA_CHECK(a, !row_ok || u.tok0 + u.i * B + r_blk < a.cu_seqlens[a.num_seqs]);
  uint16_t* orow = a.out + (int64_t)(u.tok0 + u.i * B + r_blk) * a.o_st + (int64_t)u.h * a.o_sh;
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
    a.lse[(int64_t)(u.tok0 + u.i * B + r_blk) * a.hq + u.h] = l2 > 0.f ? (b2 + log2f(l2)) * kLn2 : -INFINITY;
}

__device__ __forceinline__ float skip_threshold2(const PrefillArgs& a, int L) {
  return a.delta > 0.f ? (float)(log2((double)a.delta) - log2((double)L)) : 0.f;
}

// ---------------------------------------------------------------------------
// ring kernel: HW = 4, 2 or 1 q heads of one KV head's group per workgroup
// ---------------------------------------------------------------------------
// Two waves per head (32 rows each).  K tiles and V tiles have rings of kRing slots
// each; tiles are gathered by waves 0 .. GW-1 (with eight waves, one per SIMD: a
// page's gather instructions queue at the CU's load path for hundreds of cycles,
// and meanwhile the other wave of each SIMD runs its value side alone, which
// staggers the two).
// Step k (pages 2k, 2k+1): S^T of both pages and their 32-row partial vote margins
// (written to LDS); this wave's wait for all its outstanding gathers; a workgroup
// barrier; then the gathers of the K tiles of pages 2k+4, 2k+5 (into the K slots
// of pages 2k, 2k+1) and the V tiles of pages 2k+2, 2k+3 (into the V slots of
// pages 2k-2, 2k-1), and for each page in order the block vote from both halves'
// margins and its value side unless it is skipped.  Every page's arithmetic is
// exactly that of visiting the pages one at a time.  Every wave runs the same
// number of barriers (the visit count is workgroup-uniform), so no wait can hang.
// MEMB: a membership mask restricts each head to its own entries (otherwise every head
// takes every visit and the membership tests fold away).
template <int HW, int SUB, bool MEMB>
__global__ __launch_bounds__(128 * HW) void osk_prefill_ring_kernel(const PrefillArgs a, int heads_per_group,
                                                                    int nsub) {
  constexpr int NW = 2 * HW;   // waves
  constexpr int NT = 64 * NW;  // threads
  constexpr int GW = NW >= 4 ? NW / 2 : NW;  // waves that gather pages (waves 0 .. GW-1)
  constexpr int kWindow = window_len<SUB>();  // SUB: physical pages per logical block
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kPageBytes];
  __shared__ WindowLds<SUB> wlds;
  __shared__ uint8_t dec_lds[HW][kWindow];
  __shared__ float mar_lds[HW][kWindow];
  __shared__ float vote_val[HW][2][2][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int half = wave & 1;  // rows 32*half .. +31 of the block; the halves of a head sit on different SIMDs
  const int hl = wave >> 1;   // head within the workgroup
  const Unit u = decode_unit<HW, kPage>(a, heads_per_group, nsub, hl);
  const bool skip_on = a.delta > 0.f;
  const float scale_log2 = a.sm_scale * kLog2e;
  const float tau2 = skip_threshold2(a, u.L);
  const bool logging = a.decisions != nullptr;
  LDS_PTR(uint8_t) ring_lds = (LDS_PTR(uint8_t))ring;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring_lds;

  const int r_blk = half * 32 + (lane & 31);
  const bool row_ok = (u.i * kPage + r_blk) < u.L;
  bf16x8_t qf[8];
  load_q<kPage>(a, u, r_blk, row_ok, lane >> 5, qf);

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

  for (int x = threadIdx.x; x < (u.n_pages + 31) / 32; x += NT) wlds.seen_bits[x] = 0u;

  const int32_t* mrow = a.order_mask + ((int64_t)u.qb * a.hkv + u.g) * a.max_mask_len;
  const uint16_t* kbase = a.k + (int64_t)u.g * a.kv_sh;
  const uint16_t* vbase = a.v + (int64_t)u.g * a.kv_sh;
  const bool gatherer = wave < GW;
  TileGather<GW> tg;
  tg.init(a.kv_st, gatherer ? wave : 0, lane);

  for (int k0 = 0; k0 < u.len; k0 += kWindow) {
    const int wl = min(kWindow, u.len - k0);
    if (logging && half == 0)
      for (int x = lane; x < wl; x += 64) { dec_lds[hl][x] = 2; mar_lds[hl][x] = __builtin_nanf(""); }
    const int nv = resolve_window<NT, SUB, kPage, HW>(a, u, mrow, k0, wl, wlds, wave, lane, u.h - hl);
    COSA_CHECK(a, nv >= 0 && nv <= wl);
    wait_q_landed();
    // K tiles live in slots 0..3 of the first half of the ring, V tiles in the second
    // half; page p uses K slot p % 4 and V slot p % 4.
    auto k_slot = [&](int p) { return ring_addr + (uint32_t)(p % kRing) * kTileBytes; };
    auto v_slot = [&](int p) { return ring_addr + (uint32_t)(kRing * kTileBytes) + (uint32_t)(p % kRing) * kTileBytes; };
    // this wave's share of page p's K (is_v false) or V tile
    auto gather_tile = [&](int p, bool is_v) {
      if (!gatherer || p >= nv) return;
      const int jp = __builtin_amdgcn_readfirstlane(wlds.vis_j[p]) & 0xFFFF;
      const uint16_t* sub_base[SUB];
#pragma unroll
      for (int x = 0; x < SUB; ++x) {
        const int ph = __builtin_amdgcn_readfirstlane(wlds.vis_phys[p * SUB + x]);
        COSA_CHECK(a, ph >= 0 && ph < a.num_phys);
        sub_base[x] = (is_v ? vbase : kbase) + (int64_t)ph * a.kv_sp;
      }
      tg.template issue<SUB>(sub_base, a.page_len, is_v ? v_slot(p) : k_slot(p), u.L - jp * kPage, is_v, wave,
                             lane);
    };

    // ---- prologue: K of pages 0, 1 resident before the first QK; then V of pages 0, 1
    //      and K of pages 2, 3 in flight (they land before the first step's barrier)
    gather_tile(0, false);
    gather_tile(1, false);
    if (nv > 0) {
      wait_vmcnt<0>();
      lds_barrier();
    }
    gather_tile(0, true);
    gather_tile(1, true);
    gather_tile(2, false);
    gather_tile(3, false);

    // Step k: the key sides of pages 2k and 2k+1, one barrier, their value sides.
    const bool vote = skip_on || logging;
    for (int v = 0; v < nv; v += 2) {
      const bool has_b = v + 1 < nv;
      const int par = (v >> 1) & 1;
      // ---- key sides (Eq. (1), (2), (5)): S^T, running max, partial margins.  A head
      //      takes no part in a visit outside its membership: no logits, no vote.
      const int va = __builtin_amdgcn_readfirstlane(wlds.vis_j[v]);
      const bool mine_a = !MEMB || ((va >> (16 + hl)) & 1);
      f32x16_t acc_a[2], acc_b[2];
      float mloc_a = -INFINITY;
      if (mine_a) {
        qk_tile(k_slot(v), qf, lane, acc_a);
        mloc_a = mask_rowmax2(acc_a, va & 0xFFFF, u.i, r_blk, u.L, lane >> 5, scale_log2);
      }
      const float mnew_a = fmaxf(m2, mloc_a);
      const float dd_a = (row_ok && mloc_a != -INFINITY) ? (mloc_a - mnew_a) : -INFINITY;
      const float marg_a = max_lanes32(dd_a);
      float mnew_b = mnew_a, marg_b = -INFINITY;
      bool mine_b = false;
      if (has_b) {
        const int vb = __builtin_amdgcn_readfirstlane(wlds.vis_j[v + 1]);
        mine_b = !MEMB || ((vb >> (16 + hl)) & 1);
        float mloc_b = -INFINITY;
        if (mine_b) {
          qk_tile(k_slot(v + 1), qf, lane, acc_b);
          mloc_b = mask_rowmax2(acc_b, vb & 0xFFFF, u.i, r_blk, u.L, lane >> 5, scale_log2);
        }
        mnew_b = fmaxf(mnew_a, mloc_b);
        const float dd_b = (row_ok && mloc_b != -INFINITY) ? (mloc_b - mnew_b) : -INFINITY;
        marg_b = max_lanes32(dd_b);
      }
      if (vote && lane == 0) {
        vote_val[hl][half][par][0] = marg_a;
        vote_val[hl][half][par][1] = marg_b;
      }
      // every gather issued since the last barrier (K of pages 2k+2, 2k+3; V of pages
      // 2k, 2k+1) has landed for this wave
      wait_vmcnt<0>();
      // one barrier per two pages: past it, the K tiles of pages 2k, 2k+1 and the V tiles
      // of pages 2k-2, 2k-1 are free, the next pages' K and these pages' V are resident,
      // and both halves' margins are visible
      lds_barrier();
      const float pa = vote ? vote_val[hl][half ^ 1][par][0] : -INFINITY;
      const float pbv = vote ? vote_val[hl][half ^ 1][par][1] : -INFINITY;
      gather_tile(v + 4, false);
      gather_tile(v + 5, false);
      gather_tile(v + 2, true);
      gather_tile(v + 3, true);
      // ---- value side of page 2k, then of page 2k+1
      auto value_side = [&](int w, const f32x16_t (&acc)[2], float mnew, float marg, float partner, bool mine) {
        if (!mine) return;  // not this head's entry: logged as not visited, state unchanged
        const float margin2 = fmaxf(marg, __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(partner))));
        const bool skip = skip_on && (margin2 < tau2);
        if (logging && half == 0 && lane == 0) {
          dec_lds[hl][wlds.vis_k[w] - k0] = skip ? 1 : 0;
          mar_lds[hl][wlds.vis_k[w] - k0] = margin2 * kLn2;
        }
        m2 = mnew;
        if (!skip) {
          maybe_rebase(m2, b2, l2, o);
          bf16x8_t pb[4];
          l2 += permlane32_sum(probs_tile(acc, scale_log2, b2, pb));
          pv_tile(v_slot(w), pb, lane, o);
        }
      };
      value_side(v, acc_a, mnew_a, marg_a, pa, mine_a);
      if (has_b) value_side(v + 1, acc_b, mnew_b, marg_b, pbv, mine_b);
    }
    wait_vmcnt<0>();  // no page gather may still be writing LDS past this point
    __syncthreads();  // the window's LDS (visit list, ring, log) is reused next
    if (logging && half == 0) flush_log(a, u, k0, wl, dec_lds[hl], mar_lds[hl], lane);
    __syncthreads();
  }
  if (logging && half == 0) fill_log_tail(a, u, lane);
  store_output<kPage>(a, u, o, l2, b2, r_blk, row_ok, lane);
}

// ---------------------------------------------------------------------------
// 128-token blocks: HW = 2 or 1 q heads per workgroup, four waves per head
// ---------------------------------------------------------------------------
// CoSA Appendix D.1 takes 128-row query tiles with one skip vote per tile, the row
// groups first reducing their own rows and the partial results then combined.  Here
// each of a head's four waves owns 32 rows of the 128-row block and writes its
// partial margin to LDS; after the barrier every wave takes the max of the four.
// A 128-token key block is two 64-key tiles in consecutive ring slots (tiles 2v and
// 2v+1 of the window), so the ring schedule of the 64-token kernel applies with one
// block per step: the key sides of both tiles (one running-max update and one vote
// for the block), the barrier, then the value sides under one exponent base.
// NPB: physical pages per logical block (128 / page_len); a 64-key tile spans SUB of
// them, or lies in half of one 128-token page (NPB = 1, row offset 64 x).
template <int HW, int NPB, bool MEMB>
__global__ __launch_bounds__(256 * HW) void osk_prefill_b128_kernel(const PrefillArgs a, int heads_per_group,
                                                                    int nsub) {
  constexpr int B = 2 * kPage;  // tokens per logical block
  constexpr int NW = 4 * HW;    // waves
  constexpr int NT = 64 * NW;   // threads
  constexpr int GW = NW / 2;    // waves that gather tiles (waves 0 .. GW-1: one per SIMD at HW = 2)
  constexpr int SUB = NPB == 1 ? 1 : NPB / 2;  // physical pages per 64-key tile
  constexpr int kWindow = window_len<NPB>();
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing * kPageBytes];
  __shared__ WindowLds<NPB> wlds;
  __shared__ uint8_t dec_lds[HW][kWindow];
  __shared__ float mar_lds[HW][kWindow];
  __shared__ float vote_val[HW][2][4];  // [head][step parity][quarter]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quarter = wave & 3;  // rows 32*quarter .. +31 of the block
  const int hl = wave >> 2;      // head within the workgroup
  const int hi = lane >> 5;
  const Unit u = decode_unit<HW, B>(a, heads_per_group, nsub, hl);
  const bool skip_on = a.delta > 0.f;
  const float scale_log2 = a.sm_scale * kLog2e;
  const float tau2 = skip_threshold2(a, u.L);
  const bool logging = a.decisions != nullptr;
  LDS_PTR(uint8_t) ring_lds = (LDS_PTR(uint8_t))ring;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring_lds;

  const int r_blk = quarter * 32 + (lane & 31);
  const int c_tok = u.i * B + r_blk;
  const bool row_ok = c_tok < u.L;
  bf16x8_t qf[8];
  load_q<B>(a, u, r_blk, row_ok, hi, qf);

  // online-softmax state as in the 64-token kernel (m2 running max, b2 lazy base)
  float m2 = -INFINITY, b2 = -INFINITY, l2 = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[nt][e] = 0.f;

  for (int x = threadIdx.x; x < (u.n_pages + 31) / 32; x += NT) wlds.seen_bits[x] = 0u;

  const int32_t* mrow = a.order_mask + ((int64_t)u.qb * a.hkv + u.g) * a.max_mask_len;
  const uint16_t* kbase = a.k + (int64_t)u.g * a.kv_sh;
  const uint16_t* vbase = a.v + (int64_t)u.g * a.kv_sh;
  const bool gatherer = wave < GW;
  TileGather<GW> tg;
  tg.init(a.kv_st, gatherer ? wave : 0, lane);

  for (int k0 = 0; k0 < u.len; k0 += kWindow) {
    const int wl = min(kWindow, u.len - k0);
    if (logging && quarter == 0)
      for (int x = lane; x < wl; x += 64) { dec_lds[hl][x] = 2; mar_lds[hl][x] = __builtin_nanf(""); }
    const int nv = resolve_window<NT, NPB, B, HW>(a, u, mrow, k0, wl, wlds, wave, lane, u.h - hl);
    COSA_CHECK(a, nv >= 0 && nv <= wl);
    wait_q_landed();
    const int ntiles = 2 * nv;
    auto k_slot = [&](int t) { return ring_addr + (uint32_t)(t % kRing) * kTileBytes; };
    auto v_slot = [&](int t) { return ring_addr + (uint32_t)(kRing * kTileBytes) + (uint32_t)(t % kRing) * kTileBytes; };
    // this wave's share of tile t (half t % 2 of visit t / 2); a second half wholly past
    // the sequence end is read from the first half's rows (finite values, masked logits)
    auto gather_tile = [&](int t, bool is_v) {
      if (!gatherer || t >= ntiles) return;
      const int blk = t >> 1;
      const int jp = __builtin_amdgcn_readfirstlane(wlds.vis_j[blk]) & 0xFFFF;
      const int valid = u.L - (jp * B + (t & 1) * kPage);
      const int xs = valid > 0 ? (t & 1) : 0;
      const uint16_t* sub_base[SUB];
#pragma unroll
      for (int x = 0; x < SUB; ++x) {
        const int ph = __builtin_amdgcn_readfirstlane(wlds.vis_phys[blk * NPB + (NPB == 1 ? 0 : xs * SUB + x)]);
        COSA_CHECK(a, ph >= 0 && ph < a.num_phys);
        sub_base[x] = (is_v ? vbase : kbase) + (int64_t)ph * a.kv_sp +
                      (NPB == 1 ? (int64_t)(xs * kPage) * a.kv_st : (int64_t)0);
      }
      tg.template issue<SUB>(sub_base, a.page_len, is_v ? v_slot(t) : k_slot(t), valid, is_v, wave, lane);
    };

    // prologue: K tiles of block 0 resident; V of block 0 and K of block 1 in flight
    gather_tile(0, false);
    gather_tile(1, false);
    if (nv > 0) {
      wait_vmcnt<0>();
      lds_barrier();
    }
    gather_tile(0, true);
    gather_tile(1, true);
    gather_tile(2, false);
    gather_tile(3, false);

    const bool vote = skip_on || logging;
    for (int v = 0; v < nv; ++v) {
      const int par = v & 1;
      const int vj = __builtin_amdgcn_readfirstlane(wlds.vis_j[v]);
      const int j = vj & 0xFFFF;
      const bool mine = !MEMB || ((vj >> (16 + hl)) & 1);  // the block belongs to this head
      const int key0 = j * B;
      // ---- key side (Eq. (1), (2), (5)) over the block's 128 keys
      f32x16_t acc_a[2], acc_b[2];
      float mloc = -INFINITY;
      if (mine) {
        qk_tile(k_slot(2 * v), qf, lane, acc_a);
        qk_tile(k_slot(2 * v + 1), qf, lane, acc_b);
        const bool diag = j == u.i;
        mask_tile_at(acc_a, key0, c_tok, u.L, hi, diag || u.L - key0 < kPage);
        mask_tile_at(acc_b, key0 + kPage, c_tok, u.L, hi, diag || u.L - key0 < B);
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fmaxf(acc_a[tt][e], acc_b[tt][e]));
        mloc = mul_unfused(permlane32_max(mx), scale_log2);
      }
      const float mnew = fmaxf(m2, mloc);
      const float dd = (row_ok && mloc != -INFINITY) ? (mloc - mnew) : -INFINITY;
      const float marg = max_lanes32(dd);
      if (vote && lane == 0) vote_val[hl][par][quarter] = marg;
      // every gather issued since the last barrier (K of block v+1, V of block v) has
      // landed for this wave
      wait_vmcnt<0>();
      // past the barrier: the K tiles of block v and the V tiles of block v-1 are free,
      // block v+1's K and block v's V are resident, and the four partial margins are
      // visible
      lds_barrier();
      float margin2 = -INFINITY;
      if (vote) {
        const float m01 = fmaxf(vote_val[hl][par][0], vote_val[hl][par][1]);
        const float m23 = fmaxf(vote_val[hl][par][2], vote_val[hl][par][3]);
        margin2 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fmaxf(m01, m23))));
      }
      gather_tile(2 * v + 4, false);
      gather_tile(2 * v + 5, false);
      gather_tile(2 * v + 2, true);
      gather_tile(2 * v + 3, true);
      // ---- value side of the block: both tiles under one exponent base
      const bool skip = skip_on && (margin2 < tau2);
      if (mine && logging && quarter == 0 && lane == 0) {
        dec_lds[hl][wlds.vis_k[v] - k0] = skip ? 1 : 0;
        mar_lds[hl][wlds.vis_k[v] - k0] = margin2 * kLn2;
      }
      m2 = mnew;
      if (mine && !skip) {
        maybe_rebase(m2, b2, l2, o);
        bf16x8_t pb[4];
        float rs = probs_tile(acc_a, scale_log2, b2, pb);
        pv_tile(v_slot(2 * v), pb, lane, o);
        rs += probs_tile(acc_b, scale_log2, b2, pb);
        pv_tile(v_slot(2 * v + 1), pb, lane, o);
        l2 += permlane32_sum(rs);
      }
    }
    wait_vmcnt<0>();  // no tile gather may still be writing LDS past this point
    __syncthreads();  // the window's LDS (visit list, ring, log) is reused next
    if (logging && quarter == 0) flush_log(a, u, k0, wl, dec_lds[hl], mar_lds[hl], lane);
    __syncthreads();
  }
  if (logging && quarter == 0) fill_log_tail(a, u, lane);
  store_output<B>(a, u, o, l2, b2, r_blk, row_ok, lane);
}

// ---------------------------------------------------------------------------
// library-held scratch for the prefill's workspace (callers that cannot allocate)
// ---------------------------------------------------------------------------
// The prefill's workspace (longest-first schedule and status block) for up to
// kMaxQBlocks query blocks lives in this array, one copy per device, held until the
// process ends.  Host code never uses the array's name as a device address: the
// address of this device's copy is looked up once per device (with that device
// current) and kept.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

// KV heads the grid works on together: the largest divisor of hkv whose pool slices (K
// and V of every physical page of those heads) fit in kPhaseBytes, three quarters of the
// chip's 256 MB last-level cache.  The pages that the concurrently running workgroups
// gather then come from a working set that fits that cache, instead of from the whole
// pool (537 MB at 128K tokens).
constexpr int64_t kPhaseBytes = (int64_t)192 << 20;
static int heads_per_phase(const PrefillArgs& a) {
  const int64_t per_head = (int64_t)a.num_phys * a.page_len * kHeadDim * 2 * 2;
  int best = 1;
  for (int d = 1; d <= a.hkv; ++d)
    if (a.hkv % d == 0 && (int64_t)d * per_head <= kPhaseBytes) best = d;
  return best;
}

hipError_t launch_prefill(const PrefillArgs& args, hipStream_t stream) {
  PrefillArgs a = args;
  a.heads_per_phase = heads_per_phase(a);
  if (a.total_qblocks == 0) return hipSuccess;
  const int G = a.hq / a.hkv;
  const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  const int nsub = G / HW;
  hipLaunchKernelGGL(osk_schedule_kernel, dim3(1), dim3(1024), 0, stream, a.mask_len, a.total_qblocks, a.hkv,
                     a.max_mask_len, a.sched, a.error_count);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.block == 2 * kPage) {
    // 128-token blocks: two heads (eight waves) per workgroup when the group size is even
    const int hw = (G % 2 == 0) ? 2 : 1;
    const int ns = G / hw;
    const dim3 grid((unsigned)a.total_qblocks * (unsigned)a.hkv * (unsigned)ns);
    const int npb = 2 * kPage / a.page_len;
    auto launch = [&](auto hw_c, auto npb_c) {
      constexpr int H = decltype(hw_c)::value, N = decltype(npb_c)::value;
      if (a.membership != nullptr)
        hipLaunchKernelGGL((osk_prefill_b128_kernel<H, N, true>), grid, dim3(256 * H), 0, stream, a, G, ns);
      else
        hipLaunchKernelGGL((osk_prefill_b128_kernel<H, N, false>), grid, dim3(256 * H), 0, stream, a, G, ns);
    };
    auto by_npb = [&](auto hw_c) {
      if (npb == 1) launch(hw_c, std::integral_constant<int, 1>{});
      else if (npb == 2) launch(hw_c, std::integral_constant<int, 2>{});
      else if (npb == 4) launch(hw_c, std::integral_constant<int, 4>{});
      else launch(hw_c, std::integral_constant<int, 8>{});
    };
    if (hw == 2) by_npb(std::integral_constant<int, 2>{});
    else by_npb(std::integral_constant<int, 1>{});
    return hipGetLastError();
  }
  const dim3 grid((unsigned)a.total_qblocks * (unsigned)a.hkv * (unsigned)nsub);
  const int sub = kPage / a.page_len;
  auto launch = [&](auto hw_c, auto sub_c) {
    constexpr int H = decltype(hw_c)::value, S = decltype(sub_c)::value;
    if (a.membership != nullptr)
      hipLaunchKernelGGL((osk_prefill_ring_kernel<H, S, true>), grid, dim3(128 * H), 0, stream, a, G, nsub);
    else
      hipLaunchKernelGGL((osk_prefill_ring_kernel<H, S, false>), grid, dim3(128 * H), 0, stream, a, G, nsub);
  };
  auto by_sub = [&](auto hw_c) {
    if (sub == 1) launch(hw_c, std::integral_constant<int, 1>{});
    else if (sub == 2) launch(hw_c, std::integral_constant<int, 2>{});
    else launch(hw_c, std::integral_constant<int, 4>{});
  };
  if (HW == 4) by_sub(std::integral_constant<int, 4>{});
  else if (HW == 2) by_sub(std::integral_constant<int, 2>{});
  else by_sub(std::integral_constant<int, 1>{});
  return hipGetLastError();
}

}  // namespace cosa_osk
