// Workgroup-wide selection and sorting of 64-bit keys in LDS, shared by the
// computation-order mask builders (device code only: included by the .hip sources).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osk_internal.h"

namespace cosa_osk {

static_assert(kMaxPagesBuilder <= 65536, "radix_select skips the id word's upper digit passes");

// Radix select: for each of nh segments (segment seg holds n keys whose 64-bit value is
// (hkey[seg * stride + r] << 32) | (r + r0), all distinct, r + r0 < 2^16), the k-th smallest key (k >= 1,
// k <= n) into s_prefix[seg], by eight 8-bit digit passes that all segments share.  Waves
// 0 .. nh-1 of the NT threads search the digit histograms.  Called by every thread; ends
// with a barrier.
constexpr int kSelectMaxSegments = 8;
template <int NT>
__device__ __forceinline__ void radix_select(const uint32_t* hkey, int stride, int nh, int n, int r0, int k,
                                             int (*hist)[256], uint64_t* s_prefix, int* s_k, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  if (tid < nh) {
    s_prefix[tid] = 0ull;
    s_k[tid] = k;
  }
  for (int pass = 0; pass < 8; ++pass) {
    // the low word of a key is a block id below kMaxPagesBuilder <= 2^16: its digits at
    // bits 16..31 are 0 for every key, so those passes would keep bin 0 and the count
    if (pass == 4 || pass == 5) continue;
    const int shift = 56 - 8 * pass;
    const uint64_t pmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int x = tid; x < nh * 256; x += NT) hist[x >> 8][x & 255] = 0;
    __syncthreads();
    for (int x = tid; x < nh * n; x += NT) {
      const int seg = x / n, r = x - seg * n;
      const uint64_t key = ((uint64_t)hkey[seg * stride + r] << 32) | (uint32_t)(r + r0);
      if ((key & pmask) == (s_prefix[seg] & pmask)) atomicAdd(&hist[seg][(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (wave < nh) {
      // the bin holding the segment's kk-th smallest remaining key; lane l sums bins 4l .. 4l+3
      const int kk = s_k[wave];
      const int c0 = hist[wave][4 * lane], c1 = hist[wave][4 * lane + 1];
      const int c2 = hist[wave][4 * lane + 2], c3 = hist[wave][4 * lane + 3];
      int incl = c0 + c1 + c2 + c3;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const int excl = incl - (c0 + c1 + c2 + c3);
      const uint64_t hit = __ballot(incl >= kk);
      if (hit != 0ull && lane == __builtin_ctzll(hit)) {
        int before = excl, b = 4 * lane;
        if (before + c0 < kk) {
          before += c0;
          ++b;
          if (before + c1 < kk) {
            before += c1;
            ++b;
            if (before + c2 < kk) {
              before += c2;
              ++b;
            }
          }
        }
        s_prefix[wave] |= (uint64_t)b << shift;
        s_k[wave] = kk - before;
      }
    }
    __syncthreads();
  }
}

// Ascending bitonic sort of n (a power of two) keys in LDS by NT threads.  The stages
// of each merge size kk (partner distances kk/2, kk/4, .., 1) are taken up to three at
// a time: the 2^t elements that t consecutive stages (distances 2^(p+t-1) .. 2^p) make
// interact differ only in address bits p .. p+t-1, so one thread loads them, runs the t
// stages' compare-exchanges in registers and stores them -- the same network, one LDS
// round trip and one barrier per group of stages.
template <int T>
__device__ __forceinline__ void bitonic_stages(uint64_t* keys, int n, int kk, int p, int tid, int nt) {
  constexpr int M = 1 << T;
  for (int g = tid; g < (n >> T); g += nt) {
    const int x0 = ((g >> p) << (p + T)) | (g & ((1 << p) - 1));
    const bool up = (x0 & kk) == 0;  // bit kk lies above the group's bits: one direction
    uint64_t e[M];
#pragma unroll
    for (int m = 0; m < M; ++m) e[m] = keys[x0 + (m << p)];
#pragma unroll
    for (int s = T - 1; s >= 0; --s) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (m & (1 << s)) continue;
        const uint64_t u = e[m], v = e[m | (1 << s)];
        if ((u > v) == up) {
          e[m] = v;
          e[m | (1 << s)] = u;
        }
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) keys[x0 + (m << p)] = e[m];
  }
}
template <int NT>
__device__ __forceinline__ void bitonic_block(uint64_t* keys, int n, int tid) {
  for (int kk = 2; kk <= n; kk <<= 1) {
    int top = 0;  // log2 of the largest partner distance of this merge: kk / 2
    while ((2 << top) < kk) ++top;
    for (int hi = top; hi >= 0; hi -= 3) {
      const int t = hi + 1 < 3 ? hi + 1 : 3;  // stages in this group: distances 2^hi .. 2^(hi-t+1)
      const int p = hi - t + 1;
      if (t == 3) bitonic_stages<3>(keys, n, kk, p, tid, NT);
      else if (t == 2) bitonic_stages<2>(keys, n, kk, p, tid, NT);
      else bitonic_stages<1>(keys, n, kk, p, tid, NT);
      __syncthreads();
    }
  }
}

}  // namespace cosa_osk
