// Top-k of one (batch, kv head) pair's candidate block scores inside a single
// workgroup, for kernels that select before they attend.  The same selection
// as topk_reg_kernel (the hotdry.top post's importance selection of the
// middle blocks; "CSA + HCA 混合注意力机制" §4.4 step 3): the k highest
// scores, equal scores taken in index order, written in ascending order.
//
// Each of the NTH threads holds KPT consecutive candidates in registers.  The
// k-th largest order key T is found by four 8-bit radix passes over an LDS
// histogram (HC copies, lane l counting into copy l % HC); the kept list is
// then the keys above T and the first `remaining` keys equal to T, placed by
// two workgroup-wide prefix sums.
#pragma once

#include "bsa_device.h"

namespace bsa {

template <int NTH, int HC>
struct TopkShared {
  uint32_t hist[HC][257];
  uint32_t digit, above;
  int wtot[NTH / 64];
};

// exclusive prefix sum of x over the NTH threads in thread order; *total
// gets the sum.  Every thread of the workgroup calls it.
template <int NTH>
__device__ __forceinline__ int wg_exscan(int x, int* wtot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const int c = wtot[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + inc - x;
}

// list[c0 + r] = c0 + (index of the r-th kept candidate), r < k, for the
// candidate scores s[0, n).  Requires 0 < k < n <= NTH * KPT; every thread of
// the workgroup calls it; list may be in LDS or global memory.
template <int NTH, int KPT, int HC>
__device__ void topk_into_list(const float* __restrict__ s, int n, int k, int c0, int32_t* list,
                               TopkShared<NTH, HC>& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int i0 = tid * KPT;  // this thread's candidates [i0, i0 + KPT)
  uint32_t key[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) key[e] = order_key(s[min(i0 + e, n - 1)]);
  uint32_t prefix = 0;
  uint32_t remaining = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < HC * 257; i += NTH) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const bool match = i0 + e < n && (pass == 0 || ((key[e] ^ prefix) >> (shift + 8)) == 0);
      if (match) atomicAdd(&sh.hist[tid % HC][(key[e] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending order)
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = 0;
#pragma unroll
        for (int cp = 0; cp < HC; ++cp) c[e] += sh.hist[cp][255 - 4 * lane - e];
      }
      const uint32_t own = c[0] + c[1] + c[2] + c[3];
      uint32_t inc = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(inc, off);
        if (lane >= off) inc += t;
      }
      const uint32_t exc = inc - own;
      if (exc < remaining && remaining <= inc) {
        uint32_t acc = exc;
        for (int e = 0; e < 4; ++e) {
          if (acc + c[e] >= remaining) {
            sh.digit = (uint32_t)(255 - 4 * lane - e);
            sh.above = acc;
            break;
          }
          acc += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    remaining -= sh.above;
  }
  // keys above T are all taken, then the first `remaining` keys equal to T
  const uint32_t T = prefix;
  int n_eq = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) n_eq += (i0 + e < n && key[e] == T) ? 1 : 0;
  int tot;
  int eq_rank = wg_exscan<NTH>(n_eq, sh.wtot, &tot);
  int n_sel = 0;
  bool sel[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const bool valid = i0 + e < n;
    const bool eq = valid && key[e] == T;
    sel[e] = valid && (key[e] > T || (eq && eq_rank < (int)remaining));
    eq_rank += eq ? 1 : 0;
    n_sel += sel[e] ? 1 : 0;
  }
  int pos = c0 + wg_exscan<NTH>(n_sel, sh.wtot, &tot);
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if (sel[e]) list[pos++] = c0 + i0 + e;
}

}  // namespace bsa
