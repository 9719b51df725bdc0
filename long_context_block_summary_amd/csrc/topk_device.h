// Top-k of one (batch, kv head) pair's candidate block scores inside a single
// workgroup.  The selection of the hotdry.top post's importance ranking of
// the middle blocks ("CSA + HCA 混合注意力机制" §4.4 step 3): the k highest
// scores, equal scores taken in index order, written in ascending order.
//
// Each of the NTH threads holds KPT consecutive candidates in registers.  The
// k-th largest order key T is found in two steps:
//  1. value buckets: TOPK_BUCKETS equal-width buckets over [min, max] of the
//     scores.  The bucket of a score is a monotone function of it (one
//     subtraction, one product, a clamp and a truncation, each monotone), so
//     a higher bucket holds only higher scores; one LDS histogram and one
//     workgroup-wide scan give the bucket holding the k-th largest score and
//     how many scores lie above it;
//  2. inside that bucket: up to TOPK_RANK_MAX scores are ranked directly
//     (key descending, index ascending); a fuller bucket, or scores that are
//     not finite or all equal, go through four 8-bit radix passes over an LDS
//     histogram (HC copies, lane l counting into copy l % HC), counting only
//     the keys still in play.
// The kept list is then the keys above T and the first `remaining` keys equal
// to T (in index order), placed by two workgroup-wide prefix sums.
#pragma once

#include <float.h>

#include "bsa_device.h"

namespace bsa {

constexpr int TOPK_BUCKETS = 2048;   // value buckets of step 1
constexpr int TOPK_RANK_MAX = 256;   // bucket sizes step 2 ranks directly

template <int NTH, int HC>
struct TopkShared {
  union {
    uint32_t hist[HC][257];          // radix passes
    uint32_t bucket[TOPK_BUCKETS];   // value buckets
    uint2 cand[TOPK_RANK_MAX];       // (key, index) of the bucket holding T
  };
  float red[3][NTH / 64];
  uint32_t digit, above;
  int tb, tb_count, n_cand;
  uint32_t n_eq;
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

// sv[e] = row[base + tid * KPT + e] for the positions below len, 0 past it:
// float4 (float2) loads where the positions and the row are aligned for them
template <int KPT>
__device__ __forceinline__ void load_slots(const float* __restrict__ row, int base, int len,
                                           float (&sv)[KPT]) {
  const int p0 = base + (int)threadIdx.x * KPT;
  const bool al4 = ((base | len) & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0;
  const bool al2 = ((base | len) & 1) == 0 && (reinterpret_cast<uintptr_t>(row) & 7) == 0;
  if (KPT % 4 == 0 && al4) {  // uniform
#pragma unroll
    for (int j = 0; j < KPT / 4; ++j) {
      const float4 x = (p0 + 4 * j < len) ? *reinterpret_cast<const float4*>(row + p0 + 4 * j)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
      sv[4 * j] = x.x;
      sv[4 * j + 1] = x.y;
      sv[4 * j + 2] = x.z;
      sv[4 * j + 3] = x.w;
    }
  } else if (KPT % 2 == 0 && al2) {  // uniform
#pragma unroll
    for (int j = 0; j < KPT / 2; ++j) {
      const float2 x = (p0 + 2 * j < len) ? *reinterpret_cast<const float2*>(row + p0 + 2 * j)
                                          : make_float2(0.f, 0.f);
      sv[2 * j] = x.x;
      sv[2 * j + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int e = 0; e < KPT; ++e) sv[e] = (p0 + e < len) ? row[p0 + e] : 0.f;
  }
}

// Thread tid's sv[e] is the score of position p = base + tid * KPT + e; the
// candidates are the positions in [lo, hi) (other slots hold any value and
// are ignored).  Writes list[c0 + r] = the position of the r-th kept
// candidate, r < k, in ascending order.  Requires 0 < k < hi - lo, every
// candidate position held by some slot; every thread of the workgroup calls
// it; list may be in LDS or global memory.
template <int NTH, int KPT, int HC>
__device__ void topk_select_regs(const float (&sv)[KPT], int base, int lo, int hi, int k, int c0,
                                 int32_t* list, TopkShared<NTH, HC>& sh) {
  static_assert(TOPK_BUCKETS % NTH == 0, "whole buckets per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = base + tid * KPT;  // this thread's positions [p0, p0 + KPT)
  bool valid[KPT];
  uint32_t key[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    valid[e] = p0 + e >= lo && p0 + e < hi;
    key[e] = order_key(sv[e]);
  }

  // value range of the candidates, and whether any is not finite
  float mx = -INFINITY, nmn = -INFINITY, bad = 0.f;
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if (valid[e]) {
      mx = fmaxf(mx, sv[e]);
      nmn = fmaxf(nmn, -sv[e]);
      bad = __builtin_isfinite(sv[e]) ? bad : 1.f;
    }
  mx = wave_max(mx);
  nmn = wave_max(nmn);
  bad = wave_max(bad);
  if (lane == 0) {
    sh.red[0][wave] = mx;
    sh.red[1][wave] = nmn;
    sh.red[2][wave] = bad;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    mx = fmaxf(mx, sh.red[0][w]);
    nmn = fmaxf(nmn, sh.red[1][w]);
    bad = fmaxf(bad, sh.red[2][w]);
  }
  const float mn = -nmn;
  const float range = mx - mn;
  const float scale = (float)TOPK_BUCKETS / range;

  int tb = -1;                  // bucket holding T (-1: every candidate in play)
  uint32_t rem = (uint32_t)k;   // T's rank among the keys in play
  uint32_t T = 0, remaining = 0, n_eq_all = 0;  // n_eq_all: keys equal to T
  bool found = false;
  int bk[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) bk[e] = 0;
  if (bad == 0.f && range > 0.f && range <= FLT_MAX && scale <= FLT_MAX) {  // uniform
    for (int i = tid; i < TOPK_BUCKETS; i += NTH) sh.bucket[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      bk[e] = (int)fminf(fmaxf((sv[e] - mn) * scale, 0.f), (float)(TOPK_BUCKETS - 1));
      if (valid[e]) atomicAdd(&sh.bucket[bk[e]], 1u);
    }
    __syncthreads();
    // thread t owns buckets top - PER t .. top - PER t - PER + 1 (descending)
    constexpr int PER = TOPK_BUCKETS / NTH;
    uint32_t c[PER];
    uint32_t own = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      c[j] = sh.bucket[TOPK_BUCKETS - 1 - (tid * PER + j)];
      own += c[j];
    }
    int tot;
    const uint32_t exc = (uint32_t)wg_exscan<NTH>((int)own, sh.wtot, &tot);
    if (exc < rem && rem <= exc + own) {
      uint32_t acc = exc;
      for (int j = 0; j < PER; ++j) {
        if (acc + c[j] >= rem) {
          sh.tb = TOPK_BUCKETS - 1 - (tid * PER + j);
          sh.above = acc;
          sh.tb_count = (int)c[j];
          sh.n_cand = 0;
          break;
        }
        acc += c[j];
      }
    }
    __syncthreads();
    tb = sh.tb;
    rem -= sh.above;
    const int cnt = sh.tb_count;
    if (cnt <= TOPK_RANK_MAX) {  // uniform
#pragma unroll
      for (int e = 0; e < KPT; ++e)
        if (valid[e] && bk[e] == tb) {
          const int j = atomicAdd(&sh.n_cand, 1);
          sh.cand[j] = make_uint2(key[e], (uint32_t)(p0 + e));
        }
      __syncthreads();
      // T is the key of rank rem - 1 in (key descending, index ascending)
      for (int j = tid; j < cnt; j += NTH) {
        const uint2 me = sh.cand[j];
        uint32_t gt = 0, rank = 0, eq = 0;
        for (int i = 0; i < cnt; ++i) {
          const uint2 o = sh.cand[i];
          gt += (o.x > me.x) ? 1u : 0u;
          eq += (o.x == me.x) ? 1u : 0u;
          rank += (o.x > me.x || (o.x == me.x && o.y < me.y)) ? 1u : 0u;
        }
        if (rank == rem - 1) {
          sh.digit = me.x;
          sh.above = gt;
          sh.n_eq = eq;
        }
      }
      __syncthreads();
      T = sh.digit;
      remaining = rem - sh.above;
      n_eq_all = sh.n_eq;
      found = true;
    }
  }
  if (!found) {  // uniform: radix passes over the keys in play
    uint32_t prefix = 0;
    remaining = rem;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < HC * 257; i += NTH) (&sh.hist[0][0])[i] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const bool match = valid[e] && (tb < 0 || bk[e] == tb) &&
                           (pass == 0 || ((key[e] ^ prefix) >> (shift + 8)) == 0);
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
              sh.n_eq = c[e];  // after the last pass: the keys equal to T
              break;
            }
            acc += c[e];
          }
        }
      }
      __syncthreads();
      prefix |= sh.digit << shift;
      remaining -= sh.above;
      n_eq_all = sh.n_eq;
    }
    T = prefix;
  }
  // keys above T are all taken, then the first `remaining` keys equal to T
  // (all of them when that is every key equal to T: no rank needed)
  int tot;
  int eq_rank = 0;
  if (remaining < n_eq_all) {  // uniform
    int n_eq = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) n_eq += (valid[e] && key[e] == T) ? 1 : 0;
    eq_rank = wg_exscan<NTH>(n_eq, sh.wtot, &tot);
  }
  int n_sel = 0;
  bool sel[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const bool eq = valid[e] && key[e] == T;
    sel[e] = valid[e] && (key[e] > T || (eq && eq_rank < (int)remaining));
    eq_rank += eq ? 1 : 0;
    n_sel += sel[e] ? 1 : 0;
  }
  int pos = c0 + wg_exscan<NTH>(n_sel, sh.wtot, &tot);
#pragma unroll
  for (int e = 0; e < KPT; ++e)
    if (sel[e]) list[pos++] = p0 + e;
}

// the same for one pair's score row (nb blocks: sink [0, c0), candidates
// [c0, c1), local [c1, nb)): each thread's slots are an aligned run of row
// positions when the row fits the NTH * KPT slots, else a run of candidates
template <int NTH, int KPT, int HC>
__device__ void topk_into_list(const float* __restrict__ row, int nb, int c0, int c1, int k,
                               int32_t* list, TopkShared<NTH, HC>& sh) {
  const int base = (nb <= NTH * KPT) ? 0 : c0;
  float sv[KPT];
  load_slots<KPT>(row, base, nb, sv);
  topk_select_regs<NTH, KPT, HC>(sv, base, c0, c1, k, c0, list, sh);
}

}  // namespace bsa
