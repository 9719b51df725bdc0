// kernels_prefill.hip -- chunked prefill with compressed-sparse, compressed-dense
// and sliding-window branches ("CSA + HCA 混合注意力机制" §4.1-4.4, §5.1-5.2).
//
// A chunk of C new queries at positions P + i attends, per (tile of q_tile
// consecutive queries, kv head):
//   A  the top_k entries of the m_sparse mean-pooled stream, chosen with the
//      tile's pooled query against the fp32 copy of the pooled keys;
//   B  every entry of the m_dense mean-pooled stream;
//   C  the raw tokens [p - window + 1, p] of the cache (causal window);
// each with its own softmax; the three outputs are averaged.
//
// Kernels:
//   prefill_qbar_kernel    pooled tile queries (fp32)
//   prefill_scores_kernel  scores = qbar . pooled keys as an fp32 MFMA product
//                          ([tiles x d] . [d x entries] per kv head)
//   prefill_topk_kernel    exact top-k per (tile, kv head): MSB-first threshold
//                          search with wave ballots, then an index-ordered
//                          compaction (ascending output, lower index on ties)
//   prefill_attn_kernel    workgroups of 4 waves x 32 (query, head) rows (a
//                          256-row tile takes two workgroups); the branches' entries
//                          stream through double-buffered LDS in chunks of 64:
//                          S^T = K Q^T on bf16 MFMA, online softmax per row,
//                          O += P V on fp16 MFMA with V transposed in LDS.
#include <math.h>

#include "bsa_device.h"
#include "bsa_launch.h"

namespace bsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float PF_LOG2E = 1.4426950408889634f;
constexpr float PF_LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// pooled tile queries: qbar[b][tile][kvh][c] = sum over the tile's queries and
// the kv head's query heads of q[b][i][h][c]
__global__ void prefill_qbar_kernel(const uint16_t* __restrict__ q, int C, int Hq, int Hkv, int D,
                                    int q_tile, int n_tiles, float* __restrict__ qbar) {
  const int prob = blockIdx.x;
  const int b = prob / (n_tiles * Hkv), tile = (prob / Hkv) % n_tiles, kvh = prob % Hkv;
  const int g = Hq / Hkv;
  const int c = threadIdx.x;
  if (c >= D) return;
  const int i0 = tile * q_tile, i1 = min(C, i0 + q_tile);
  float s = 0.f;
  for (int i = i0; i < i1; ++i) {
    const uint16_t* qi = q + (((int64_t)b * C + i) * Hq + (int64_t)kvh * g) * D + c;
    for (int h = 0; h < g; ++h) s += __uint_as_float((uint32_t)qi[(int64_t)h * D] << 16);
  }
  qbar[(((int64_t)b * n_tiles + tile) * Hkv + kvh) * D + c] = s;
}

// ---------------------------------------------------------------------------
// scores[b][kvh][tile][j] = qbar[b][tile][kvh] . ks[b][kvh][j] (fp32).
// A wave computes S^T[16 entries x 16 tiles] with v_mfma_f32_16x16x4_f32:
// A = pooled-key rows (lane l: entry l%16), B = qbar^T (lane l: tile l%16);
// the k index l/16 of every step maps to dim 16m + 4(l/16) + e on both sides.
template <int D>
__global__ __launch_bounds__(256) void prefill_scores_kernel(const float* __restrict__ ks,
                                                             const float* __restrict__ qbar,
                                                             int n_tiles, int Hkv, int E,
                                                             float* __restrict__ scores) {
  constexpr int M = D / 16;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, j4 = lane >> 4;
  const int e0 = blockIdx.x * 64 + 16 * wave;
  if (e0 >= E) return;
  const float* krow = ks + (((int64_t)b * Hkv + kvh) * E + min(e0 + l16, E - 1)) * D;
  float4 ka[M];
#pragma unroll
  for (int m = 0; m < M; ++m) ka[m] = ld_stream(reinterpret_cast<const float4*>(krow + 16 * m + 4 * j4));
  for (int ng = 0; ng * 16 < n_tiles; ++ng) {
    const int tile = 16 * ng + l16;
    float4 qb[M];
    const float* qrow = qbar + (((int64_t)b * n_tiles + min(tile, n_tiles - 1)) * Hkv + kvh) * D;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      qb[m] = *reinterpret_cast<const float4*>(qrow + 16 * m + 4 * j4);
      if (tile >= n_tiles) qb[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m].x, qb[m].x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m].y, qb[m].y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m].z, qb[m].z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[m].w, qb[m].w, acc, 0, 0, 0);
    }
    // lane l holds entries e0 + 4(l/16) + i of tile 16ng + l%16
    if (tile < n_tiles) {
      float* dst = scores + (((int64_t)b * Hkv + kvh) * n_tiles + tile) * E;
      const int e = e0 + 4 * j4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e + i < E) dst[e + i] = acc[i];
    }
  }
}

// ---------------------------------------------------------------------------
// top-k per (b, tile, kvh).  Thread t owns the keys [KPT*t, KPT*t + KPT) in
// registers.  T = the k-th largest key is built bit by bit from the MSB:
// keep bit b set if at least k keys are >= (T | bit).  Then every key > T is
// taken and the first k - #(> T) keys equal to T in index order.
constexpr int PTK_THREADS = 1024;
constexpr int PTK_WAVES = PTK_THREADS / 64;

__device__ __forceinline__ int ptk_block_sum(int v, int* red, int parity) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[parity * PTK_WAVES + wave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < PTK_WAVES; ++w) t += red[parity * PTK_WAVES + w];
  return t;
}

// exclusive prefix over threads in thread order; *total gets the sum
__device__ __forceinline__ int ptk_block_exscan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < PTK_WAVES; ++w) {
    const int c = red[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

template <int KPT>
__global__ __launch_bounds__(PTK_THREADS) void prefill_topk_kernel(const float* __restrict__ scores,
                                                                   int n_tiles, int Hkv, int E,
                                                                   int k, int32_t* __restrict__ sel) {
  __shared__ int red[2 * PTK_WAVES];
  const int prob = blockIdx.x;  // sel order: [b][tile][kvh]
  const int b = prob / (n_tiles * Hkv), tile = (prob / Hkv) % n_tiles, kvh = prob % Hkv;
  const float* s = scores + (((int64_t)b * Hkv + kvh) * n_tiles + tile) * E;
  int32_t* out = sel + (int64_t)prob * k;
  const int tid = threadIdx.x;
  if (k >= E) {
    for (int j = tid; j < E; j += PTK_THREADS) out[j] = j;
    return;
  }
  uint32_t key[KPT];
  const int j0 = KPT * tid;
#pragma unroll
  for (int u = 0; u < KPT; ++u) key[u] = (j0 + u < E) ? order_key(s[j0 + u]) : 0u;  // 0: below any real key
  uint32_t T = 0;
  int parity = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) cnt += __popcll(__ballot(key[u] >= cand));
    const int total = ptk_block_sum((threadIdx.x & 63) == 0 ? cnt : 0, red, parity);
    parity ^= 1;
    if (total >= k) T = cand;
  }
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    n_gt += key[u] > T;
    n_eq += key[u] == T;
  }
  __syncthreads();
  int tot_gt, tot_eq, tot_sel;
  (void)ptk_block_exscan(n_gt, red, &tot_gt);
  const int need_eq = k - tot_gt;                 // >= 1 by the choice of T
  const int eq_first = ptk_block_exscan(n_eq, red, &tot_eq);
  // selected keys of this thread: all > T, and the keys == T whose rank in
  // index order is below need_eq
  int n_sel = n_gt + max(0, min(n_eq, need_eq - eq_first));
  int pos = ptk_block_exscan(n_sel, red, &tot_sel);
  int rank = eq_first;
#pragma unroll
  for (int u = 0; u < KPT; ++u) {
    bool take = key[u] > T;
    if (key[u] == T) take = rank++ < need_eq;
    if (take) out[pos++] = j0 + u;
  }
}

// ---------------------------------------------------------------------------
// attention over the three branches.
constexpr int PF_CH = 64;  // entries per chunk

struct PrefillAttnArgs {
  const uint16_t* q;     // [B][C][Hq][D]
  const uint16_t* k;     // [B][Hkv][stride][D]
  const uint16_t* v;
  const uint16_t* k4;    // [B][Hkv][E4][D]
  const uint16_t* v4;
  const uint16_t* k128;  // [B][Hkv][E128][D]
  const uint16_t* v128;
  const int32_t* sel;    // [B][n_tiles][Hkv][ksel]
  float* out;            // [B][C][Hq][D]
  float* lse3;           // [3][B][C][Hq] or null
  int B, C, Hq, Hkv, P, stride, E4, E128, ksel, window, q_tile, n_tiles;
  float scale_log2;
};

template <int NW, int NT>
__global__ __launch_bounds__(NW * 64) void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int D = 128, KS = D / 32, NTH = NW * 64;
  constexpr int RW = 16 * NT;  // (query, head) rows per wave
  constexpr int U = (PF_CH * (D / 8)) / NTH;  // 16-byte K (and V) pieces per thread per chunk
  __shared__ __align__(16) uint4 k_lds[2][PF_CH * (D / 8)];      // entry rows, 16 B pieces, xor-swizzled
  __shared__ __align__(16) uint16_t vt_lds[2][D * PF_CH];        // V^T fp16 [dim][entry], 8 B pieces swizzled
  __shared__ __align__(16) float xch[NW][2][RW];
  __shared__ __align__(16) uint4 q_lds[NW * RW * (D / 8)];      // the tile's rows, xor-swizzled

  constexpr int RWG = NW * RW;  // rows per workgroup
  const int g = a.Hq / a.Hkv;
  const int nrb = (a.q_tile * g) / RWG;  // workgroups per (tile, kv head)
  const int prob = blockIdx.x / nrb;
  const int row0 = (blockIdx.x % nrb) * RWG;  // this workgroup's first row of the tile
  const int b = prob / (a.n_tiles * a.Hkv), tile = (prob / a.Hkv) % a.n_tiles, kvh = prob % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  const int64_t pair = (int64_t)b * a.Hkv + kvh;

  // the tile's (query, head) rows -> LDS; row r = query r / g of the tile, head r % g
  for (int c = tid; c < NW * RW * (D / 8); c += NTH) {
    const int r = c / (D / 8), col = c % (D / 8);
    const int i = min(tile * a.q_tile + (row0 + r) / g, a.C - 1);
    const int h = kvh * g + (row0 + r) % g;
    q_lds[r * (D / 8) + (col ^ (r & 15))] =
        reinterpret_cast<const uint4*>(a.q + (((int64_t)b * a.C + i) * a.Hq + h) * D)[col];
  }
  int qpos[NT];  // absolute position of the row's query (for the window mask)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) qpos[nt] = a.P + tile * a.q_tile + (row0 + RW * wave + 16 * nt + l16) / g;

  // chunk schedule
  const int nA = (a.ksel + PF_CH - 1) / PF_CH;
  const int nB = (a.E128 + PF_CH - 1) / PF_CH;
  const int T0 = max(0, a.P + tile * a.q_tile - a.window + 1);
  const int T1 = min(a.P + a.C, a.P + tile * a.q_tile + a.q_tile);
  const int nC = (T1 - T0 + PF_CH - 1) / PF_CH;
  const int total = nA + nB + nC;
  const int32_t* sel = a.sel + ((int64_t)(b * a.n_tiles + tile) * a.Hkv + kvh) * a.ksel;

  // global -> registers for one chunk
  uint4 kreg[U], vreg[U];
  auto load_chunk = [&](int gc) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = tid + NTH * u;
      const int e = c / (D / 8), col = c % (D / 8);
      const uint16_t *kr, *vr;
      if (gc < nA) {
        const int j = min(gc * PF_CH + e, a.ksel - 1);
        const int64_t row = pair * a.E4 + sel[j];
        kr = a.k4 + row * D;
        vr = a.v4 + row * D;
      } else if (gc < nA + nB) {
        const int j = min((gc - nA) * PF_CH + e, a.E128 - 1);
        const int64_t row = pair * a.E128 + j;
        kr = a.k128 + row * D;
        vr = a.v128 + row * D;
      } else {
        const int t = min(T0 + (gc - nA - nB) * PF_CH + e, T1 - 1);
        const int64_t row = pair * a.stride + t;
        kr = a.k + row * D;
        vr = a.v + row * D;
      }
      kreg[u] = ld_stream(reinterpret_cast<const uint4*>(kr) + col);
      vreg[u] = ld_stream(reinterpret_cast<const uint4*>(vr) + col);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = tid + NTH * u;
      const int e = c / (D / 8), col = c % (D / 8);
      k_lds[buf][e * (D / 8) + (col ^ (e & 15))] = kreg[u];
      const uint32_t w[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int dim = 8 * col + 2 * x + y;
          const float f = y ? bf_hi(w[x]) : bf_lo(w[x]);
          const _Float16 hv = (_Float16)f;
          vt_lds[buf][dim * PF_CH + ((((e >> 2) ^ (dim & 15)) << 2) | (e & 3))] =
              __builtin_bit_cast(uint16_t, hv);
        }
      }
    }
  };

  f32x4_t O[NT][D / 16], osum[NT][D / 16];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int nd = 0; nd < D / 16; ++nd) {
      O[nt][nd] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      osum[nt][nd] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  load_chunk(0);
  for (int gc = 0; gc < total; ++gc) {
    const int buf = gc & 1;
    store_chunk(buf);
    __syncthreads();
    if (gc + 1 < total) load_chunk(gc + 1);
    // what this chunk holds
    const int br = gc < nA ? 0 : (gc < nA + nB ? 1 : 2);
    const int nvalid = br == 0 ? min(PF_CH, a.ksel - gc * PF_CH)
                               : (br == 1 ? min(PF_CH, a.E128 - (gc - nA) * PF_CH)
                                          : min(PF_CH, T1 - T0 - (gc - nA - nB) * PF_CH));
    const int tbase = T0 + (gc - nA - nB) * PF_CH;  // branch C: token of entry 0
    // S^T = K Q^T : lane gets entries 16mt + 4(l/16) + i of row 16nt + l%16
    f32x4_t s[NT][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      uint4 ka[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[ks] = k_lds[buf][(16 * mt + l16) * (D / 8) + ((4 * ks + j4) ^ l16)];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // Q^T fragment: lane l holds row RW*wave + 16nt + l%16, dims 32ks + 8(l/16) .. +8
        const int r = RW * wave + 16 * nt + l16;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 qv = q_lds[r * (D / 8) + ((4 * ks + j4) ^ l16)];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[ks]),
                                                        __builtin_bit_cast(bf16x8_t, qv),
                                                        acc, 0, 0, 0);
        }
        s[nt][mt] = acc;
      }
    }
    // online softmax per row; P packed to fp16 as the A operand of P V
    f16x8_t pa[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float z[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 16 * mt + 4 * j4 + i;
          bool ok = e < nvalid;
          if (br == 2) {
            const int t = tbase + e;
            ok = ok && t <= qpos[nt] && t > qpos[nt] - a.window;
          }
          z[mt][i] = ok ? s[nt][mt][i] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, z[mt][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
      m_run[nt] = m_new;
      float ps = 0.f;
      float p[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = __builtin_amdgcn_exp2f(z[mt][i] - m_use);
          ps += p[mt][i];
        }
      l_run[nt] = l_run[nt] * alpha + ps;
      if (j4 == 0) xch[wave][0][16 * nt + l16] = alpha;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pa[nt][kk][i] = (_Float16)p[2 * kk][i];
          pa[nt][kk][4 + i] = (_Float16)p[2 * kk + 1][i];
        }
    }
    wave_lds_sync();
    // rescale O rows (lane holds rows 16nt + 4(l/16) + i) by their alpha
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float4 al = *reinterpret_cast<const float4*>(&xch[wave][0][16 * nt + 4 * j4]);
#pragma unroll
      for (int nd = 0; nd < D / 16; ++nd) {
        O[nt][nd][0] *= al.x;
        O[nt][nd][1] *= al.y;
        O[nt][nd][2] *= al.z;
        O[nt][nd][3] *= al.w;
      }
    }
    // O += P V: B operand lane l = dim 16nd + l%16, entries of the P k-slots
#pragma unroll
    for (int nd = 0; nd < D / 16; ++nd) {
      const int dim = 16 * nd + l16;
      const uint2* vrow = reinterpret_cast<const uint2*>(&vt_lds[buf][dim * PF_CH]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint2 lo = vrow[(8 * kk + j4) ^ (dim & 15)];
        const uint2 hi = vrow[(8 * kk + 4 + j4) ^ (dim & 15)];
        const uint4 vb4 = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const f16x8_t vb = __builtin_bit_cast(f16x8_t, vb4);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          O[nt][nd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[nt][kk], vb, O[nt][nd], 0, 0, 0);
      }
    }
    // end of a branch: normalise, add into the running sum, reset
    const bool last = (gc == nA - 1) || (gc == nA + nB - 1) || (gc == total - 1);
    if (last) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float lt = l_run[nt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (j4 == 0) {
          xch[wave][1][16 * nt + l16] = lt;
          const int r = row0 + RW * wave + 16 * nt + l16;
          const int i = tile * a.q_tile + r / g;
          if (a.lse3 && i < a.C) {
            const int h = kvh * g + r % g;
            a.lse3[(((int64_t)br * a.B + b) * a.C + i) * a.Hq + h] = (m_run[nt] + log2f(lt)) * PF_LN2;
          }
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 l4 = *reinterpret_cast<const float4*>(&xch[wave][1][16 * nt + 4 * j4]);
        const float inv[4] = {1.f / l4.x, 1.f / l4.y, 1.f / l4.z, 1.f / l4.w};
#pragma unroll
        for (int nd = 0; nd < D / 16; ++nd) {
#pragma unroll
          for (int i = 0; i < 4; ++i) osum[nt][nd][i] = fmaf(O[nt][nd][i], inv[i], osum[nt][nd][i]);
          O[nt][nd] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        }
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.f;
      }
    }
    wave_lds_sync();
  }
  // out = (o_A + o_B + o_C) / 3; lane holds rows 16nt + 4(l/16) + i, dim 16nd + l%16
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + RW * wave + 16 * nt + 4 * j4 + i;
      const int qi = tile * a.q_tile + r / g;
      if (qi >= a.C) continue;
      const int h = kvh * g + r % g;
      float* dst = a.out + (((int64_t)b * a.C + qi) * a.Hq + h) * D + l16;
#pragma unroll
      for (int nd = 0; nd < D / 16; ++nd) dst[16 * nd] = osum[nt][nd][i] * (1.f / 3.f);
    }
}

// ---------------------------------------------------------------------------
size_t prefill_workspace_bytes(int B, int Hkv, int D, int n_tiles, int E4, int ksel, bool need_sel) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t s = al((size_t)B * n_tiles * Hkv * D * 4);           // qbar
  s += al((size_t)B * Hkv * n_tiles * (size_t)E4 * 4);        // scores
  if (need_sel) s += al((size_t)B * n_tiles * Hkv * (size_t)ksel * 4);
  return s;
}

int prefill_topk_kpt(int E4) {
  int kpt = 1;
  while (kpt * PTK_THREADS < E4) kpt *= 2;
  return kpt;
}

bool launch_prefill(const PrefillLaunch& L, hipStream_t st) {
  const int D = 128;
  const int g = L.Hq / L.Hkv;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* ws = static_cast<char*>(L.workspace);
  float* qbar = reinterpret_cast<float*>(ws);
  ws += al((size_t)L.B * L.n_tiles * L.Hkv * D * 4);
  float* scores = reinterpret_cast<float*>(ws);
  ws += al((size_t)L.B * L.Hkv * L.n_tiles * (size_t)L.E4 * 4);
  int32_t* sel = L.sel_out ? L.sel_out : reinterpret_cast<int32_t*>(ws);
  const unsigned probs = (unsigned)(L.B * L.n_tiles * L.Hkv);
  prefill_qbar_kernel<<<probs, D, 0, st>>>(L.q, L.C, L.Hq, L.Hkv, D, L.q_tile, L.n_tiles, qbar);
  dim3 sg((L.E4 + 63) / 64, L.Hkv, L.B);
  prefill_scores_kernel<128><<<sg, 256, 0, st>>>(L.k4f, qbar, L.n_tiles, L.Hkv, L.E4, scores);
  const int kpt = prefill_topk_kpt(L.E4);
#define BSA_PTK(KK)                                                                              \
  case KK:                                                                                       \
    prefill_topk_kernel<KK><<<probs, PTK_THREADS, 0, st>>>(scores, L.n_tiles, L.Hkv, L.E4,      \
                                                           L.ksel, sel);                         \
    break;
  switch (kpt) {
    BSA_PTK(1) BSA_PTK(2) BSA_PTK(4) BSA_PTK(8) BSA_PTK(16) BSA_PTK(32) BSA_PTK(64) BSA_PTK(128)
    default: return false;
  }
#undef BSA_PTK
  PrefillAttnArgs a;
  a.q = L.q; a.k = L.k; a.v = L.v; a.k4 = L.k4b; a.v4 = L.v4b; a.k128 = L.k128b; a.v128 = L.v128b;
  a.sel = sel; a.out = L.out; a.lse3 = L.lse3;
  a.B = L.B; a.C = L.C; a.Hq = L.Hq; a.Hkv = L.Hkv; a.P = L.P; a.stride = L.stride;
  a.E4 = L.E4; a.E128 = L.E128; a.ksel = L.ksel; a.window = L.window; a.q_tile = L.q_tile;
  a.n_tiles = L.n_tiles; a.scale_log2 = L.scale * PF_LOG2E;
  const int rows = L.q_tile * g;
  // 4 waves of 32 (query, head) rows per workgroup; 64-row tiles use 16 rows per wave
  switch (rows) {
    case 64: prefill_attn_kernel<4, 1><<<probs, 256, 0, st>>>(a); break;
    case 128: prefill_attn_kernel<4, 2><<<probs, 256, 0, st>>>(a); break;
    case 256: prefill_attn_kernel<4, 2><<<probs * 2, 256, 0, st>>>(a); break;
    default: return false;
  }
  return true;
}

}  // namespace bsa
