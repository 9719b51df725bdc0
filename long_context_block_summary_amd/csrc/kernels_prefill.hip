// kernels_prefill.hip -- chunked prefill with compressed-sparse, compressed-dense
// and sliding-window branches ("CSA + HCA 混合注意力机制" §4.1-4.4, §5.1-5.4).
//
// A chunk of C new queries at positions P + i attends, per (tile of q_tile
// consecutive queries, kv head):
//   A  the top_k entries of the m_sparse mean-pooled stream, chosen with the
//      tile's pooled query against the bf16 pooled keys themselves (or, as an
//      option, against an fp32 copy of them);
//   B  every entry of the m_dense mean-pooled stream;
//   C  the raw tokens [p - window + 1, p] of the cache (causal window).
// The branches are averaged (each with its own softmax) or joined in one
// softmax over their concatenated logits (§4.3); an optional per-head sink
// logit (§5.4) joins the softmax with a zero value.
//
// Kernels:
//   prefill_qbar_kernel    pooled tile queries (fp32)
//   prefill_scores_bf16_kernel  scores = qbar . bf16 pooled keys ([tiles x d] .
//                          [d x entries] per kv head) on bf16 MFMA, qbar split
//                          exactly into three bf16 terms
//   prefill_scores_kernel  the same against the fp32 keys, fp32 MFMA
//   prefill_topk_kernel    exact top-k per (tile, kv head): the k-th largest
//                          key bracketed from a sample (else fixed by MSB-first
//                          bit passes), its open bits as radix digits over the
//                          keys staged in LDS, then an index-ordered output
//                          (ascending, lower index on ties)
//   prefill_attn_kernel    one workgroup of 16*NT*NW (query, head) rows per
//                          (tile, kv head); the branches' entries stream through
//                          double-buffered LDS in chunks of 64: S^T = K Q^T on
//                          bf16 MFMA, online softmax per row, O += P V on fp16
//                          MFMA with V transposed in LDS; branch ends fold O / l
//                          into a partial sum kept in LDS (fp16), written to the
//                          output once, at the last branch.
#include <math.h>

#include "bsa_device.h"
#include "bsa_launch.h"

namespace bsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float PF_LOG2E = 1.4426950408889634f;
constexpr float PF_LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// pooled tile queries: qbar[b][tile][kvh][c] = sum over the tile's queries and
// the kv head's query heads of q[b][i][h][c].  One workgroup per (b, tile,
// kv head): thread t sums the 16-byte piece t%16 of every 16th (query, head)
// row, then the 16 row groups are added through LDS.
__global__ __launch_bounds__(256) void prefill_qbar_kernel(const uint16_t* __restrict__ q, int C,
                                                           int Hq, int Hkv, int q_tile, int n_tiles,
                                                           float* __restrict__ qbar) {
  constexpr int D = 128;
  __shared__ float part[16][D];
  const int prob = blockIdx.x;
  const int b = prob / (n_tiles * Hkv), tile = (prob / Hkv) % n_tiles, kvh = prob % Hkv;
  const int g = Hq / Hkv;
  const int t = threadIdx.x, col = t % 16, rg = t / 16;
  const int i0 = tile * q_tile;
  const int rows = min(q_tile, C - i0) * g;  // valid (query, head) rows of the tile
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  // r / g as (r * gm) >> 24 with gm = ceil(2^24 / g): exact for r, g <= 256
  // (a tile holds at most 256 rows), and one multiply instead of an integer
  // division per row
  const uint32_t gm = (1u << 24) / (uint32_t)g + ((1u << 24) % (uint32_t)g != 0u ? 1u : 0u);
  // rows in batches of 16 per thread, each batch's loads issued together
  // (a batch slot past the tile's end reads row 0 and adds nothing); the
  // rows are still added in order
  constexpr int RB = 16;
  for (int r0 = rg; r0 < rows; r0 += 16 * RB) {
    uint4 piece[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int r = r0 + 16 * u < rows ? r0 + 16 * u : 0;
      const int rq = (int)(((uint32_t)r * gm) >> 24);
      const int i = i0 + rq, h = kvh * g + (r - rq * g);
      piece[u] = reinterpret_cast<const uint4*>(q + (((int64_t)b * C + i) * Hq + h) * D)[col];
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      float f[8];
      unpack8(piece[u], f);
      if (r0 + 16 * u < rows) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += f[c];
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) part[rg][8 * col + c] = acc[c];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][t];
    qbar[(((int64_t)b * n_tiles + tile) * Hkv + kvh) * D + t] = s;
  }
}

// ---------------------------------------------------------------------------
// scores[b][kvh][tile][j] = qbar[b][tile][kvh] . ks[b][kvh][j] (fp32), row
// stride Es.  A wave computes S^T[16 entries x 16 tiles] tiles with
// v_mfma_f32_16x16x4_f32: A = pooled-key rows (lane l: entry l%16), B = qbar^T
// (lane l: tile l%16); the k index l/16 of every step maps to dim
// 16m + 4(l/16) + e on both sides.  Each wave walks PSC_GROUPS groups of 16
// consecutive entries, loading group i+1 into a second register set while the
// MFMAs of group i run; the pooled queries of all tiles sit in LDS.
constexpr int PSC_GROUPS = 8;     // 16-entry groups per wave
constexpr int PSC_MAX_TILES = 64; // pooled queries held in LDS per workgroup

template <int D, int NTB>
__global__ __launch_bounds__(256) void prefill_scores_kernel(const float* __restrict__ ks,
                                                             const float* __restrict__ qbar,
                                                             int n_tiles, int Hkv, int E, int Es,
                                                             float* __restrict__ scores) {
  constexpr int M = D / 16;
  __shared__ __align__(16) float qs[PSC_MAX_TILES][D + 4];  // +16 B per row: rows spread over the banks
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  // NTB = ceil(n_tiles / 16) tile blocks of 16, a compile-time count: with
  // the stores in a loop of run-time length the compiler waited for every
  // load (the next group's prefetch included) before each group's MFMAs
  constexpr int ntb = NTB;
  for (int c = tid; c < ntb * 16 * D; c += 256) {
    const int tl = c / D, dd = c % D;
    qs[tl][dd] = tl < n_tiles ? qbar[(((int64_t)b * n_tiles + tl) * Hkv + kvh) * D + dd] : 0.f;
  }
  __syncthreads();
  const float* kbase = ks + ((int64_t)b * Hkv + kvh) * E * D;
  float* sbase = scores + ((int64_t)b * Hkv + kvh) * n_tiles * Es;
  const int e_first = (blockIdx.x * 4 + wave) * (16 * PSC_GROUPS);
  float4 ka[2][M];
  auto load = [&](int set, int gi) {
    const float* krow = kbase + (int64_t)min(e_first + 16 * gi + l16, E - 1) * D;
#pragma unroll
    for (int m = 0; m < M; ++m)
      ka[set][m] = ld_stream(reinterpret_cast<const float4*>(krow + 16 * m + 4 * j4));
  };
  auto group = [&](int set, int gi) {
    const int e = e_first + 16 * gi + 4 * j4;  // lane's first entry of the output tile
#pragma unroll
    for (int tb = 0; tb < ntb; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float4 qb = *reinterpret_cast<const float4*>(&qs[16 * tb + l16][16 * m + 4 * j4]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[set][m].x, qb.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[set][m].y, qb.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[set][m].z, qb.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[set][m].w, qb.w, acc, 0, 0, 0);
      }
      // lane l holds entries e + i of tile 16tb + l%16
      const int tile = 16 * tb + l16;
      if (tile < n_tiles) {
        float* dst = sbase + (int64_t)tile * Es;
        if (e + 3 < E) {
          *reinterpret_cast<float4*>(dst + e) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e + i < E) dst[e + i] = acc[i];
        }
      }
    }
  };
  // groups past E are loaded clamped (and their stores skipped), so the
  // loads stay unconditional
  load(0, 0);
#pragma unroll
  for (int gi = 0; gi < PSC_GROUPS; gi += 2) {
    load(1, gi + 1);
    group(0, gi);
    if (gi + 2 < PSC_GROUPS) load(0, gi + 2);
    group(1, gi + 1);
  }
}

// ---------------------------------------------------------------------------
// The same scores against the bf16 pooled keys (the compressed cache branch A
// attends).  The pooled query of a tile (fp32) is split into three bf16 terms
// hi + mid + lo, each the next 8 significant bits, which sum to it exactly;
// v_mfma_f32_16x16x32_bf16 then forms every product key_c * term_c exactly and
// only the fp32 accumulation rounds, as in the fp32 kernel.  A = key rows
// (lane l: entry l%16, dims 32f + 8(l/16) .. +8, one 16-byte load per step),
// B = the terms of 16 tiles (lane l: tile l%16, the same dims), read from LDS
// rows padded by 16 bytes so the 16 tiles of one read fall on distinct banks.
// The output layout and the 16-entry groups per wave are the fp32 kernel's.
constexpr int PSB_GROUPS = 8;  // 16-entry groups per wave

template <int D, int NTB>
__global__ __launch_bounds__(256) void prefill_scores_bf16_kernel(
    const uint16_t* __restrict__ kb, const float* __restrict__ qbar, int n_tiles, int Hkv, int E,
    int Es, float* __restrict__ scores) {
  constexpr int F = D / 32;      // 32-dim steps of one MFMA
  constexpr int RU = D / 8 + 1;  // 16-byte units per LDS row (+1 of padding)
  __shared__ __align__(16) uint4 qt[3][NTB * 16][RU];
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  // the three terms of 8 consecutive dims of one tile per thread and step
  for (int c = tid; c < NTB * 16 * (D / 8); c += 256) {
    const int tl = c / (D / 8), p = c % (D / 8);
    float x[8];
    if (tl < n_tiles) {
      const float4* src =
          reinterpret_cast<const float4*>(qbar + (((int64_t)b * n_tiles + tl) * Hkv + kvh) * D + 8 * p);
      const float4 x0 = src[0], x1 = src[1];
      x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
      x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    uint32_t t[3][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // x - hi and r1 - mid are exact in fp32 (at most 16 and 8 significant bits)
      t[0][e] = bf16_rne(x[e]);
      const float r1 = x[e] - bf_lo(t[0][e]);
      t[1][e] = bf16_rne(r1);
      t[2][e] = bf16_rne(r1 - bf_lo(t[1][e]));
    }
#pragma unroll
    for (int s = 0; s < 3; ++s)
      qt[s][tl][p] = make_uint4(t[s][0] | (t[s][1] << 16), t[s][2] | (t[s][3] << 16),
                                t[s][4] | (t[s][5] << 16), t[s][6] | (t[s][7] << 16));
  }
  __syncthreads();
  const uint16_t* kbase = kb + ((int64_t)b * Hkv + kvh) * E * D;
  float* sbase = scores + ((int64_t)b * Hkv + kvh) * n_tiles * Es;
  const int e_first = (blockIdx.x * 4 + wave) * (16 * PSB_GROUPS);
  uint4 ka[2][F];
  auto load = [&](int set, int gi) {
    const uint4* krow =
        reinterpret_cast<const uint4*>(kbase + (int64_t)min(e_first + 16 * gi + l16, E - 1) * D);
#pragma unroll
    for (int f = 0; f < F; ++f) ka[set][f] = ld_stream(krow + 4 * f + j4);
  };
  auto group = [&](int set, int gi) {
    const int e = e_first + 16 * gi + 4 * j4;  // lane's first entry of the output tile
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < F; ++f)
#pragma unroll
        for (int s = 2; s >= 0; --s)  // smallest term first
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, ka[set][f]),
              __builtin_bit_cast(bf16x8_t, qt[s][16 * tb + l16][4 * f + j4]), acc, 0, 0, 0);
      // lane l holds entries e + i of tile 16tb + l%16
      const int tile = 16 * tb + l16;
      if (tile < n_tiles) {
        float* dst = sbase + (int64_t)tile * Es;
        if (e + 3 < E) {
          *reinterpret_cast<float4*>(dst + e) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (e + i < E) dst[e + i] = acc[i];
        }
      }
    }
  };
  // groups past E are loaded clamped (and their stores skipped)
  load(0, 0);
#pragma unroll
  for (int gi = 0; gi < PSB_GROUPS; gi += 2) {
    load(1, gi + 1);
    group(0, gi);
    if (gi + 2 < PSB_GROUPS) load(0, gi + 2);
    group(1, gi + 1);
  }
}

// ---------------------------------------------------------------------------
// top-k per (b, tile, kvh) over the E scores of a row (row stride Es, a
// multiple of 4).  Wave w owns the keys [64*KPT*w, 64*KPT*(w+1)); lane l holds
// keys 256v + 4l + c (v < KPT/4, c < 4) of that range, so each float4 load of
// a wave reads 1 KB of consecutive scores.  T = the k-th largest key; every
// key > T is taken, and the first k - #(> T) keys equal to T in index order;
// the output is written in index order.  How T is found is described at the
// threshold search below.
constexpr int PTK_MAX_WAVES = 16;  // 1024 threads
static_assert(PTK_MAX_WAVES * 64 * 128 >= PREFILL_MAX_E4, "largest key count per thread is 128");

constexpr int PTK_UND = 16384;  // undecided keys staged in LDS for the open bits
constexpr int PTK_BUCKETS = 2048;  // value buckets over the staged keys' range
constexpr int PTK_RANK_MAX = 256;  // keys of the threshold bucket ranked directly

// block sum of one value per wave (lane 0's), through LDS slot set `parity`
template <int NWV>
__device__ __forceinline__ int ptk_block_sum(int v, int (*red)[PTK_MAX_WAVES], int parity) {
  if ((threadIdx.x & 63) == 0) red[parity][threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) t += red[parity][w];
  return t;
}

// exclusive prefix over threads in thread order; *total gets the sum
template <int NWV>
__device__ __forceinline__ int ptk_block_exscan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  __syncthreads();
  if (lane == 63) red[wave] = inc;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int c = red[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// cnt + (key >= cand), through VCC: one compare mask live at a time (the
// compiler otherwise keeps every compare of an unrolled pass in SGPR pairs)
__device__ __forceinline__ int add_ge(int cnt, uint32_t key, uint32_t cand) {
  asm("v_cmp_ge_u32_e32 vcc, %1, %2\n\tv_addc_co_u32_e32 %0, vcc, 0, %0, vcc"
      : "+v"(cnt)
      : "v"(key), "v"(cand)
      : "vcc");
  return cnt;
}

// exclusive prefix of x over the lanes of the wave; *total gets the wave sum
__device__ __forceinline__ int wave_exscan(int x, int* total) {
  const int lane = threadIdx.x & 63;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(inc, off);
    if (lane >= off) inc += t;
  }
  *total = __shfl(inc, 63);
  return inc - x;
}

template <int KPT, int PTK_THREADS>
__global__ __launch_bounds__(PTK_THREADS) void prefill_topk_kernel(const float* __restrict__ scores,
                                                                   int n_tiles, int Hkv, int E,
                                                                   int Es, int k,
                                                                   int32_t* __restrict__ sel) {
  constexpr int NV = KPT / 4;
  constexpr int PTK_WAVES = PTK_THREADS / 64;
  __shared__ int red[2][PTK_MAX_WAVES];
  __shared__ int wcnt[2][PTK_WAVES];
  // staged keys (the bracket path: in index order, their indices in und_idx);
  // a dummy slot per lane past UND takes the writes of unstaged keys.  A row
  // never stages more keys than a workgroup holds, so the small variants keep
  // small arrays (and room for more workgroups per CU).
  constexpr int UND = PTK_THREADS * KPT < PTK_UND ? PTK_THREADS * KPT : PTK_UND;
  __shared__ uint32_t und[UND + 64];
  __shared__ uint32_t und_idx[UND + 64];
  __shared__ uint32_t dhist[4][256];      // one histogram per digit of the open bits
  __shared__ uint32_t samp[PTK_THREADS];  // the bracket's sample
  __shared__ int bsum[PTK_WAVES];
  __shared__ uint32_t bmax[PTK_WAVES];
  __shared__ uint32_t bhist[PTK_BUCKETS];  // value buckets of the staged keys
  __shared__ uint2 bcand[PTK_RANK_MAX];    // (key, staged position) of the bucket holding T
  __shared__ int bk_sel, bk_cnt, bk_n;
  __shared__ uint32_t bk_above, bk_T;
  const int prob = blockIdx.x;  // sel order: [b][tile][kvh]
  const int b = prob / (n_tiles * Hkv), tile = (prob / Hkv) % n_tiles, kvh = prob % Hkv;
  const float* s = scores + (((int64_t)b * Hkv + kvh) * n_tiles + tile) * Es;
  int32_t* out = sel + (int64_t)prob * k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (k >= E) {
    for (int j = tid; j < E; j += PTK_THREADS) out[j] = j;
    return;
  }
  const int wbase = wave * 64 * KPT;
  // All loads are issued before any key is formed: the raw bits land in the
  // key registers themselves, so every load of the row is in flight at once
  // (with the keys formed load by load, the compiler issued the loads one
  // memory latency apart).
  uint32_t key[NV][4];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    // branch-free: the load is clamped into the (padded) row
    const int j = wbase + 256 * v + 4 * lane;
    const uint4 r = *reinterpret_cast<const uint4*>(s + min(j, Es - 4));
    key[v][0] = r.x;
    key[v][1] = r.y;
    key[v][2] = r.z;
    key[v][3] = r.w;
  }
  // the empty asm statements are ordered after the barrier, and each key is
  // formed from its statement's output: no key work moves between the loads
  // (only where the compiler serialized them: the wide 512-thread variants;
  // the 1024-thread variant's keys exceed its registers anyway)
  if constexpr (PTK_THREADS <= 512 && KPT >= 64) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < NV; ++v)
      asm volatile("" : "+v"(key[v][0]), "+v"(key[v][1]), "+v"(key[v][2]), "+v"(key[v][3]));
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int j = wbase + 256 * v + 4 * lane;
    // all-ones where j + c < E (sign of j + c - E), else 0: keys past E are 0,
    // below any real key
#pragma unroll
    for (int c = 0; c < 4; ++c)
      key[v][c] = order_key(__uint_as_float(key[v][c])) & (uint32_t)((j + c - E) >> 31);
  }
  // Threshold search: T = the k-th largest key.
  //
  // First a bracket from a sample.  Each thread contributes one key, from its
  // register group lane % NV so that the sample spreads over the row; with
  // mu = k * samples / E the expected number of samples at or above T, the
  // r-th largest sample, r = mu + 7 sqrt(mu) + 4, lies below T with a wide
  // margin.  One pass counts the keys at or above it (n_lo) and finds the
  // row's largest key; when k <= n_lo <= UND those keys are staged in LDS
  // and T lies between the bracket and the maximum, sharing their common
  // leading bits.  Otherwise (a sample that misses: heavy ties, tiny rows)
  // full passes over the registers fix T bit by bit from the MSB until at
  // most UND keys remain undecided, and those are staged.  The open low
  // bits of T are then found as 8-bit radix digits over the staged keys.
  uint32_t T = 0;
  int n_top = 0;  // keys above the undecided range (all among the top k)
  int n_und = 0;  // undecided keys staged in und
  int sh = 32;    // the bits of T below sh are open
  bool staged = false;
  uint32_t b_lo = 0u, b_hi = 0u;  // the staged keys' range [bracket, row maximum]
  {
    uint32_t t[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) t[v] = key[v][0];
#pragma unroll
    for (int step = 1; step < NV; step <<= 1)
#pragma unroll
      for (int v = 0; v + step < NV; v += 2 * step) t[v] = (lane & step) ? t[v + step] : t[v];
    samp[tid] = t[0];  // keys past E are 0: below every candidate
  }
  __syncthreads();
  const float mu = (float)k * (float)PTK_THREADS / (float)E;
  const int r_s = __builtin_amdgcn_readfirstlane((int)ceilf(mu + 7.f * sqrtf(mu) + 4.f));
  if (r_s <= PTK_THREADS / 2) {  // uniform
    // every wave finds the r_s-th largest sample itself (no barrier)
    constexpr int NS = PTK_THREADS / 64;
    uint32_t sm[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) sm[i] = samp[NS * lane + i];
    uint32_t ts = 0;
    for (int b = 31; b >= 0; --b) {
      const uint32_t cand = ts | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < NS; ++i) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(sm[i] >= cand));
      if (cnt >= r_s) ts = cand;
    }
    if (ts != 0u) {  // uniform
      int mine = 0;
      uint32_t kmx = 0;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          mine = add_ge(mine, key[v][c], ts);
          kmx = max(kmx, key[v][c]);
        }
      int inc = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int x = __shfl_up(inc, off);
        if (lane >= off) inc += x;
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, off));
      if (lane == 63) bsum[wave] = inc;
      if (lane == 0) bmax[wave] = kmx;
      __syncthreads();
      int before = 0, n_lo = 0;
      uint32_t mx = 0;
#pragma unroll
      for (int w = 0; w < PTK_WAVES; ++w) {
        const int cw = bsum[w];
        before += w < wave ? cw : 0;
        n_lo += cw;
        mx = max(mx, bmax[w]);
      }
      if (n_lo >= k && n_lo <= UND) {  // uniform
        // The keys at or above the bracket, with their indices, in index
        // order: the wave's block starts after the earlier waves' keys; per
        // group of 256 keys the lane's count (0..4) as three ballots of its
        // bits gives its position (weighted mbcnt) and the group's total
        // (weighted popcount).  Branch-free: unstaged keys write a dummy slot.
        int pos = 0;
#pragma unroll
        for (int w = 0; w < PTK_WAVES; ++w) pos += w < wave ? bsum[w] : 0;
        const int dummy = UND + lane;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          int ns = 0;
#pragma unroll
          for (int c = 0; c < 4; ++c) ns += key[v][c] >= ts ? 1 : 0;
          const uint64_t b0 = __builtin_amdgcn_ballot_w64((ns & 1) != 0);
          const uint64_t b1 = __builtin_amdgcn_ballot_w64((ns & 2) != 0);
          const uint64_t b2 = __builtin_amdgcn_ballot_w64((ns & 4) != 0);
          int p = pos + (int)(lane_prefix(b0) + 2 * lane_prefix(b1) + 4 * lane_prefix(b2));
          // the group's indices from an opaque copy of the lane id: formed
          // here, not ahead of time for every group
          int lnv = lane;
          asm volatile("" : "+v"(lnv));
          const int j = wbase + 256 * v + 4 * lnv;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool in = key[v][c] >= ts;
            // separate arrays: a 64-bit write would need each key in a
            // register pair with its index
            const int a = in ? p : dummy;
            und[a] = key[v][c];
            und_idx[a] = (uint32_t)(j + c);
            p += in ? 1 : 0;
          }
          pos += __builtin_popcountll(b0) + 2 * __builtin_popcountll(b1) +
                 4 * __builtin_popcountll(b2);
          __builtin_amdgcn_sched_barrier(0);  // one group's masks live at a time
        }
        n_und = n_lo;
        sh = ts == mx ? 0 : 32 - __builtin_clz(ts ^ mx);
        T = sh == 32 ? 0u : (ts >> sh) << sh;
        staged = true;
        b_lo = ts;
        b_hi = mx;
      }
    }
  }
  if (!staged) {  // uniform
    // Before each bit the undecided keys are those in [T, T + 2^(bit+1));
    // n_ge counts keys >= T and n_top keys above the range.
    int parity = 0;
    int bit = 31;
    int n_ge = PTK_THREADS * KPT;
    for (; bit >= 0 && n_ge - n_top > UND; --bit) {  // uniform
      const uint32_t cand = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) cnt = add_ge(cnt, key[v][c], cand);
      cnt = ptk_block_sum<PTK_WAVES>((int)wave_sum((float)cnt), red, parity);  // exact: < 2^24
      parity ^= 1;
      if (cnt >= k) {
        T = cand;
        n_ge = cnt;
      } else {
        n_top = cnt;
      }
    }
    sh = bit + 1;
    if (sh > 0) {  // uniform
      // undecided: key in [T, T + 2^sh), T a multiple of 2^sh.  Branch-free:
      // out-of-range keys go to a per-lane dummy slot past UND.
      const uint32_t pre = sh == 32 ? 0u : (T >> sh);
      auto outside_p = [&](uint32_t kv, uint32_t p) -> uint32_t {  // 1 when kv is decided
        const uint32_t x = sh == 32 ? 0u : ((kv >> sh) ^ p);
        return (x | (0u - x)) >> 31;
      };
      int mine = 0;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) mine += 1 - (int)outside_p(key[v][c], pre);
      int at = ptk_block_exscan<PTK_WAVES>(mine, red[0], &n_und);
      const int dummy = UND + lane;
      // recomputed from an opaque copy of the prefix: not kept live across the scan
      uint32_t pre2 = pre;
      asm volatile("" : "+v"(pre2));
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t o = outside_p(key[v][c], pre2);
          const uint32_t m = 0u - o;  // all ones when decided
          und[((uint32_t)at & ~m) | ((uint32_t)dummy & m)] = key[v][c];
          at += 1 - (int)o;
        }
    }
  }
  // Staged keys, all in [bracket, row maximum]: T by value buckets first.
  // PTK_BUCKETS equal-width buckets over that range of the order keys (a key's bucket is a
  // monotone function of it: a subtraction, a conversion, a product and a
  // truncation), one histogram pass over the staged keys, a scan from the top
  // for the bucket holding the k-th largest key; when that bucket holds at
  // most PTK_RANK_MAX keys, T is the key of the remaining rank among them
  // (key descending, staged position ascending).  Otherwise the radix digits
  // below fix T.
  bool found = false;
  if (staged && sh > 0) {  // uniform
    const float bscale = (float)PTK_BUCKETS / ((float)(b_hi - b_lo) + 1.f);
    auto bucket_of = [&](uint32_t kv) {
      return min((int)((float)(kv - b_lo) * bscale), PTK_BUCKETS - 1);
    };
    for (int i = tid; i < PTK_BUCKETS; i += PTK_THREADS) bhist[i] = 0u;
    __syncthreads();
    for (int j = tid; j < n_und; j += PTK_THREADS) atomicAdd(&bhist[bucket_of(und[j])], 1u);
    __syncthreads();
    // thread t owns buckets top - PER t .. top - PER t - PER + 1 (descending)
    constexpr int PER = PTK_BUCKETS / PTK_THREADS;
    uint32_t c[PER];
    uint32_t own = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      c[j] = bhist[PTK_BUCKETS - 1 - (tid * PER + j)];
      own += c[j];
    }
    int tot;
    const uint32_t exc = (uint32_t)ptk_block_exscan<PTK_WAVES>((int)own, red[0], &tot);
    const uint32_t rem = (uint32_t)k;  // no key lies above the staged range here
    if (exc < rem && rem <= exc + own) {
      uint32_t acc = exc;
      for (int j = 0; j < PER; ++j) {
        if (acc + c[j] >= rem) {
          bk_sel = PTK_BUCKETS - 1 - (tid * PER + j);
          bk_above = acc;
          bk_cnt = (int)c[j];
          bk_n = 0;
          break;
        }
        acc += c[j];
      }
    }
    __syncthreads();
    const int tbk = bk_sel, cnt = bk_cnt;
    if (cnt <= PTK_RANK_MAX) {  // uniform
      for (int j = tid; j < n_und; j += PTK_THREADS) {
        const uint32_t kv = und[j];
        if (bucket_of(kv) == tbk) bcand[atomicAdd(&bk_n, 1)] = make_uint2(kv, (uint32_t)j);
      }
      __syncthreads();
      const uint32_t want = rem - bk_above - 1u;  // T's rank in the bucket, from 0
      for (int i = tid; i < cnt; i += PTK_THREADS) {
        const uint2 me = bcand[i];
        uint32_t rank = 0u;
        for (int o = 0; o < cnt; ++o) {
          const uint2 x = bcand[o];
          rank += (x.x > me.x || (x.x == me.x && x.y < me.y)) ? 1u : 0u;
        }
        if (rank == want) bk_T = me.x;
      }
      __syncthreads();
      T = bk_T;
      found = true;
    }
  }
  if (!found) {  // uniform
    for (int i = tid; i < 4 * 256; i += PTK_THREADS) (&dhist[0][0])[i] = 0u;
    __syncthreads();
    {
      // The open sh bits of T, in digits of up to 8 bits from the top: a
      // histogram of the digit over the staged keys that share T's bits above
      // it, then the digit whose bin reaches the remaining rank counting from
      // the top.  The histograms were cleared up front and every wave scans the
      // bins itself, so each digit costs one barrier.  Staged padding keys (0,
      // past E) lie below the k-th largest key, which is a real one.
      uint32_t remaining = (uint32_t)(k - n_top);  // rank of T among the staged keys
      int lo = sh;
      for (int p = 0; lo > 0; ++p) {  // uniform, at most 4 digits
        const int w = min(8, lo);
        lo -= w;
        const int hi = lo + w;  // bits [lo, hi) are this digit
        for (int j = tid; j < n_und; j += PTK_THREADS) {
          const uint32_t kv = und[j];
          const bool same = hi == 32 || ((kv ^ T) >> hi) == 0u;
          if (same) atomicAdd(&dhist[p][(kv >> lo) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        // lane l owns bins 255-4l .. 252-4l (descending order)
        uint32_t c4[4];
  #pragma unroll
        for (int e = 0; e < 4; ++e) c4[e] = dhist[p][255 - 4 * lane - e];
        const uint32_t own = c4[0] + c4[1] + c4[2] + c4[3];
        uint32_t inc = own;
  #pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t t = __shfl_up(inc, off);
          if (lane >= off) inc += t;
        }
        const uint32_t exc = inc - own;
        const bool here = exc < remaining && remaining <= inc;  // exactly one lane
        uint32_t dg = 0u, above = exc;
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool take = dg == 0u && above + c4[e] >= remaining;
          dg = take ? (uint32_t)(256 - 4 * lane - e) : dg;  // digit + 1
          above = (dg == 0u) ? above + c4[e] : above;
        }
        const int src = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(here));
        const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)dg, src) - 1u;
        remaining -= (uint32_t)__builtin_amdgcn_readlane((int)above, src);
        T |= d << lo;
      }
    }
  }
  if (staged) {  // uniform
    // The top k are the staged keys above T and the first k - #(> T) keys
    // equal to T in index order.  Thread t walks the staged entries
    // [t ch, (t + 1) ch), contiguous in index order; one workgroup scan of its
    // two counts (packed: each total is below 2^15) places its selections.
    const int ch = (n_und + PTK_THREADS - 1) / PTK_THREADS;
    const int e0 = min(tid * ch, n_und), e1 = min(e0 + ch, n_und);
    int ng = 0, nq = 0;
    for (int e = e0; e < e1; ++e) {
      const uint32_t kv = und[e];
      ng += kv > T ? 1 : 0;
      nq += kv == T ? 1 : 0;
    }
    int tot;
    const int pre = ptk_block_exscan<PTK_WAVES>(ng | (nq << 16), red[0], &tot);
    const int need_eq = k - (tot & 0xFFFF);  // >= 1 by the choice of T
    int qr = pre >> 16;
    int p = (pre & 0xFFFF) + min(qr, need_eq);
    for (int e = e0; e < e1; ++e) {
      const uint32_t kv = und[e];
      const bool eq = kv == T;
      if ((kv > T || (eq && qr < need_eq)) && p < k) out[p++] = (int32_t)und_idx[e];
      qr += eq ? 1 : 0;
    }
    return;
  }
  // per-wave counts above and equal to T, prefixes over the waves
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      n_gt = add_ge(n_gt, key[v][c], T + 1);  // T < 2^32 - 1: keys are finite floats
      n_eq = add_ge(n_eq, key[v][c], T);
    }
  n_eq -= n_gt;  // counted >= T above
  n_gt = (int)wave_sum((float)n_gt);
  n_eq = (int)wave_sum((float)n_eq);
  if (lane == 0) {
    wcnt[0][wave] = n_gt;
    wcnt[1][wave] = n_eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0, tot_gt = 0, tot_eq = 0;
#pragma unroll
  for (int w = 0; w < PTK_WAVES; ++w) {
    const int cg = wcnt[0][w], ce = wcnt[1][w];
    tot_gt += cg;
    tot_eq += ce;
    gt_before += w < wave ? cg : 0;
    eq_before += w < wave ? ce : 0;
  }
  const int need_eq = k - tot_gt;  // >= 1 by the choice of T
  // entry indices from an opaque copy of the lane id: computed here instead of
  // being kept live from the loads on
  int ln = lane;
  asm volatile("" : "+v"(ln));
  // (not in the 1024-thread variant, whose 128 keys per thread already exceed
  // its registers)
  if (PTK_THREADS <= 512 && tot_eq == need_eq) {  // uniform: every key equal to T is taken
    // Per group of 256 keys, the lane's count (0..4) as three ballots of its
    // bits: the lane's position is their weighted mbcnt, the group total their
    // weighted popcount.  The indices are staged in LDS (und is free: its last
    // reads precede the barriers since) and written out as whole rows.
    int pos = gt_before + eq_before;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      int ns = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) ns += key[v][c] >= T ? 1 : 0;
      const uint64_t b0 = __builtin_amdgcn_ballot_w64((ns & 1) != 0);
      const uint64_t b1 = __builtin_amdgcn_ballot_w64((ns & 2) != 0);
      const uint64_t b2 = __builtin_amdgcn_ballot_w64((ns & 4) != 0);
      int p = pos + (int)(lane_prefix(b0) + 2 * lane_prefix(b1) + 4 * lane_prefix(b2));
      const int j = wbase + 256 * v + 4 * ln;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (key[v][c] >= T) und[p++] = (uint32_t)(j + c);
      pos += __builtin_popcountll(b0) + 2 * __builtin_popcountll(b1) + 4 * __builtin_popcountll(b2);
    }
    __syncthreads();
    for (int i = tid; i < k; i += PTK_THREADS) out[i] = (int32_t)und[i];
    return;
  }
  // ties at T: the first need_eq equal keys in index order are taken
  int pos = gt_before + min(eq_before, need_eq);  // selected keys of the earlier waves
  int eq_rank = eq_before;                        // equal keys before this group
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    // keys of group v in index order: lane-major, then c
    int ne = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) ne += key[v][c] == T ? 1 : 0;
    int eq_cnt;
    const int eq_pre = wave_exscan(ne, &eq_cnt);
    bool t[4];
    int own = 0, ns = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool e = key[v][c] == T;
      t[c] = key[v][c] > T || (e && eq_rank + eq_pre + own < need_eq);
      own += e ? 1 : 0;
      ns += t[c] ? 1 : 0;
    }
    int sel_cnt;
    int p = pos + wave_exscan(ns, &sel_cnt);
    const int j = wbase + 256 * v + 4 * ln;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (t[c]) out[p++] = j + c;
    pos += sel_cnt;
    eq_rank += eq_cnt;
  }
}

// ---------------------------------------------------------------------------
// attention over the three branches.
constexpr int PF_CH = 64;         // entries per chunk
constexpr int PF_MAX_SEL = PREFILL_MAX_SEL;  // branch-A entries per (tile, kv head) kept in LDS

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
  const float* sink;     // [Hq] sink logits (natural log) or null
  int B, C, Hq, Hkv, P, stride, E4, E128, ksel, window, q_tile, n_tiles;
  int combine;           // 0: average of the branches, 1: one softmax over all of them
  float scale_log2;
};

// Piece of an entry row handled by one thread: 8 bytes (512 threads) or 16.
template <int PB> struct PieceT;
template <> struct PieceT<8> { using type = uint2; };
template <> struct PieceT<16> { using type = uint4; };
__device__ __forceinline__ uint32_t piece_word(const uint2& p, int i) { return i == 0 ? p.x : p.y; }
__device__ __forceinline__ uint32_t piece_word(const uint4& p, int i) {
  return i == 0 ? p.x : (i == 1 ? p.y : (i == 2 ? p.z : p.w));
}

// V^T rows hold 64 fp16 entries as 16 groups of 4 (8 bytes); group G of dim
// row d sits at slot G ^ vt_swz(d).  vt_swz is a bijection on any 16
// consecutive dims (the PV operand reads) and on the dims x + 4m and x + 8m,
// m < 16 (the stores of one instruction), so neither pattern repeats a slot
// within 16 lanes.
__device__ __forceinline__ int vt_swz(int dim) { return (dim & 15) ^ ((dim >> 4) & 7); }


// One workgroup per (b, tile, kv head): NW waves of 16*NT (query, head) rows.
// Per chunk of 64 entries: S^T = K Q^T (bf16 MFMA, Q fragments in registers),
// online softmax in base 2 with the row maximum raised only when it grows by
// more than 2^8 (exact: the weights and their sum share the stale maximum),
// P in fp16, O += P V (fp16 MFMA, V^T staged in LDS).  At the end of a branch
// the normalised rows are added into a partial sum in LDS (fp16, each lane's
// own values), which the last branch folds into `out` with one write.
template <int NW, int NT>
__global__ __launch_bounds__(NW * 64, 1) void prefill_attn_kernel(PrefillAttnArgs a) {
  constexpr int D = 128, KS = D / 32, NTH = NW * 64;
  constexpr int RW = 16 * NT;          // (query, head) rows per wave
  constexpr int PB = 4096 / NTH;       // bytes of each of its 4 entry rows a thread moves per chunk
  constexpr int LPR = 256 / PB;        // threads per entry row
  constexpr int NDT = PB / 2;          // dims per thread per entry
  using Piece = typename PieceT<PB>::type;
  static_assert(PF_CH == 64 && NTH / LPR == 16, "16 groups of 4 entries per chunk");
  __shared__ __align__(16) uint4 k_lds[2][PF_CH * (D / 8)];      // entry rows, 16 B pieces, xor-swizzled
  __shared__ __align__(16) uint16_t vt_lds[2][D * PF_CH];        // V^T fp16 [dim][entry], 8 B groups swizzled
  __shared__ __align__(16) float xch[NW][3][RW];  // alpha, row max, running concat lse
  __shared__ __align__(16) uint32_t sel_lds[PF_MAX_SEL];         // the tile's branch-A row offsets
  // the output's partial sum over the branches done so far, fp16, in each
  // lane's own accumulator layout [wave][nt][nd][lane] x 4 rows: only that
  // lane reads it back, so no barrier; out is written once, at the last branch
  __shared__ __align__(16) uint2 part_lds[NW][NT][D / 16][64];

  const int g = a.Hq / a.Hkv;
  const int prob = blockIdx.x;
  const int b = prob / (a.n_tiles * a.Hkv), tile = (prob / a.Hkv) % a.n_tiles, kvh = prob % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  const int64_t pair = (int64_t)b * a.Hkv + kvh;

  // Q^T fragments (B operand of S^T): lane l holds row RW*wave + 16nt + l%16,
  // dims 32ks + 8(l/16) .. +8.  Row r = query r / g of the tile, head r % g.
  uint4 qf[NT][KS];
  int qpos[NT];  // absolute position of the row's query (for the window mask)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = RW * wave + 16 * nt + l16;
    const int i = min(tile * a.q_tile + r / g, a.C - 1);
    const uint4* qp =
        reinterpret_cast<const uint4*>(a.q + (((int64_t)b * a.C + i) * a.Hq + kvh * g + r % g) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nt][ks] = qp[4 * ks + j4];
    qpos[nt] = a.P + tile * a.q_tile + r / g;
  }

  // chunk schedule: branch A (selected entries), B (all dense entries), C (window)
  const int nA = (a.ksel + PF_CH - 1) / PF_CH;
  const int nB = (a.E128 + PF_CH - 1) / PF_CH;
  const int T0 = max(0, a.P + tile * a.q_tile - a.window + 1);
  const int T1 = min(a.P + a.C, a.P + tile * a.q_tile + a.q_tile);
  const int nC = (T1 - T0 + PF_CH - 1) / PF_CH;
  const int total = nA + nB + nC;
  // rows are addressed as a uniform base (the pair's stream; for the window,
  // its first token) plus a 32-bit byte offset: every stream a pair reads
  // spans less than 4 GiB, and the loads take the offset in one VGPR
  constexpr uint32_t RB = D * 2;  // bytes per entry row
  const int eg = tid / LPR, pc = tid % LPR;
  const uint32_t pcb = (uint32_t)(PB * pc);  // the thread's piece within a row
  {
    // the tile's branch-A entries as row offsets, padded to whole chunks with
    // the last entry; clamped: a caller's out-of-range index never leaves the stream
    const int32_t* sel = a.sel + ((int64_t)(b * a.n_tiles + tile) * a.Hkv + kvh) * a.ksel;
    for (int j = tid; j < nA * PF_CH; j += NTH)
      sel_lds[j] = (uint32_t)min(max(sel[min(j, a.ksel - 1)], 0), a.E4 - 1) * RB;
  }
  __syncthreads();
  const char* const kA = reinterpret_cast<const char*>(a.k4 + pair * a.E4 * D);
  const char* const vA = reinterpret_cast<const char*>(a.v4 + pair * a.E4 * D);
  const char* const kB = reinterpret_cast<const char*>(a.k128 + pair * a.E128 * D);
  const char* const vB = reinterpret_cast<const char*>(a.v128 + pair * a.E128 * D);
  const char* const kC = reinterpret_cast<const char*>(a.k + (pair * a.stride + T0) * D);
  const char* const vC = reinterpret_cast<const char*>(a.v + (pair * a.stride + T0) * D);
  const uint32_t lastB = (uint32_t)(a.E128 - 1) * RB + pcb, lastC = (uint32_t)(T1 - T0 - 1) * RB + pcb;

  // global -> registers two chunks ahead (two register sets), stored to LDS
  // after the compute of the chunk before it.  Thread t moves bytes
  // [PB*(t % LPR), +PB) of the four consecutive entries 4*(t / LPR) + u: one
  // load instruction reads whole rows.
  Piece kreg[2][4], vreg[2][4];
  auto load_chunk = [&](int set, int gc) {
    const char *kb, *vb;
    uint32_t off[4];
    if (gc < nA) {  // uniform
      const uint4 o = *reinterpret_cast<const uint4*>(&sel_lds[gc * PF_CH + 4 * eg]);
      off[0] = o.x + pcb;
      off[1] = o.y + pcb;
      off[2] = o.z + pcb;
      off[3] = o.w + pcb;
      kb = kA;
      vb = vA;
    } else if (gc < nA + nB) {
      const uint32_t r0 = (uint32_t)((gc - nA) * PF_CH + 4 * eg) * RB + pcb;
#pragma unroll
      for (int u = 0; u < 4; ++u) off[u] = min(r0 + u * RB, lastB);
      kb = kB;
      vb = vB;
    } else {
      const uint32_t r0 = (uint32_t)((gc - nA - nB) * PF_CH + 4 * eg) * RB + pcb;
#pragma unroll
      for (int u = 0; u < 4; ++u) off[u] = min(r0 + u * RB, lastC);
      kb = kC;
      vb = vC;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kreg[set][u] = ld_stream(reinterpret_cast<const Piece*>(kb + off[u]));
      vreg[set][u] = ld_stream(reinterpret_cast<const Piece*>(vb + off[u]));
    }
  };
  auto store_chunk = [&](int set, int buf) {
    const int p16 = (pc * PB) / 16, sub = ((pc * PB) % 16) / PB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * eg + u;
      reinterpret_cast<Piece*>(&k_lds[buf][e * (D / 8) + (p16 ^ (e & 15))])[sub] = kreg[set][u];
    }
    uint2* vt = reinterpret_cast<uint2*>(vt_lds[buf]);
#pragma unroll
    for (int x = 0; x < NDT; ++x) {
      _Float16 h[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w = piece_word(vreg[set][u], x >> 1);
        h[u] = (_Float16)((x & 1) ? bf_hi(w) : bf_lo(w));
      }
      const int dim = NDT * pc + x;
      vt[dim * (PF_CH / 4) + (eg ^ vt_swz(dim))] =
          make_uint2(__builtin_bit_cast(uint32_t, (f16x2_t){h[0], h[1]}),
                     __builtin_bit_cast(uint32_t, (f16x2_t){h[2], h[3]}));
    }
  };

  f32x4_t O[NT][D / 16];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int nd = 0; nd < D / 16; ++nd) O[nt][nd] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  // running maximum per row (lane l%16 of the S layout) and row sums of the
  // weights in the O layout (rows 4(l/16) + i): the sums come from the
  // matrix cores as P times a B operand of ones
  float m_run[NT];
  f32x4_t Lc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    Lc[nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }
  const f16x8_t ones = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  const float c = a.scale_log2;

  auto chunk = [&](int gc, int set) {  // set == gc & 1
    const int buf = set;
    // unconditional (the last chunk again past the end) so that the wait
    // before each store counts exactly the newer set's loads
    load_chunk(set, min(gc + 2, total - 1));
    // what this chunk holds
    const int br = gc < nA ? 0 : (gc < nA + nB ? 1 : 2);
    const int nvalid = br == 0 ? min(PF_CH, a.ksel - gc * PF_CH)
                               : (br == 1 ? min(PF_CH, a.E128 - (gc - nA) * PF_CH)
                                          : min(PF_CH, T1 - T0 - (gc - nA - nB) * PF_CH));
    const int tbase = T0 + (gc - nA - nB) * PF_CH;  // branch C: token of entry 0
    const bool masked = br == 2 || nvalid < PF_CH;   // uniform
    // S^T = K Q^T : lane gets entries 16mt + 4(l/16) + i of row 16nt + l%16
    // K fragments of entry tile mt + 1 are read while the MFMAs of tile mt run
    f32x4_t s[NT][4];
    uint4 ka[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[0][ks] = k_lds[buf][l16 * (D / 8) + ((4 * ks + j4) ^ l16)];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt + 1 < 4) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[(mt + 1) & 1][ks] = k_lds[buf][(16 * (mt + 1) + l16) * (D / 8) + ((4 * ks + j4) ^ l16)];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka[mt & 1][ks]),
                                                        __builtin_bit_cast(bf16x8_t, qf[nt][ks]),
                                                        acc, 0, 0, 0);
        s[nt][mt] = acc;
      }
      __builtin_amdgcn_sched_barrier(0);  // bound the hoisted fragment reads
    }
    if (masked) {
      // valid entries of row 16nt + l%16 are e in [lo, hi]
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        int lo = 0, hi = nvalid - 1;
        if (br == 2) {
          lo = max(lo, qpos[nt] - a.window + 1 - tbase);
          hi = min(hi, qpos[nt] - tbase);
        }
        const uint32_t span = (uint32_t)(hi - lo);  // huge when hi < lo: nothing valid
        const int d0 = 4 * j4 - lo;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = hi >= lo && (uint32_t)(d0 + 16 * mt + i) <= span;
            s[nt][mt][i] = ok ? s[nt][mt][i] : -INFINITY;
          }
      }
    }
    // row maxima of the chunk (scaled to base 2); raise the running maximum
    // only where it grows by more than 8
    float mc[NT];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmax_nc(mx, s[nt][mt][i]);
      mx = pair32_max(pair16_max(mx));
      mc[nt] = mx * c;
      grow = grow || (mc[nt] > m_run[nt] + 8.f);
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // uniform
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float m_new = fmax_nc(m_run[nt], mc[nt]);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new);
        m_run[nt] = m_new;
        if (j4 == 0) xch[wave][0][16 * nt + l16] = alpha;
      }
      wave_lds_sync();
      // rescale O rows and their sums (lane holds rows 16nt + 4(l/16) + i)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 al = *reinterpret_cast<const float4*>(&xch[wave][0][16 * nt + 4 * j4]);
        Lc[nt][0] *= al.x;
        Lc[nt][1] *= al.y;
        Lc[nt][2] *= al.z;
        Lc[nt][3] *= al.w;
#pragma unroll
        for (int nd = 0; nd < D / 16; ++nd) {
          O[nt][nd][0] *= al.x;
          O[nt][nd][1] *= al.y;
          O[nt][nd][2] *= al.z;
          O[nt][nd][3] *= al.w;
        }
      }
    }
    // P = 2^(s c - m) in fp16 as the A operand of P V
    f16x8_t pa[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float neg_m = m_run[nt] == -INFINITY ? 0.f : -m_run[nt];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pa[nt][mt >> 1][4 * (mt & 1) + i] =
              (_Float16)__builtin_amdgcn_exp2f(fmaf(s[nt][mt][i], c, neg_m));
    }
    // row sums of the fp16 weights (the ones PV multiplies)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        Lc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[nt][kk], ones, Lc[nt], 0, 0, 0);
    // O += P V: B operand lane l = dim 16nd + l%16, entries of the P k-slots;
    // the fragments of column tile nd + 1 are read while the MFMAs of nd run
    auto vfrag = [&](int nd, int kk) {
      const int dim = 16 * nd + l16;
      const uint2* vrow = reinterpret_cast<const uint2*>(&vt_lds[buf][dim * PF_CH]);
      const int sw = vt_swz(dim);
      const uint2 lo = vrow[(8 * kk + j4) ^ sw];
      const uint2 hi = vrow[(8 * kk + 4 + j4) ^ sw];
      return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    uint4 vf[2][2];
    vf[0][0] = vfrag(0, 0);
    vf[0][1] = vfrag(0, 1);
#pragma unroll
    for (int nd = 0; nd < D / 16; ++nd) {
      if (nd + 1 < D / 16) {
        vf[(nd + 1) & 1][0] = vfrag(nd + 1, 0);
        vf[(nd + 1) & 1][1] = vfrag(nd + 1, 1);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8_t vb = __builtin_bit_cast(f16x8_t, vf[nd & 1][kk]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          O[nt][nd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[nt][kk], vb, O[nt][nd], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // end of a branch: normalise, fold into the LDS partial sum (A writes it, B
    // adds, C adds and writes out), reset
    const bool last = (gc == nA - 1) || (gc == nA + nB - 1) || (gc == total - 1);
    if (last) {
      // end of a branch: per-row sum l and lse = (m + log2 l) ln 2, then the
      // branch output O / l is folded into the sum (sum = ca sum + cb O / l):
      //   average:  sum = (o_A k_A + o_B k_B + o_C k_C) / 3, k = 1 without a sink
      //             logit z, else 1 / (1 + e^(z - lse)) (the sink joins each softmax);
      //   concat:   one softmax over all branches' logits: the sum accumulates
      //             e^(lse_X - L) o_X with the running L = log sum e^lse_X kept
      //             in LDS per row; the sink logit scales by 1 / (1 + e^(z - L)).
      // The partial sums stay within the values' range, so fp16 holds them
      // (rounding each by at most 2^-11 relative).
      // the row maxima move to the O layout through LDS
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (j4 == 0) xch[wave][1][16 * nt + l16] = m_run[nt];
      wave_lds_sync();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // row addresses from an opaque copy of the lane id: computed here
        // rather than kept live across the chunk loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int jo = ln >> 4;
        const float4 m4 = *reinterpret_cast<const float4*>(&xch[wave][1][16 * nt + 4 * jo]);
        const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
        float lv[4], lse[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lv[i] = Lc[nt][i];
          lse[i] = (mv[i] + log2f(lv[i])) * PF_LN2;
        }
        float ca[4], cb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = RW * wave + 16 * nt + 4 * jo + i;
          const int qi = tile * a.q_tile + r / g;
          const int h = kvh * g + r % g;
          if (a.lse3 && qi < a.C && (ln & 15) == 0)
            a.lse3[(((int64_t)br * a.B + b) * a.C + qi) * a.Hq + h] = lse[i];
          // coefficients: sum = ca * sum + cb * (O / l)
          ca[i] = 0.f;
          cb[i] = 1.f;
          if (a.combine == 0) {  // uniform
            // the sum holds (k_A o_A + k_B o_B) / 3 so far: |sum| <= 2/3 max |v|
            if (a.sink) cb[i] = 1.f / (1.f + __expf(a.sink[h] - lse[i]));
            cb[i] *= 1.f / 3.f;
            ca[i] = br == 0 ? 0.f : 1.f;
          } else {
            float* Lp = &xch[wave][2][16 * nt + 4 * jo + i];
            float L = lse[i];
            if (br > 0) {
              const float Lo = *Lp, mx = fmaxf(Lo, lse[i]);
              L = mx + __logf(__expf(Lo - mx) + __expf(lse[i] - mx));
              ca[i] = __expf(Lo - L);
              cb[i] = __expf(lse[i] - L);
            }
            if ((ln & 15) == 0) *Lp = L;
            if (br == 2 && a.sink) {
              const float keep = 1.f / (1.f + __expf(a.sink[h] - L));
              ca[i] *= keep;
              cb[i] *= keep;
            }
          }
          cb[i] *= __builtin_amdgcn_rcpf(lv[i]);
        }
        const int r0 = RW * wave + 16 * nt + 4 * jo;
#pragma unroll
        for (int nd = 0; nd < D / 16; ++nd) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = O[nt][nd][i] * cb[i];
          uint2* pp = &part_lds[wave][nt][nd][ln];
          if (br > 0) {  // uniform
            const uint2 w = *pp;
            const f16x2_t p01 = __builtin_bit_cast(f16x2_t, w.x), p23 = __builtin_bit_cast(f16x2_t, w.y);
            v[0] = fmaf((float)p01[0], ca[0], v[0]);
            v[1] = fmaf((float)p01[1], ca[1], v[1]);
            v[2] = fmaf((float)p23[0], ca[2], v[2]);
            v[3] = fmaf((float)p23[1], ca[3], v[3]);
          }
          if (br < 2) {  // uniform
            *pp = make_uint2(__builtin_bit_cast(uint32_t, (f16x2_t){(_Float16)v[0], (_Float16)v[1]}),
                             __builtin_bit_cast(uint32_t, (f16x2_t){(_Float16)v[2], (_Float16)v[3]}));
          } else {
            // the last branch: out is written once; rows past the chunk's end
            // belong to no query
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = r0 + i;
              const int qi = tile * a.q_tile + r / g;
              const int h = kvh * g + r % g;
              if (qi < a.C)
                a.out[(((int64_t)b * a.C + qi) * a.Hq + h) * D + 16 * nd + (ln & 15)] = v[i];
            }
          }
        }
#pragma unroll
        for (int nd = 0; nd < D / 16; ++nd) O[nt][nd] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        m_run[nt] = -INFINITY;
        Lc[nt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      }
    }
    // the other buffer was last read in chunk gc - 1, which every wave
    // finished before the barrier that ended it
    if (gc + 1 < total) store_chunk(set ^ 1, buf ^ 1);
    __syncthreads();
  };
  load_chunk(0, 0);
  if (total > 1) load_chunk(1, 1);
  store_chunk(0, 0);
  __syncthreads();
  for (int gc = 0; gc < total; gc += 2) {
    chunk(gc, 0);
    if (gc + 1 < total) chunk(gc + 1, 1);
  }
}

// ---------------------------------------------------------------------------
size_t prefill_workspace_bytes(int B, int Hkv, int D, int n_tiles, int E4, int ksel, bool need_sel) {  // R2 scratch (+ sel)
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t s = al((size_t)B * n_tiles * Hkv * D * 4);           // qbar
  s += al((size_t)B * Hkv * n_tiles * (size_t)((E4 + 3) & ~3) * 4);  // scores, rows padded to 4
  if (need_sel) s += al((size_t)B * n_tiles * Hkv * (size_t)ksel * 4);
  return s;
}

// keys per thread for 512 threads (up to 128 keys: 65536 entries), else 1024
int prefill_topk_kpt(int E4, int* threads) {
  *threads = E4 > 512 * 128 ? 1024 : 512;
  int kpt = 4;  // multiple of 4: one float4 per lane per group
  while (kpt * *threads < E4) kpt *= 2;
  return kpt;
}

// R2: pooled tile queries, scores against the bf16 keys (or the fp32 stream),
// top-k -> sel
bool launch_prefill_select(const PrefillLaunch& L, int32_t* sel, hipStream_t st) {
  const int D = 128;
  if (L.n_tiles > PSC_MAX_TILES) return false;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* ws = static_cast<char*>(L.workspace);
  float* qbar = reinterpret_cast<float*>(ws);
  ws += al((size_t)L.B * L.n_tiles * L.Hkv * D * 4);
  float* scores = reinterpret_cast<float*>(ws);
  const int Es = (L.E4 + 3) & ~3;
  const unsigned probs = (unsigned)(L.B * L.n_tiles * L.Hkv);
  prefill_qbar_kernel<<<probs, 256, 0, st>>>(L.q, L.C, L.Hq, L.Hkv, L.q_tile, L.n_tiles, qbar);
  const int ntb = (L.n_tiles + 15) / 16;
  if (L.indexer_f32) {
    dim3 sg((L.E4 + 64 * PSC_GROUPS - 1) / (64 * PSC_GROUPS), L.Hkv, L.B);
    switch (ntb) {
      case 1: prefill_scores_kernel<128, 1><<<sg, 256, 0, st>>>(L.k4f, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      case 2: prefill_scores_kernel<128, 2><<<sg, 256, 0, st>>>(L.k4f, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      case 3: prefill_scores_kernel<128, 3><<<sg, 256, 0, st>>>(L.k4f, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      case 4: prefill_scores_kernel<128, 4><<<sg, 256, 0, st>>>(L.k4f, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      default: return false;
    }
  } else {
    dim3 sg((L.E4 + 64 * PSB_GROUPS - 1) / (64 * PSB_GROUPS), L.Hkv, L.B);
    switch (ntb) {
      case 1: prefill_scores_bf16_kernel<128, 1><<<sg, 256, 0, st>>>(L.k4b, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      case 2: prefill_scores_bf16_kernel<128, 2><<<sg, 256, 0, st>>>(L.k4b, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      case 3: prefill_scores_bf16_kernel<128, 3><<<sg, 256, 0, st>>>(L.k4b, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      case 4: prefill_scores_bf16_kernel<128, 4><<<sg, 256, 0, st>>>(L.k4b, qbar, L.n_tiles, L.Hkv, L.E4, Es, scores); break;
      default: return false;
    }
  }
  int nthr;
  const int kpt = prefill_topk_kpt(L.E4, &nthr);
#define BSA_PTK(KK, NT)                                                                         \
  if (kpt == KK && nthr == NT) {                                                                \
    prefill_topk_kernel<KK, NT><<<probs, NT, 0, st>>>(scores, L.n_tiles, L.Hkv, L.E4, Es, L.ksel, \
                                                      sel);                                     \
    return true;                                                                                \
  }
  BSA_PTK(4, 512) BSA_PTK(8, 512) BSA_PTK(16, 512) BSA_PTK(32, 512) BSA_PTK(64, 512)
  BSA_PTK(128, 512) BSA_PTK(128, 1024)
#undef BSA_PTK
  return false;
}

// R3-R6: the three branches over a given selection, averaged into out
bool launch_prefill_attend(const PrefillLaunch& L, const int32_t* sel, hipStream_t st) {
  const int g = L.Hq / L.Hkv;
  const unsigned probs = (unsigned)(L.B * L.n_tiles * L.Hkv);
  PrefillAttnArgs a;
  a.q = L.q; a.k = L.k; a.v = L.v; a.k4 = L.k4b; a.v4 = L.v4b; a.k128 = L.k128b; a.v128 = L.v128b;
  a.sel = sel; a.out = L.out; a.lse3 = L.lse3; a.sink = L.sink; a.combine = L.combine;
  a.B = L.B; a.C = L.C; a.Hq = L.Hq; a.Hkv = L.Hkv; a.P = L.P; a.stride = L.stride;
  a.E4 = L.E4; a.E128 = L.E128; a.ksel = L.ksel; a.window = L.window; a.q_tile = L.q_tile;
  a.n_tiles = L.n_tiles; a.scale_log2 = L.scale * PF_LOG2E;
  // one workgroup per (b, tile, kv head); 16 rows per MFMA tile, NT tiles per wave
  switch (L.q_tile * g) {
    case 64: prefill_attn_kernel<4, 1><<<probs, 256, 0, st>>>(a); break;
    case 128: prefill_attn_kernel<4, 2><<<probs, 256, 0, st>>>(a); break;
    case 256: prefill_attn_kernel<8, 2><<<probs, 512, 0, st>>>(a); break;
    default: return false;
  }
  return true;
}

}  // namespace bsa
