// kernels_select.hip -- block summaries, block scoring and top-k selection.
//
// Block summaries are the per-block means of the key rows (blocks of 64
// tokens as the unit of importance evaluation: hotdry.top post
// "claude-opus-long-context-kv-cache-sparse-attention", section
// 稀疏注意力与 KV Cache 压缩的工程实现; mean pooling per "CSA + HCA
// 混合注意力机制" §4.1).  Scoring and top-k follow §4.4 steps 1-3 of that
// page: every block gets a score, the highest-scoring ones are kept.
#include <type_traits>

#include "bsa_device.h"
#include "bsa_launch.h"
#include "topk_device.h"

namespace bsa {

// ---------------------------------------------------------------------------
// Summaries.  One thread owns 8 consecutive columns of one block and walks
// its rows in token order, so each 16-lane row group of a wave reads one
// contiguous 256-byte key row per load.  HBM-bound: every key byte is read
// once, the output is 2*(d*4)/(bs*d*2) of the input for bs=64.
template <int D>
__global__ __launch_bounds__(256) void summaries_kernel(const uint16_t* __restrict__ x,
                                                        int64_t items, int N, int stride, int bs,
                                                        int j0, int nbr, int ostride,
                                                        float* __restrict__ out_f32,
                                                        uint16_t* __restrict__ out_bf16) {
  constexpr int TPR = D / 8;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t item = gid / TPR;
  const int part = (int)(gid % TPR);
  if (item >= items) return;
  const int64_t pair = item / nbr;          // nbr blocks [j0, j0 + nbr) per pair
  const int j = j0 + (int)(item % nbr);
  const int t0 = j * bs;
  const int n = min(bs, N - t0);
  const uint4* src = reinterpret_cast<const uint4*>(x + ((int64_t)pair * stride + t0) * D) + part;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  int t = 0;
  for (; t + 8 <= n; t += 8) {
    uint4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = ld_stream(src + (int64_t)(t + u) * TPR);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float f[8];
      unpack8(w[u], f);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] += f[c];
    }
  }
  for (; t < n; ++t) {
    float f[8];
    unpack8(ld_stream(src + (int64_t)t * TPR), f);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += f[c];
  }
  const float fn = (float)n;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = acc[c] / fn;
  const int64_t o = (pair * ostride + j) * D + part * 8;
  if (out_f32) {
    float4* dst = reinterpret_cast<float4*>(out_f32 + o);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (out_bf16) {
    uint4 w;
    w.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    w.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    w.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    w.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out_bf16 + o) = w;
  }
}

void launch_summaries(const uint16_t* x, int64_t pairs, int N, int stride, int d, int bs,
                      int j0, int ostride, float* out_f32, uint16_t* out_bf16, hipStream_t st) {
  const int nb = (N + bs - 1) / bs;
  const int nbr = nb - j0;
  if (nbr <= 0) return;
  const int64_t items = pairs * nbr;
  const int64_t threads = items * (d / 8);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (d == 128)
    summaries_kernel<128><<<grid, 256, 0, st>>>(x, items, N, stride, bs, j0, nbr, ostride,
                                                out_f32, out_bf16);
  else
    summaries_kernel<64><<<grid, 256, 0, st>>>(x, items, N, stride, bs, j0, nbr, ostride,
                                               out_f32, out_bf16);
}

// K/V rows of n_new tokens appended at position N of each (b, kv head)
__global__ __launch_bounds__(256) void append_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, int64_t pieces,
                                                     int n_new, int N, int stride, int ppr) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= pieces) return;
  const int64_t row = i / ppr;  // [pair][n_new] rows of ppr 16-byte pieces
  const int part = (int)(i % ppr);
  const int64_t pair = row / n_new;
  const int t = (int)(row % n_new);
  dst[(pair * stride + N + t) * ppr + part] = src[i];
}

// Append + summary refresh in one launch: one workgroup per (pair, block
// holding new tokens).  It writes the block's new K and V rows, stages the
// block's key rows in LDS (new rows from the source, older ones from the
// cache), then one thread per column adds them in token order and divides by
// the count: the same fp32 operations, in the same order, as summaries_kernel,
// so the result is bit-identical to a rebuild.
template <int D>
__global__ __launch_bounds__(256) void append_update_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, int n_new, int N, int stride,
    int bs, int j_first, int n_blk, int ostride, float* __restrict__ out_f32,
    uint16_t* __restrict__ out_bf16) {
  constexpr int PPR = D / 8;  // 16-byte pieces per row
  __shared__ uint16_t rows[APPEND_MAX_BS][D];
  const int64_t pair = blockIdx.x / n_blk;
  const int j = j_first + (int)(blockIdx.x % n_blk);
  const int t0 = j * bs, t1 = min(t0 + bs, N + n_new);  // the block's tokens after the append
  const int n = t1 - t0;
  const uint4* ksrc = reinterpret_cast<const uint4*>(k_new) + pair * n_new * PPR;
  const uint4* vsrc = reinterpret_cast<const uint4*>(v_new) + pair * n_new * PPR;
  uint4* kdst = reinterpret_cast<uint4*>(k_cache) + pair * stride * PPR;
  uint4* vdst = reinterpret_cast<uint4*>(v_cache) + pair * stride * PPR;
  for (int i = threadIdx.x; i < n * PPR; i += 256) {
    const int t = t0 + i / PPR, part = i % PPR;
    uint4 kv;
    if (t >= N) {  // a new token: write it and stage it from the source
      const int64_t si = (int64_t)(t - N) * PPR + part;
      kv = ksrc[si];
      kdst[(int64_t)t * PPR + part] = kv;
      vdst[(int64_t)t * PPR + part] = vsrc[si];
    } else {
      kv = kdst[(int64_t)t * PPR + part];
    }
    reinterpret_cast<uint4*>(rows[t - t0])[part] = kv;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float acc = 0.f;
    for (int t = 0; t < n; ++t) acc += __uint_as_float((uint32_t)rows[t][c] << 16);
    acc = acc / (float)n;
    const int64_t o = (pair * ostride + j) * D + c;
    if (out_f32) out_f32[o] = acc;
    if (out_bf16) out_bf16[o] = (uint16_t)bf16_rne(acc);
  }
}

void launch_append_update(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                          uint16_t* v_cache, int64_t pairs, int n_new, int N, int stride, int d,
                          int bs, int ostride, float* out_f32, uint16_t* out_bf16,
                          hipStream_t st) {
  if (n_new <= 0 || pairs <= 0) return;
  const int j_first = N / bs, j_last = (N + n_new - 1) / bs;
  const int n_blk = j_last - j_first + 1;
  const unsigned grid = (unsigned)(pairs * n_blk);
  if (d == 128)
    append_update_kernel<128><<<grid, 256, 0, st>>>(k_new, v_new, k_cache, v_cache, n_new, N,
                                                    stride, bs, j_first, n_blk, ostride, out_f32,
                                                    out_bf16);
  else
    append_update_kernel<64><<<grid, 256, 0, st>>>(k_new, v_new, k_cache, v_cache, n_new, N,
                                                   stride, bs, j_first, n_blk, ostride, out_f32,
                                                   out_bf16);
}

// FP8 (OCP E4M3) quantization of a K or V cache, one scale per (pair, block):
// amax = max |x| over the block's valid tokens, scale = amax / 448 and
// inv = 448 / amax (fp32, correctly rounded), code = RNE_E4M3(clamp(x * inv,
// +-448)) by v_cvt_pk_fp8_f32; an all-zero block gets scale 0 and zero codes.
template <int D>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ x,
                                                           uint8_t* __restrict__ out,
                                                           float* __restrict__ scales, int N,
                                                           int stride, int bs, int nb,
                                                           int sstride) {
  constexpr int PPR = D / 8;  // 8-value pieces per row
  __shared__ float red[4];
  const int64_t pair = blockIdx.x / nb;
  const int j = blockIdx.x % nb;
  const int t0 = j * bs, n = min(bs, N - t0);
  const uint4* src = reinterpret_cast<const uint4*>(x + (pair * stride + t0) * D);
  uint32_t amax_bits = 0;  // |bf16| bit patterns order like the values
  for (int i = threadIdx.x; i < n * PPR; i += 256) {
    const uint4 w = src[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      amax_bits = max(amax_bits, max(ws[c] & 0x7FFFu, (ws[c] >> 16) & 0x7FFFu));
  }
  float amax = __uint_as_float(amax_bits << 16);
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  if (threadIdx.x == 0) scales[pair * sstride + j] = amax / 448.f;
  uint2* dst = reinterpret_cast<uint2*>(out + (pair * stride + t0) * D);
  for (int i = threadIdx.x; i < n * PPR; i += 256) {
    const uint4 w = src[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float y[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      y[2 * c] = fminf(fmaxf(bf_lo(ws[c]) * inv, -448.f), 448.f);
      y[2 * c + 1] = fminf(fmaxf(bf_hi(ws[c]) * inv, -448.f), 448.f);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    dst[i] = make_uint2((uint32_t)lo, (uint32_t)hi);
  }
}

void launch_quantize_fp8(const uint16_t* x, uint8_t* out, float* scales, int64_t pairs, int N,
                         int stride, int d, int bs, int sstride, hipStream_t st) {
  const int nb = (N + bs - 1) / bs;
  if (nb <= 0 || pairs <= 0) return;
  const unsigned grid = (unsigned)(pairs * nb);
  if (d == 128)
    quantize_fp8_kernel<128><<<grid, 256, 0, st>>>(x, out, scales, N, stride, bs, nb, sstride);
  else
    quantize_fp8_kernel<64><<<grid, 256, 0, st>>>(x, out, scales, N, stride, bs, nb, sstride);
}

void launch_append(const uint16_t* src, uint16_t* dst, int64_t pairs, int n_new, int N,
                   int stride, int d, hipStream_t st) {
  const int ppr = d / 8;
  const int64_t pieces = pairs * n_new * ppr;
  if (pieces <= 0) return;
  append_kernel<<<(unsigned)((pieces + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), pieces, n_new, N, stride,
      ppr);
}

// ---------------------------------------------------------------------------
// Scores.  16 lanes share one summary row (512 B for d=128) and reduce their
// partial dot products with DPP inside the row; each lane builds the pooled
// query qbar (fp32 sum over the group's query heads, in head order) for its
// own dims from the query rows staged in LDS.  All of a workgroup's summary
// loads are issued before anything waits.  Grid: (row chunks, pairs) so that
// even 8 pairs spread over the whole chip.
// 128 summary rows (64 KB at d = 128) per workgroup: against 64 and 256 rows
// the select measured 17.4 vs 18.1 and 18.1 us at 128K (32 pairs), 27.6 vs
// 28.5 and 28.6 us at 1M (8 pairs)
constexpr int SCORE_ROWS_PER_WG = 128;
constexpr int SCORE_QH = 16;  // query heads staged in LDS at a time

template <int D, bool BF>
__global__ __launch_bounds__(256) void scores_kernel(const uint16_t* __restrict__ q,
                                                     const void* __restrict__ summ_v, int Hq,
                                                     int Hkv, int nb, int sstride, int c0, int c1,
                                                     float* __restrict__ scores) {
  constexpr int PER = D / 16;                       // values of a row per lane
  constexpr int PASSES = SCORE_ROWS_PER_WG / 16;    // 16 rows per pass of 256 threads
  const int pair = blockIdx.y;
  const int b = pair / Hkv, kvh = pair % Hkv, g = Hq / Hkv;
  const int tid = threadIdx.x, l16 = tid & 15;
  const int r0 = c0 + blockIdx.x * SCORE_ROWS_PER_WG;
  const int r1 = min(c1, r0 + SCORE_ROWS_PER_WG);
  // every summary load is in flight before the query is read (rows past r1
  // re-read row r1 - 1 and are not stored); fp32 rows as float4s, bf16 rows
  // as PER 2-byte values in one 16- or 8-byte load
  using BfPiece = typename std::conditional<PER == 8, uint4, uint2>::type;
  float4 w[PASSES][PER / 4];  // fp32 rows
  BfPiece wb[PASSES];         // bf16 rows
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = min(r0 + (tid >> 4) + 16 * p, r1 - 1);
    if constexpr (BF) {
      const uint16_t* base = static_cast<const uint16_t*>(summ_v) + (int64_t)pair * sstride * D +
                             l16 * PER;
      wb[p] = ld_stream(reinterpret_cast<const BfPiece*>(base + (int64_t)r * D));
    } else {
      const float* base = static_cast<const float*>(summ_v) + (int64_t)pair * sstride * D +
                          l16 * PER;
#pragma unroll
      for (int c = 0; c < PER / 4; ++c)
        w[p][c] = ld_stream(reinterpret_cast<const float4*>(base + (int64_t)r * D) + c);
    }
  }
  // pooled query over the g heads of the group, this lane's PER dims: up to
  // SCORE_QH heads at a time are read with one 16-byte load per thread into
  // LDS (all requested together), then each lane sums its dims in head order
  __shared__ __align__(16) float qs[SCORE_QH][D];
  float qv[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) qv[c] = 0.f;
  const uint16_t* qg = q + ((int64_t)b * Hq + (int64_t)kvh * g) * D;
  for (int h0 = 0; h0 < g; h0 += SCORE_QH) {
    const int hn = min(SCORE_QH, g - h0);
    for (int i = tid; i < hn * (D / 8); i += 256) {
      const int h = i / (D / 8), c8 = (i % (D / 8)) * 8;
      const uint4 u = *reinterpret_cast<const uint4*>(qg + (int64_t)(h0 + h) * D + c8);
      *reinterpret_cast<float4*>(&qs[h][c8]) = make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
      *reinterpret_cast<float4*>(&qs[h][c8 + 4]) = make_float4(bf_lo(u.z), bf_hi(u.z), bf_lo(u.w), bf_hi(u.w));
    }
    __syncthreads();
    for (int h = 0; h < hn; ++h) {
#pragma unroll
      for (int c = 0; c < PER; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&qs[h][l16 * PER + c]);
        qv[c] += x.x;
        qv[c + 1] += x.y;
        qv[c + 2] += x.z;
        qv[c + 3] += x.w;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    float x[PER];
    if constexpr (BF) {
      const uint32_t* u = reinterpret_cast<const uint32_t*>(&wb[p]);
#pragma unroll
      for (int c = 0; c < PER / 2; ++c) {
        x[2 * c] = bf_lo(u[c]);
        x[2 * c + 1] = bf_hi(u[c]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < PER / 4; ++c) {
        x[4 * c] = w[p][c].x;
        x[4 * c + 1] = w[p][c].y;
        x[4 * c + 2] = w[p][c].z;
        x[4 * c + 3] = w[p][c].w;
      }
    }
    float sc = 0.f;
#pragma unroll
    for (int c = 0; c < PER; ++c) sc = fmaf(qv[c], x[c], sc);
    sc = row16_sum(sc);
    const int r = r0 + (tid >> 4) + 16 * p;
    if (l16 == 0 && r < r1) scores[(int64_t)pair * nb + r] = sc;
  }
}

void launch_scores(const uint16_t* q, const void* summ, bool summ_bf16, int B, int Hq, int Hkv,
                   int d, int nb, int sstride, int c0, int c1, float* scores, hipStream_t st) {
  const int n = c1 - c0;
  if (n <= 0) return;
  dim3 grid((n + SCORE_ROWS_PER_WG - 1) / SCORE_ROWS_PER_WG, B * Hkv);
#define BSA_SCORES(DD, BB)                                                                \
  scores_kernel<DD, BB><<<grid, 256, 0, st>>>(q, summ, Hq, Hkv, nb, sstride, c0, c1, scores)
  if (d == 128) {
    if (summ_bf16) BSA_SCORES(128, true); else BSA_SCORES(128, false);
  } else {
    if (summ_bf16) BSA_SCORES(64, true); else BSA_SCORES(64, false);
  }
#undef BSA_SCORES
}

// ---------------------------------------------------------------------------
// Top-k.  One workgroup per (batch, kv head): 256, 512 or 1024 threads by the
// candidate count (the strided kernel: 1024).
// 1. T = the k-th largest order-preserving uint32 key, and how many keys
//    equal to T must be taken (the ones with the lowest block index).
// 2. An ordered compaction in index order writes the kept candidates
//    ascending, so the output list (sink, selected, local) is sorted with no
//    extra sort.
// Up to 16384 candidates (topk_reg_kernel) each thread keeps a contiguous run
// of KPT candidates in registers for the whole select (one read of the
// scores), T comes from a value-bucket pass and a rank inside the bucket
// holding it (topk_select_regs), and the compaction is two block-wide scans
// of per-thread counts.  Longer lists use topk_kernel: radix passes of 8 bits
// with a 256-bin LDS histogram that re-read the scores (L2) every pass, and a
// compaction in 1024-candidate strides.
constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / 64;
// histogram copies of the register-resident select: 8 from 8 candidates per
// thread on (where the first passes' same-address atomics dominate), else 1
template <int KPT> struct TopkCopies { static constexpr int value = KPT >= 8 ? 8 : 1; };

// block-wide exclusive prefix count of `flag` in thread order; returns the
// thread's prefix and sets *total.  Uses wcnt[TOPK_WAVES] of LDS.
__device__ __forceinline__ int block_prefix(bool flag, int* wcnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int pre = (int)lane_prefix(m);
  if (lane == 0) wcnt[wave] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TOPK_WAVES; ++w) {
    const int c = wcnt[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + pre;
}

// ad.on: anchor-adaptive k (the hotdry.top post's anchor selection): the
// sink and local blocks are anchors, tau = a_max + margin * (a_max - a_min)
// over their scores (fp32), k = #(candidates > tau) clamped to [k_lo, k_hi];
// the list is padded with -1 up to n_keep (the widest list).
struct AdaptiveSel {
  int on, k_lo, k_hi;
  float margin;
};

__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const float* __restrict__ scores,
                                                            int nb, int c0, int c1, int k,
                                                            int n_keep, AdaptiveSel ad,
                                                            int32_t* __restrict__ idx_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit, sh_above;
  __shared__ int wcnt[TOPK_WAVES];
  __shared__ float ext[2][TOPK_WAVES];
  const int pair = blockIdx.x;
  const int tid = threadIdx.x;
  const float* s = scores + (int64_t)pair * nb + c0;
  int32_t* out = idx_out + (int64_t)pair * n_keep;
  const int n = c1 - c0;
  if (ad.on) {  // uniform
    const float* all = scores + (int64_t)pair * nb;
    float amax = -INFINITY, amin = INFINITY;
    for (int i = tid; i < c0 + (nb - c1); i += TOPK_THREADS) {
      const float a = all[i < c0 ? i : c1 + (i - c0)];
      amax = fmaxf(amax, a);
      amin = fminf(amin, a);
    }
    amax = wave_max(amax);
    amin = -wave_max(-amin);
    if ((tid & 63) == 0) {
      ext[0][tid >> 6] = amax;
      ext[1][tid >> 6] = amin;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < TOPK_WAVES; ++w) {
      amax = fmaxf(amax, ext[0][w]);
      amin = fminf(amin, ext[1][w]);
    }
    const float tau = (c0 + (nb - c1) > 0) ? amax + ad.margin * (amax - amin) : -INFINITY;
    int cnt = 0;
    for (int base = 0; base < n; base += TOPK_THREADS) {
      int tot;
      block_prefix(base + tid < n && s[base + tid] > tau, wcnt, &tot);
      cnt += tot;
    }
    k = min(max(cnt, ad.k_lo), ad.k_hi);
    for (int i = c0 + k + (nb - c1) + tid; i < n_keep; i += TOPK_THREADS) out[i] = -1;  // absent
  }
  for (int i = tid; i < c0; i += TOPK_THREADS) out[i] = i;                 // sink
  for (int i = tid; i < nb - c1; i += TOPK_THREADS) out[c0 + k + i] = c1 + i;  // local
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += TOPK_THREADS) out[c0 + i] = c0 + i;
    return;
  }
  uint32_t prefix = 0;
  uint32_t remaining = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += TOPK_THREADS) {
      const uint32_t key = order_key(s[i]);
      const bool match = (pass == 0) || ((key ^ prefix) >> (shift + 8)) == 0;
      if (match) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending order)
      const int lane = tid;
      uint32_t c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = hist[255 - 4 * lane - e];
      const uint32_t own = c[0] + c[1] + c[2] + c[3];
      // inclusive scan over lanes (lane 0 = highest bins)
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
            sh_digit = (uint32_t)(255 - 4 * lane - e);
            sh_above = acc;
            break;
          }
          acc += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    remaining -= sh_above;
    __syncthreads();
  }
  // T = prefix: keys above T are all taken, plus the first `remaining` keys equal to T
  const uint32_t T = prefix;
  const int need_eq = (int)remaining;
  int carry_eq = 0, carry_sel = 0;
  for (int base = 0; base < n; base += TOPK_THREADS) {
    const int i = base + tid;
    const bool valid = i < n;
    const uint32_t key = valid ? order_key(s[i]) : 0u;
    const bool eq = valid && key == T;
    int tot_eq, tot_sel;
    const int eq_rank = carry_eq + block_prefix(eq, wcnt, &tot_eq);
    const bool sel = valid && (key > T || (eq && eq_rank < need_eq));
    const int pos = carry_sel + block_prefix(sel, wcnt, &tot_sel);
    if (sel) out[c0 + pos] = c0 + i;
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
}

template <int NTH, int KPT>
__global__ __launch_bounds__(NTH) void topk_reg_kernel(const float* __restrict__ scores,
                                                                int nb, int c0, int c1, int k,
                                                                int n_keep, AdaptiveSel ad,
                                                                int32_t* __restrict__ idx_out) {
  constexpr int NW = NTH / 64;
  __shared__ TopkShared<NTH, TopkCopies<KPT>::value> sh;
  __shared__ float ext[2][NW];
  const int pair = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = scores + (int64_t)pair * nb;
  int32_t* out = idx_out + (int64_t)pair * n_keep;
  const int n = c1 - c0;
  // this thread's slots: row positions [p0, p0 + KPT), an aligned run of the
  // row when it fits the slots, else a run of the candidates
  const int base = (nb <= NTH * KPT) ? 0 : c0;
  const int p0 = base + tid * KPT;
  float sv[KPT];
  load_slots<KPT>(row, base, nb, sv);
  if (ad.on) {  // uniform
    const float* all = scores + (int64_t)pair * nb;
    float amax = -INFINITY, amin = INFINITY;
    for (int i = tid; i < c0 + (nb - c1); i += NTH) {
      const float a = all[i < c0 ? i : c1 + (i - c0)];
      amax = fmaxf(amax, a);
      amin = fminf(amin, a);
    }
    amax = wave_max(amax);
    amin = -wave_max(-amin);
    if ((tid & 63) == 0) {
      ext[0][tid >> 6] = amax;
      ext[1][tid >> 6] = amin;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      amax = fmaxf(amax, ext[0][w]);
      amin = fminf(amin, ext[1][w]);
    }
    const float tau = (c0 + (nb - c1) > 0) ? amax + ad.margin * (amax - amin) : -INFINITY;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) cnt += (p0 + e >= c0 && p0 + e < c1 && sv[e] > tau) ? 1 : 0;
    wg_exscan<NTH>(cnt, sh.wtot, &cnt);
    k = min(max(cnt, ad.k_lo), ad.k_hi);
    for (int i = c0 + k + (nb - c1) + tid; i < n_keep; i += NTH) out[i] = -1;  // absent
  }
  for (int i = tid; i < c0; i += NTH) out[i] = i;                 // sink
  for (int i = tid; i < nb - c1; i += NTH) out[c0 + k + i] = c1 + i;  // local
  if (k <= 0) return;
  if (k >= n) {
    for (int i = tid; i < n; i += NTH) out[c0 + i] = c0 + i;
    return;
  }
  topk_select_regs<NTH, KPT, TopkCopies<KPT>::value>(sv, base, c0, c1, k, c0, out, sh);
}

void launch_topk(const float* scores, int64_t pairs, int nb, int c0, int c1, int k, int n_keep,
                 int32_t* idx_out, hipStream_t st, bool adaptive, int k_lo, int k_hi,
                 float margin) {
  if (pairs <= 0) return;
  AdaptiveSel ad{adaptive ? 1 : 0, k_lo, k_hi, margin};
  const int n = c1 - c0;
  // workgroup size by candidate count (measured: 509 candidates 12.7 us per
  // select with 256 threads against 13.1 / 14.3 with 512 / 1024; 2,045
  // candidates 16.5 us with 512 against 16.7 / 17.5), then the fewest
  // candidates per thread that hold them
#define BSA_TOPK_REG(NT, KK)                                                                    \
  if (n <= NT * KK)                                                                             \
    return topk_reg_kernel<NT, KK><<<(unsigned)pairs, NT, 0, st>>>(scores, nb, c0, c1, k, n_keep, \
                                                                   ad, idx_out);
  if (n <= 1024) {
    BSA_TOPK_REG(256, 1) BSA_TOPK_REG(256, 2) BSA_TOPK_REG(256, 4)
  } else if (n <= 4096) {
    BSA_TOPK_REG(512, 4) BSA_TOPK_REG(512, 8)
  } else {
    BSA_TOPK_REG(1024, 8) BSA_TOPK_REG(1024, 16)
  }
#undef BSA_TOPK_REG
  topk_kernel<<<(unsigned)pairs, TOPK_THREADS, 0, st>>>(scores, nb, c0, c1, k, n_keep, ad,
                                                        idx_out);
}

}  // namespace bsa
