// kernels_decode.hip -- split-K sparse decode attention over kept 64-token blocks.
//
// Exact softmax(q K^T * scale) V over the tokens of the kept blocks only
// ("CSA + HCA 混合注意力机制" §2.1 and §4.4 step 4).  Decode reads the whole
// kept KV once per step and does g flop per KV byte (g = query heads per kv
// head), so the kernel is built to stream bf16 K/V at HBM rate on the VALU:
//
//  * a workgroup = 4 waves owns one split (a contiguous run of the pair's
//    kept-block list); wave w takes every 4th block of the run;
//  * QK: lane t owns token t of the block and holds its whole key row
//    (d/8 16-byte loads, one contiguous row per lane), the group's queries
//    sit in LDS and are read as broadcasts; v_dot2_f32_bf16 does 2 MACs per
//    lane per instruction with exact bf16 products and fp32 sums;
//  * online softmax in base 2 with a wave-uniform running max per head;
//  * PV: lane (tg, dc) owns 8 value columns (dc) of every TG-th token (tg),
//    so each load instruction reads TG consecutive value rows (1 KiB
//    contiguous for d=128); the weights go through LDS (written by token
//    lanes, read as 16-byte broadcasts), fp32 FMA accumulation;
//  * the 4 waves merge in LDS and write one (o, m, l) partial per head;
//  * a second kernel merges the splits exactly with log-sum-exp weights.
#include <math.h>

#include "bsa_device.h"
#include "bsa_launch.h"

namespace bsa {

constexpr int DEC_WAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int D, int G>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, int n_keep, int Hq, int Hkv,
    int N, int stride, float scale_log2, int bps, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int DC = D / 8;        // 16-byte column chunks per row
  constexpr int TG = 64 / DC;      // token groups in the PV layout
  constexpr int TPL = 64 / TG;     // tokens per lane in the PV layout
  constexpr int PROW = TPL + 4;    // padded LDS row of weights (bank spread)
  __shared__ __align__(16) uint4 q_lds[G * DC];
  __shared__ __align__(16) float p_lds[DEC_WAVES][G][TG * PROW];
  __shared__ __align__(16) float m_lds[DEC_WAVES][G][2];
  __shared__ __align__(16) float o_lds[DEC_WAVES][G][D];

  const int split = blockIdx.x;
  const int pair = blockIdx.y;
  const int b = pair / Hkv, kvh = pair % Hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  {  // the group's queries -> LDS
    const uint4* qs = reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + (int64_t)kvh * G) * D);
    for (int i = tid; i < G * DC; i += 256) q_lds[i] = qs[i];
  }
  __syncthreads();

  const int blk0 = split * bps;
  const int blk1 = min(n_keep, blk0 + bps);
  const int32_t* list = idx + (int64_t)pair * n_keep;
  const uint16_t* kbase = k + (int64_t)pair * stride * D;
  const uint16_t* vbase = v + (int64_t)pair * stride * D;
  const int tg = lane / DC, dc = lane % DC;

  float m_run[G], l_lane[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }

  for (int blk = blk0 + wave; blk < blk1; blk += DEC_WAVES) {
    const int t0 = list[blk] * 64;
    // key row of token t0 + lane; values: TPL rows per lane
    uint4 kr[DC];
    uint4 vr[TPL];
    const bool kvalid = t0 + lane < N;
    {
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + (int64_t)(t0 + lane) * D);
#pragma unroll
      for (int c = 0; c < DC; ++c) kr[c] = kvalid ? ld_stream(kp + c) : make_uint4(0, 0, 0, 0);
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + (int64_t)(t0 + tg) * D) + dc;
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const bool ok = t0 + i * TG + tg < N;
        vr[i] = ok ? ld_stream(vp + (int64_t)i * TG * DC) : make_uint4(0, 0, 0, 0);
      }
    }
    // logits (base 2) of this lane's token for every head
    float z[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const uint4 qq = q_lds[h * DC + c];
        s0 = dot2(qq.x, kr[c].x, s0);
        s1 = dot2(qq.y, kr[c].y, s1);
        s0 = dot2(qq.z, kr[c].z, s0);
        s1 = dot2(qq.w, kr[c].w, s1);
      }
      z[h] = kvalid ? (s0 + s1) * scale_log2 : -INFINITY;
    }
    // online softmax; weights of token `lane` go to LDS in the PV layout
    const int pw = (lane % TG) * PROW + lane / TG;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m_new = fmaxf(m_run[h], wave_max(z[h]));
      const float alpha = exp2f(m_run[h] - m_new);
      const float p = exp2f(z[h] - m_new);
      l_lane[h] = l_lane[h] * alpha + p;
      m_run[h] = m_new;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= alpha;
      p_lds[wave][h][pw] = p;
    }
    wave_lds_sync();
    // PV
#pragma unroll
    for (int i4 = 0; i4 < TPL; i4 += 4) {
      float vf[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) unpack8(vr[i4 + u], vf[u]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float4 pp = *reinterpret_cast<const float4*>(&p_lds[wave][h][tg * PROW + i4]);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float a = acc[h][c];
          a = fmaf(pp.x, vf[0][c], a);
          a = fmaf(pp.y, vf[1][c], a);
          a = fmaf(pp.z, vf[2][c], a);
          a = fmaf(pp.w, vf[3][c], a);
          acc[h][c] = a;
        }
      }
    }
    wave_lds_sync();
  }

  // per wave: combine token groups (lanes dc + DC*tg) and the per-lane l
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lt = wave_sum(l_lane[h]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float a = acc[h][c];
#pragma unroll
      for (int off = DC; off < 64; off <<= 1) a += __shfl_xor(a, off);
      acc[h][c] = a;
    }
    if (lane < DC) {
      float4* dst = reinterpret_cast<float4*>(&o_lds[wave][h][lane * 8]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (lane == 0) {
      m_lds[wave][h][0] = m_run[h];
      m_lds[wave][h][1] = lt;
    }
  }
  __syncthreads();
  // merge the 4 waves (a wave with no block has m = -inf, l = 0, o = 0)
  const int64_t pbase = ((int64_t)pair * n_splits + split) * G;
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, m_lds[w][h][0]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float mw = m_lds[w][h][0];
      const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      o = fmaf(sc, o_lds[w][h][c], o);
    }
    part_o[(pbase + h) * D + c] = o;
    if (c == 0) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < DEC_WAVES; ++w) {
        const float mw = m_lds[w][h][0];
        const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        L = fmaf(sc, m_lds[w][h][1], L);
      }
      part_ml[(pbase + h) * 2 + 0] = M;
      part_ml[(pbase + h) * 2 + 1] = L;
    }
  }
}

// exact merge of the splits of one (batch, query head): one wave, d/64 columns per lane
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int G, int Hq, int Hkv, int S,
                                                          float* __restrict__ out,
                                                          float* __restrict__ lse) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int pair = b * Hkv + h / G, hh = h % G;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(((int64_t)pair * S + s) * G + hh) * 2]);
  float L = 0.f, o[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) o[c] = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t r = ((int64_t)pair * S + s) * G + hh;
    const float ms = part_ml[r * 2];
    const float sc = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
    L = fmaf(sc, part_ml[r * 2 + 1], L);
#pragma unroll
    for (int c = 0; c < PER; ++c) o[c] = fmaf(sc, part_o[r * D + lane + 64 * c], o[c]);
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int c = 0; c < PER; ++c) out[(int64_t)bh * D + lane + 64 * c] = o[c] * inv;
  if (lse && lane == 0) lse[bh] = (M + log2f(L)) * LN2;
}

DecodePlan plan_decode(int64_t pairs, int n_keep, int g, int n_splits_req) {
  DecodePlan p;
  p.g = g;
  if (n_splits_req > 0) {
    const int s = n_splits_req < n_keep ? n_splits_req : n_keep;
    p.bps = (n_keep + s - 1) / s;
  } else {
    // about 1024 workgroups (4 per CU), at least one block per wave
    const int64_t total = pairs * (int64_t)n_keep;
    int64_t bps = (total + 1023) / 1024;
    if (bps < DEC_WAVES) bps = DEC_WAVES;
    bps = (bps + DEC_WAVES - 1) / DEC_WAVES * DEC_WAVES;
    if (bps > n_keep) bps = n_keep;
    p.bps = (int)bps;
  }
  p.n_splits = (n_keep + p.bps - 1) / p.bps;
  return p;
}

size_t decode_workspace_bytes(int64_t pairs, int d, const DecodePlan& p) {
  return (size_t)pairs * p.n_splits * p.g * (size_t)(d + 2) * sizeof(float);
}

template <int D, int G>
static void launch_decode_t(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int N,
                            int stride, float scale, const DecodePlan& plan, float* ws,
                            float* out, float* lse, hipStream_t st) {
  const int64_t pairs = (int64_t)B * Hkv;
  float* part_o = ws;
  float* part_ml = ws + (size_t)pairs * plan.n_splits * G * D;
  dim3 grid(plan.n_splits, (unsigned)pairs);
  decode_partial_kernel<D, G><<<grid, 256, 0, st>>>(q, k, v, idx, n_keep, Hq, Hkv, N, stride,
                                                    scale * LOG2E, plan.bps, plan.n_splits,
                                                    part_o, part_ml);
  decode_merge_kernel<D><<<(unsigned)(B * Hq), 64, 0, st>>>(part_o, part_ml, G, Hq, Hkv,
                                                            plan.n_splits, out, lse);
}

void launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                   int n_keep, int B, int Hq, int Hkv, int d, int N, int stride, float scale,
                   const DecodePlan& plan, float* ws, float* out, float* lse, hipStream_t st) {
#define BSA_DEC(DD, GG)                                                                        \
  if (d == DD && plan.g == GG)                                                                 \
    return launch_decode_t<DD, GG>(q, k, v, idx, n_keep, B, Hq, Hkv, N, stride, scale, plan,  \
                                   ws, out, lse, st);
  BSA_DEC(128, 1) BSA_DEC(128, 2) BSA_DEC(128, 4) BSA_DEC(128, 8) BSA_DEC(128, 16)
  BSA_DEC(64, 1) BSA_DEC(64, 2) BSA_DEC(64, 4) BSA_DEC(64, 8) BSA_DEC(64, 16)
#undef BSA_DEC
}

}  // namespace bsa
