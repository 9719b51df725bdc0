// kernels_decode.hip -- split-K sparse decode attention over kept 64-token blocks.
//
// Exact softmax(q K^T * scale) V over the tokens of the kept blocks only
// ("CSA + HCA 混合注意力机制" §2.1 and §4.4 step 4).  Decode streams the kept
// KV once per step; its rate is set by how many bytes each CU keeps in
// flight, so the kernel is built around a deep per-wave load pipeline:
//
//  * a workgroup of 4 waves owns one split (a contiguous run of one
//    (batch, kv head) pair's kept-block list); wave w owns tokens
//    [16w, 16w+16) of every block of the run, i.e. one 16-token tile per
//    block, and keeps its own online-softmax state;
//  * per tile a wave needs only 4 KiB of K and 4 KiB of V, so P tiles
//    (P = 3, or 2 for 16 query heads per kv head) are requested ahead into
//    registers: the loop always issues the tile P-1 steps ahead (a dummy
//    broadcast load past the end) and never branches around its loads;
//  * QK on the matrix cores: the g query heads of the kv group share each
//    key tile, S^T[16 x 16] = K_tile[16 x d] q^T[d x 16] is d/32
//    v_mfma_f32_16x16x32_bf16 (heads past g are zero); q stays in
//    registers as the B operand; K fragments come straight from HBM in the
//    A-operand layout (lane l: token l%16, 16 bytes at 32*kstep + 8*(l/16));
//  * online softmax in base 2 per head in the MFMA accumulator layout, the
//    tile max across the 4 lanes of a head by two cross-lane exchanges;
//  * PV on the VALU: lane (ts, dq) owns 4 value columns (dq) of every
//    (64/(d/4))-th token of the tile, so each 8-byte load instruction reads
//    whole value rows; the weights reach those lanes through LDS;
//  * the 4 waves merge in LDS into one (o, m, l) partial per head, and a
//    second small kernel merges the splits exactly with log-sum-exp weights.
#include <math.h>

#include "bsa_device.h"
#include "bsa_launch.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int DEC_WAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// blocks in flight per wave (register budget: two waves per SIMD)
template <int G> struct DecStages { static constexpr int value = G >= 16 ? 2 : 3; };

template <int D, int G, int P>
__global__ __launch_bounds__(256, 2) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, int n_keep, int Hq, int Hkv,
    int N, int stride, float scale_log2, int bps, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int KS = D / 32;        // MFMA k-steps over the head dim
  constexpr int DQ = D / 4;         // 4-column groups per row: lane owns one group
  constexpr int VT = 64 / DQ;       // token subgroups in the PV layout (2 for d=128)
  constexpr int TPL = 16 / VT;      // tokens of the tile per lane (PV layout)
  constexpr int GP = G < 4 ? 4 : G;  // padded weights row
  __shared__ __align__(16) float p_lds[DEC_WAVES][16 * GP];
  __shared__ __align__(16) float a_lds[DEC_WAVES][GP];
  __shared__ __align__(16) float m_lds[DEC_WAVES][G][2];
  __shared__ __align__(16) float o_lds[DEC_WAVES][G][D];

  const int split = blockIdx.x;
  const int pair = blockIdx.y;
  const int b = pair / Hkv, kvh = pair % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, j4 = lane >> 4;
  const int dq = lane % DQ, ts = lane / DQ;

  // q^T as the MFMA B operand: lane l holds head l%16, dims 32*ks + 8*(l/16) .. +8
  uint4 qf[KS];
  {
    const uint4* qs = reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + (int64_t)kvh * G) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (l16 < G) ? qs[l16 * (D / 8) + ks * 4 + j4] : make_uint4(0, 0, 0, 0);
  }

  const int blk0 = split * bps;
  int nblk = min(n_keep, blk0 + bps) - blk0;
  const int32_t* list = idx + (int64_t)pair * n_keep + blk0;
  // a list may end in -1 (absent entries of an adaptive selection): this
  // split's blocks are its valid prefix (one scalar load when the run is full)
  if (nblk > 0 && list[nblk - 1] < 0) {
    int nv = 0;
    while (nv < nblk && list[nv] >= 0) ++nv;
    nblk = nv;
  }
  const char* kb = reinterpret_cast<const char*>(k + (int64_t)pair * stride * D);
  const char* vb = reinterpret_cast<const char*>(v + (int64_t)pair * stride * D);
  const int tile0 = 16 * wave;  // this wave's 16 tokens of every block

  float m_run = -INFINITY, l_run = 0.f;  // head l16 over this lane's tokens
  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.f;

  // register pipeline: P blocks in flight per wave (K tile + V tile)
  uint4 kbuf[P][KS];
  uint2 vbuf[P][TPL];
  // j >= nblk issues a dummy load (every lane reads the pair's first row) so
  // the pipeline never branches around its loads
  auto issue = [&](int slot, int j) {
    const bool real = j < nblk;
    const int t0 = list[real ? j : 0] * 64 + tile0;
    const uint32_t koff =
        real ? (uint32_t)min(t0 + l16, N - 1) * (D * 2) + j4 * 16 : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kbuf[slot][ks] = ld_stream(reinterpret_cast<const uint4*>(kb + koff + (real ? ks * 64 : 0)));
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t voff =
          real ? (uint32_t)min(t0 + ts + VT * i, N - 1) * (D * 2) + dq * 8 : 0u;
      vbuf[slot][i] = ld_stream(reinterpret_cast<const uint2*>(vb + voff));
    }
  };
  float* pl = p_lds[wave];
  auto compute = [&](int slot, int j) {
    const int t0 = list[j] * 64 + tile0;
    // S^T tile: lane l gets tokens 4*(l/16) + i of the tile, head l%16
    f32x4v sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kbuf[slot][ks]), as_bf16x8(qf[ks]),
                                                   sc, 0, 0, 0);
    float z[4];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = (t0 + 4 * j4 + i < N) ? sc[i] * scale_log2 : -INFINITY;
      bm = fmaxf(bm, z[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    // a tile past seq_len has no valid token: keep everything at zero
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(z[i] - m_use);
      ps += p;
      if (l16 < G) pl[(4 * j4 + i) * GP + l16] = p;
    }
    l_run = l_run * alpha + ps;
    if (j4 == 0 && l16 < G) a_lds[wave][l16] = alpha;
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = a_lds[wave][h];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[h][c] *= al;
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const float vv[4] = {bf_lo(vbuf[slot][i].x), bf_hi(vbuf[slot][i].x),
                           bf_lo(vbuf[slot][i].y), bf_hi(vbuf[slot][i].y)};
      const float* prow = pl + (ts + VT * i) * GP;
#pragma unroll
      for (int h4 = 0; h4 < G; h4 += 4) {
        const float4 pp = *reinterpret_cast<const float4*>(prow + h4);
        const float pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (h4 + u < G) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[h4 + u][c] = fmaf(pv[u], vv[c], acc[h4 + u][c]);
          }
      }
    }
    wave_lds_sync();
  };

#pragma unroll
  for (int s = 0; s < P - 1; ++s) issue(s, s);
  for (int it = 0; it < nblk; it += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      issue((s + P - 1) % P, it + s + P - 1);
      if (it + s < nblk) compute(s, it + s);
    }
  }

  // per wave: l over the 4 lanes of a head; acc over the token subgroups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int off = DQ; off < 64; off <<= 1)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[h][c] += __shfl_xor(acc[h][c], off);
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      *reinterpret_cast<float4*>(&o_lds[wave][h][4 * dq]) =
          make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  }
  if (j4 == 0 && l16 < G) {
    m_lds[wave][l16][0] = m_run;
    m_lds[wave][l16][1] = l_run;
  }
  __syncthreads();
  // merge the 4 waves: each holds a softmax partial over its quarter of every block
  const int64_t pbase = ((int64_t)pair * n_splits + split) * G;
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, m_lds[w][h][0]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float mw = m_lds[w][h][0];
      const float sc = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      o = fmaf(sc, o_lds[w][h][c], o);
      L = fmaf(sc, m_lds[w][h][1], L);
    }
    part_o[(pbase + h) * D + c] = o;
    if (c == 0) {
      part_ml[(pbase + h) * 2 + 0] = M;
      part_ml[(pbase + h) * 2 + 1] = L;
    }
  }
}

// FP8 (OCP E4M3) cache variant of decode_kernel.  K and V rows are one byte
// per value with one fp32 scale per (b, kv head, 64-token block) each; the
// E4M3 values convert exactly to bf16 / fp32 (v_cvt_pk_f32_fp8), the K scale
// multiplies the block's logits and the V scale the weights the PV step
// reads, so the arithmetic is that of the bf16 kernel on the dequantized
// cache.  Half the bytes per block, so P (blocks in flight) is one deeper.
// The MFMA k order is permuted so a lane's 8*KS key bytes are contiguous:
// lane l holds dims [8*KS*(l/16) + 8*ks, +8) of k-step ks, on both operands.
template <int G> struct DecStagesFp8 { static constexpr int value = G >= 16 ? 2 : 4; };

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  // two E4M3 values (bytes 2*HI, 2*HI + 1 of w) -> two bf16 (exact: E4M3 fits bf16)
  typedef float f2v __attribute__((ext_vector_type(2)));
  const f2v f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xFFFF0000u);
}

template <int D, int G, int P>
__global__ __launch_bounds__(256, 2) void decode_fp8_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const float* __restrict__ ksc, const float* __restrict__ vsc, int sstride,
    const int32_t* __restrict__ idx, int n_keep, int Hq, int Hkv, int N, int stride,
    float scale_log2, int bps, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int KS = D / 32;        // MFMA k-steps over the head dim
  constexpr int KB = KS / 2;        // 16-byte key loads per lane per tile
  constexpr int DQ = D / 4;         // 4-column groups per row: lane owns one group
  constexpr int VT = 64 / DQ;       // token subgroups in the PV layout
  constexpr int TPL = 16 / VT;      // tokens of the tile per lane (PV layout)
  constexpr int GP = G < 4 ? 4 : G;
  static_assert(KS % 2 == 0, "head dim a multiple of 64");
  __shared__ __align__(16) float p_lds[DEC_WAVES][16 * GP];
  __shared__ __align__(16) float a_lds[DEC_WAVES][GP];
  __shared__ __align__(16) float m_lds[DEC_WAVES][G][2];
  __shared__ __align__(16) float o_lds[DEC_WAVES][G][D];

  const int split = blockIdx.x;
  const int pair = blockIdx.y;
  const int b = pair / Hkv, kvh = pair % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;
  const int dq = lane % DQ, ts = lane / DQ;

  // q^T fragments in the permuted k order
  uint4 qf[KS];
  {
    const uint4* qs = reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + (int64_t)kvh * G) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (l16 < G) ? qs[l16 * (D / 8) + j4 * KS + ks] : make_uint4(0, 0, 0, 0);
  }

  const int blk0 = split * bps;
  int nblk = min(n_keep, blk0 + bps) - blk0;
  const int32_t* list = idx + (int64_t)pair * n_keep + blk0;
  if (nblk > 0 && list[nblk - 1] < 0) {  // a -1-padded (adaptive) list
    int nv = 0;
    while (nv < nblk && list[nv] >= 0) ++nv;
    nblk = nv;
  }
  const uint8_t* kb = k + (int64_t)pair * stride * D;
  const uint8_t* vb = v + (int64_t)pair * stride * D;
  const float* ks_row = ksc + (int64_t)pair * sstride;
  const float* vs_row = vsc + (int64_t)pair * sstride;
  const int tile0 = 16 * wave;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.f;

  uint4 kbuf[P][KB];
  uint32_t vbuf[P][TPL];
  float skb[P], svb[P];
  auto issue = [&](int slot, int j) {
    const bool real = j < nblk;
    const int blk = list[real ? j : 0];
    const int t0 = blk * 64 + tile0;
    const uint32_t koff = real ? (uint32_t)min(t0 + l16, N - 1) * D + j4 * (8 * KS) : 0u;
#pragma unroll
    for (int u = 0; u < KB; ++u)
      kbuf[slot][u] = ld_stream(reinterpret_cast<const uint4*>(kb + koff) + (real ? u : 0));
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      const uint32_t voff = real ? (uint32_t)min(t0 + ts + VT * i, N - 1) * D + dq * 4 : 0u;
      vbuf[slot][i] = *reinterpret_cast<const uint32_t*>(vb + voff);
    }
    skb[slot] = ks_row[blk];
    svb[slot] = vs_row[blk];
  };
  float* pl = p_lds[wave];
  auto compute = [&](int slot, int j) {
    const int t0 = list[j] * 64 + tile0;
    f32x4v sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 w = kbuf[slot][ks / 2];
      const uint32_t lo = (ks & 1) ? w.z : w.x, hi = (ks & 1) ? w.w : w.y;
      const uint4 kk = make_uint4(fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo),
                                  fp8x2_to_bf16x2<false>(hi), fp8x2_to_bf16x2<true>(hi));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kk), as_bf16x8(qf[ks]), sc, 0, 0, 0);
    }
    const float zs = scale_log2 * skb[slot];  // the block's K scale folds into the logits
    float z[4];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = (t0 + 4 * j4 + i < N) ? sc[i] * zs : -INFINITY;
      bm = fmaxf(bm, z[i]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float ps = 0.f;
    const float sv = svb[slot];  // the block's V scale folds into the weights PV reads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(z[i] - m_use);
      ps += p;
      if (l16 < G) pl[(4 * j4 + i) * GP + l16] = p * sv;
    }
    l_run = l_run * alpha + ps;
    if (j4 == 0 && l16 < G) a_lds[wave][l16] = alpha;
    wave_lds_sync();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = a_lds[wave][h];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[h][c] *= al;
    }
#pragma unroll
    for (int i = 0; i < TPL; ++i) {
      typedef float f2v __attribute__((ext_vector_type(2)));
      const f2v v01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vbuf[slot][i], false);
      const f2v v23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vbuf[slot][i], true);
      const float vv[4] = {v01.x, v01.y, v23.x, v23.y};
      const float* prow = pl + (ts + VT * i) * GP;
#pragma unroll
      for (int h4 = 0; h4 < G; h4 += 4) {
        const float4 pp = *reinterpret_cast<const float4*>(prow + h4);
        const float pv[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (h4 + u < G) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[h4 + u][c] = fmaf(pv[u], vv[c], acc[h4 + u][c]);
          }
      }
    }
    wave_lds_sync();
  };

#pragma unroll
  for (int s = 0; s < P - 1; ++s) issue(s, s);
  for (int it = 0; it < nblk; it += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      issue((s + P - 1) % P, it + s + P - 1);
      if (it + s < nblk) compute(s, it + s);
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int off = DQ; off < 64; off <<= 1)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[h][c] += __shfl_xor(acc[h][c], off);
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      *reinterpret_cast<float4*>(&o_lds[wave][h][4 * dq]) =
          make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
  }
  if (j4 == 0 && l16 < G) {
    m_lds[wave][l16][0] = m_run;
    m_lds[wave][l16][1] = l_run;
  }
  __syncthreads();
  const int64_t pbase = ((int64_t)pair * n_splits + split) * G;
  for (int e = tid; e < G * D; e += 256) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, m_lds[w][h][0]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float mw = m_lds[w][h][0];
      const float scw = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      o = fmaf(scw, o_lds[w][h][c], o);
      L = fmaf(scw, m_lds[w][h][1], L);
    }
    part_o[(pbase + h) * D + c] = o;
    if (c == 0) {
      part_ml[(pbase + h) * 2 + 0] = M;
      part_ml[(pbase + h) * 2 + 1] = L;
    }
  }
}

// Exact merge of the splits of one (batch, query head): M = max m_s,
// L = sum 2^(m_s - M) l_s, o = sum 2^(m_s - M) o_s / L, lse = (M + log2 L) ln 2.
// One workgroup of D threads per (batch, query head); the split weights are
// computed once into LDS, then every column sums its splits with independent
// loads.  A separate launch: the kernel boundary makes the partials of all
// workgroups visible (an agent-scope fence per workgroup is far more costly
// on a multi-XCD part).
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         int G, int Hq, int Hkv, int S,
                                                         float* __restrict__ out,
                                                         float* __restrict__ lse) {
  constexpr int SMAX = 1024;
  __shared__ float w_lds[SMAX];
  __shared__ float red[D / 64][2];
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int pair = b * Hkv + h / G, hh = h % G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = (int64_t)pair * S * G + hh;  // row of split s: r0 + s * G
  float M = -INFINITY;
  for (int s2 = tid; s2 < S; s2 += D) M = fmaxf(M, part_ml[(r0 + (int64_t)s2 * G) * 2]);
  M = wave_max(M);
  if (lane == 0) red[wave][0] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < D / 64; ++w) M = fmaxf(M, red[w][0]);
  float L = 0.f, o = 0.f;
  for (int sb = 0; sb < S; sb += SMAX) {
    const int se = min(S, sb + SMAX);
    __syncthreads();
    for (int s2 = sb + tid; s2 < se; s2 += D) {
      const int64_t r = r0 + (int64_t)s2 * G;
      const float ms = part_ml[r * 2];
      const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      w_lds[s2 - sb] = w;
      L = fmaf(w, part_ml[r * 2 + 1], L);
    }
    __syncthreads();
#pragma unroll 8
    for (int s2 = sb; s2 < se; ++s2) o = fmaf(w_lds[s2 - sb], part_o[(r0 + (int64_t)s2 * G) * D + tid], o);
  }
  L = wave_sum(L);
  if (lane == 0) red[wave][1] = L;
  __syncthreads();
  L = 0.f;
#pragma unroll
  for (int w = 0; w < D / 64; ++w) L += red[w][1];
  out[(int64_t)bh * D + tid] = o / L;
  if (lse && tid == 0) lse[bh] = (M + log2f(L)) * LN2;
}

// Two workgroups of 4 waves fit per CU (two waves per SIMD), so the plan aims
// at one full round of 512 workgroups over the MI355X's 256 CUs: splits per
// pair = round(512 / pairs), each split a contiguous run of the kept-block
// list.  More pairs than that: one split per pair.
constexpr int DEC_TARGET_WGS = 512;

DecodePlan plan_decode(int64_t pairs, int n_keep, int g, int n_splits_req) {
  DecodePlan p;
  p.g = g;
  int64_t s = n_splits_req;
  if (s <= 0) {
    s = (DEC_TARGET_WGS + pairs / 2) / pairs;
    if (s < 1) s = 1;
  }
  if (s > n_keep) s = n_keep;
  p.bps = (int)((n_keep + s - 1) / s);
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
  float* part_ml = ws;
  float* part_o = part_ml + (size_t)pairs * plan.n_splits * G * 2;
  dim3 grid(plan.n_splits, (unsigned)pairs);
  decode_kernel<D, G, DecStages<G>::value><<<grid, 256, 0, st>>>(
      q, k, v, idx, n_keep, Hq, Hkv, N, stride, scale * LOG2E, plan.bps, plan.n_splits, part_o,
      part_ml);
  decode_merge_kernel<D><<<(unsigned)(B * Hq), D, 0, st>>>(part_o, part_ml, G, Hq, Hkv,
                                                           plan.n_splits, out, lse);
}

template <int D, int G>
static void launch_decode_fp8_t(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                                const float* ksc, const float* vsc, int sstride,
                                const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int N,
                                int stride, float scale, const DecodePlan& plan, float* ws,
                                float* out, float* lse, hipStream_t st) {
  const int64_t pairs = (int64_t)B * Hkv;
  float* part_ml = ws;
  float* part_o = part_ml + (size_t)pairs * plan.n_splits * G * 2;
  dim3 grid(plan.n_splits, (unsigned)pairs);
  decode_fp8_kernel<D, G, DecStagesFp8<G>::value><<<grid, 256, 0, st>>>(
      q, k, v, ksc, vsc, sstride, idx, n_keep, Hq, Hkv, N, stride, scale * LOG2E, plan.bps,
      plan.n_splits, part_o, part_ml);
  decode_merge_kernel<D><<<(unsigned)(B * Hq), D, 0, st>>>(part_o, part_ml, G, Hq, Hkv,
                                                           plan.n_splits, out, lse);
}

void launch_decode_fp8(const uint16_t* q, const uint8_t* k, const uint8_t* v, const float* ksc,
                       const float* vsc, int sstride, const int32_t* idx, int n_keep, int B,
                       int Hq, int Hkv, int d, int N, int stride, float scale,
                       const DecodePlan& plan, float* ws, float* out, float* lse,
                       hipStream_t st) {
#define BSA_DEC(DD, GG)                                                                        \
  if (d == DD && plan.g == GG)                                                                 \
    return launch_decode_fp8_t<DD, GG>(q, k, v, ksc, vsc, sstride, idx, n_keep, B, Hq, Hkv, N, \
                                       stride, scale, plan, ws, out, lse, st);
  BSA_DEC(128, 1) BSA_DEC(128, 2) BSA_DEC(128, 4) BSA_DEC(128, 8) BSA_DEC(128, 16)
  BSA_DEC(64, 1) BSA_DEC(64, 2) BSA_DEC(64, 4) BSA_DEC(64, 8) BSA_DEC(64, 16)
#undef BSA_DEC
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
