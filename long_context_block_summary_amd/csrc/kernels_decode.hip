// kernels_decode.hip -- split-K sparse decode attention over kept 64-token blocks.
//
// Exact softmax(q K^T * scale) V over the tokens of the kept blocks only
// ("CSA + HCA 混合注意力机制" §2.1 and §4.4 step 4).  Decode streams the kept
// KV once per step, so the kernel keeps a deep per-wave load pipeline and
// puts both products on the matrix cores (a P.V product on the vector ALU
// costs ~256 FMAs per lane per tile and made the kernel issue-bound):
//
//  * a workgroup of 4 waves owns one split (a contiguous run of one
//    (batch, kv head) pair's kept-block list); wave w owns tokens
//    [16w, 16w+16) of every block of the run, i.e. one 16-token tile per
//    block, and keeps its own online-softmax state;
//  * P tiles (K tile + V tile) are requested ahead into registers: the loop
//    always issues the tile P-1 steps ahead (a dummy broadcast load past the
//    end) and never branches around its loads;
//  * QK: S^T[16 tok x 16 heads] = K_tile q^T, d/32 v_mfma_f32_16x16x32_bf16
//    (heads past g are zero); q stays in registers as the B operand and the
//    K fragments come straight from HBM in the A-operand layout;
//  * online softmax in base 2 per head in the accumulator layout; the
//    running max moves only when a logit exceeds it by more than 2^8 (exact:
//    o and l always share the same reference max);
//  * PV: O^T[d x 16 heads] += V^T_tile P^T, one 16x16x32 MFMA per 16 value
//    columns.  The S^T accumulator is already the B-operand layout of P^T; P
//    enters as a bf16 pair hi + lo (k 0..3 and 4..7 of each lane) so the
//    product keeps ~16 bits of the fp32 weight.  V rows are loaded
//    coalesced, transposed 4x4 in registers (v_perm) and staged per wave in
//    LDS as V^T, from where each lane reads its A fragment with one 8-byte
//    read;
//  * the 4 waves merge in LDS into one (o, m, l) partial per head, and a
//    second small kernel merges the splits exactly with log-sum-exp weights.
#include <math.h>

#include <type_traits>

#include "bsa_device.h"
#include "bsa_launch.h"
#include "topk_device.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int DEC_WAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float DEC_RESCALE_LOG2 = 8.f;  // lazy max threshold (weights stay <= 2^8)

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// V^T staging: per wave D rows (value columns) of 16 bf16 tokens = 4 groups
// of 4 tokens (8 bytes).  Row r lives at physical row r ^ ((r >> 3) & 7): a
// bijection within every 16-row group, so the fragment reads (16 consecutive
// rows) stay one contiguous 512-byte span, while the transposing writes
// (rows 4 or 8 apart) spread over all banks.
__device__ __forceinline__ int vt_row(int r) { return r ^ ((r >> 3) & 7); }

// the two 16-bit halves (sel: low halves 0x05040100, high halves 0x07060302)
// of a and b -> one bf16 pair {a, b}
__device__ __forceinline__ uint32_t pick16(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(b, a, sel);
}

// p (fp32, >= 0) -> bf16 hi part (truncation) and bf16 lo part p - hi; the
// B fragment of P^T: k 0..3 = hi of the lane's 4 tokens, k 4..7 = lo
__device__ __forceinline__ uint4 split_weights(const float p[4]) {
  float lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lo[i] = p[i] - __uint_as_float(__float_as_uint(p[i]) & 0xffff0000u);
  return make_uint4(pick16(__float_as_uint(p[0]), __float_as_uint(p[1]), 0x07060302u),
                    pick16(__float_as_uint(p[2]), __float_as_uint(p[3]), 0x07060302u),
                    pick16(__float_as_uint(lo[0]), __float_as_uint(lo[1]), 0x07060302u),
                    pick16(__float_as_uint(lo[2]), __float_as_uint(lo[3]), 0x07060302u));
}

// Per-tile online softmax + PV shared by the bf16 and FP8 kernels.
// sc: S^T accumulator (lane l: tokens 4*(l/16)+i of the tile, head l%16);
// zscale: logit scale (log2 units); n_valid: tokens of the tile below seq_len
// relative to this lane's first token; wscale: factor on the weights PV reads;
// vt: this wave's V^T rows (already written, wave-synchronised).
template <int NC>
__device__ __forceinline__ void softmax_pv(const f32x4v& sc, float zscale, int n_valid,
                                           float wscale, const uint2* vt, int l16, int j4,
                                           float& m_run, float& l_run, f32x4v* acc) {
  float z[4];
  float bm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = (i < n_valid) ? sc[i] * zscale : -INFINITY;
    bm = fmax_nc(bm, z[i]);
  }
  bm = pair32_max(pair16_max(bm));
  // the 4 lanes of a head agree on bm and m_run, so on grow
  const bool grow = bm > m_run + DEC_RESCALE_LOG2;
  if (__builtin_amdgcn_ballot_w64(grow)) {  // wave-uniform
    const float m_new = grow ? bm : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 from -inf, 1 if kept
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] *= alpha;
    l_run *= alpha;
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
  float p[4];
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(z[i] - m_use);
    ps += p[i];
    p[i] *= wscale;
  }
  l_run += ps;
  const uint4 pb = split_weights(p);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint2 w = vt[vt_row(16 * c + l16) * 4 + j4];
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(make_uint4(w.x, w.y, w.x, w.y)),
                                                     as_bf16x8(pb), acc[c], 0, 0, 0);
  }
}

// Per wave: (m, l) over the tile lanes of a head, o^T from the accumulators,
// then the 4 waves merge into the split's partial.
template <int D, int G>
__device__ __forceinline__ void decode_finish(float m_run, float l_run, const f32x4v* acc,
                                              float (*m_lds)[G][2], float (*o_lds)[G][D],
                                              int wave, int tid, int64_t pbase,
                                              float* __restrict__ part_o,
                                              float* __restrict__ part_ml) {
  constexpr int NC = D / 16;
  const int lane = tid & 63, l16 = lane & 15, j4 = lane >> 4;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (l16 < G) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *reinterpret_cast<float4*>(&o_lds[wave][l16][16 * c + 4 * j4]) =
          make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
    if (j4 == 0) {
      m_lds[wave][l16][0] = m_run;
      m_lds[wave][l16][1] = l_run;
    }
  }
  __syncthreads();
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

// The kept-block run of this split; a list may end in -1 (absent entries of
// an adaptive selection): the split's blocks are its valid prefix (one scalar
// load when the run is full).
__device__ __forceinline__ int split_blocks(const int32_t* list, int n_keep, int blk0, int bps) {
  int nblk = min(n_keep, blk0 + bps) - blk0;
  if (nblk > 0 && list[nblk - 1] < 0) {
    int nv = 0;
    while (nv < nblk && list[nv] >= 0) ++nv;
    nblk = nv;
  }
  return nblk;
}

// blocks in flight per wave.  The bf16 kernel keeps the register budget of
// two waves per SIMD (deeper pipelines at one wave per SIMD, 4-6 stages,
// measured slower); the FP8 kernel, with half the bytes per tile, takes 5
// stages at one wave per SIMD (one workgroup per CU is what the plan launches)
constexpr int DEC_STAGES = 3;
constexpr int DEC_STAGES_FP8 = 5;

// SEL: the workgroup first selects its pair's kept blocks from the block
// scores itself (the same list select_blocks writes; split 0 also writes it
// to sel.idx_out) instead of reading idx: no separate top-k launch.
struct FusedSelect {
  const float* scores;  // [pairs][nb] block scores (candidates [c0, c1) written)
  int nb, c0, c1, k;    // sink blocks [0, c0), candidates [c0, c1), local [c1, nb); top-k
  int32_t* idx_out;     // [pairs][n_keep] kept list, written by split 0
};
constexpr int DEC_SEL_KPT = 16;                 // candidates per thread: up to 4096
constexpr int DEC_SEL_MAX_CAND = 256 * DEC_SEL_KPT;
constexpr int DEC_SEL_MAX_KEEP = DEC_SEL_MAX_CAND + 64;

template <int D, int G, int P, int SELK = 0>
__global__ __launch_bounds__(256, 2) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, int n_keep, int Hq, int Hkv,
    int N, int stride, float scale_log2, int bps, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml, FusedSelect fs = {}) {
  constexpr int KS = D / 32;  // QK k-steps over the head dim
  constexpr int NB = D / 64;  // 64-column blocks of a V row (16 lanes x 4 columns)
  constexpr int NC = D / 16;  // PV column chunks
  static_assert(G <= 16 && D % 64 == 0, "16 heads per MFMA tile, head dim a multiple of 64");
  __shared__ __align__(16) uint2 vt_lds[DEC_WAVES][D * 4];
  __shared__ __align__(16) float m_lds[DEC_WAVES][G][2];
  __shared__ __align__(16) float o_lds[DEC_WAVES][G][D];

  const int split = blockIdx.x;
  const int pair = blockIdx.y;
  const int b = pair / Hkv, kvh = pair % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, j4 = lane >> 4;

  // q^T as the MFMA B operand: lane l holds head l%16, dims 32*ks + 8*(l/16) .. +8
  uint4 qf[KS];
  {
    const uint4* qs = reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + (int64_t)kvh * G) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (l16 < G) ? qs[l16 * (D / 8) + ks * 4 + j4] : make_uint4(0, 0, 0, 0);
  }

  constexpr bool SEL = SELK > 0;
  using SelShared = std::conditional_t<SEL, TopkShared<256, 8>, char>;
  __shared__ SelShared sel_sh;
  __shared__ int32_t list_lds[SEL ? DEC_SEL_MAX_KEEP : 1];
  if constexpr (SEL) {
    // the pair's kept list into LDS: sink, the top-k of the candidates, local
    const int n = fs.c1 - fs.c0;
    for (int i = tid; i < fs.c0; i += 256) list_lds[i] = i;
    for (int i = tid; i < fs.nb - fs.c1; i += 256) list_lds[fs.c0 + fs.k + i] = fs.c1 + i;
    if (fs.k >= n) {  // uniform
      for (int i = tid; i < n; i += 256) list_lds[fs.c0 + i] = fs.c0 + i;
    } else if (fs.k > 0) {
      topk_into_list<256, (SEL ? SELK : 1), 8>(fs.scores + (int64_t)pair * fs.nb, fs.nb, fs.c0,
                                                fs.c1, fs.k, list_lds, sel_sh);
    }
    __syncthreads();
    if (split == 0)
      for (int i = tid; i < n_keep; i += 256) fs.idx_out[(int64_t)pair * n_keep + i] = list_lds[i];
  }
  const int blk0 = split * bps;
  const int32_t* list = SEL ? list_lds + blk0 : idx + (int64_t)pair * n_keep + blk0;
  const int nblk = split_blocks(list, n_keep, blk0, bps);
  const char* kb = reinterpret_cast<const char*>(k + (int64_t)pair * stride * D);
  const char* vb = reinterpret_cast<const char*>(v + (int64_t)pair * stride * D);
  const int tile0 = 16 * wave;  // this wave's 16 tokens of every block

  float m_run = -INFINITY, l_run = 0.f;  // head l16
  f32x4v acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x4v{0.f, 0.f, 0.f, 0.f};

  // register pipeline: K fragments (lane: token l16, bytes 16*j4 of each
  // 64-byte k-step) and V rows 4*j4 + r, columns 64*nb + 4*l16 .. +3
  uint4 kbuf[P][KS];
  uint2 vbuf[P][NB][4];
  // j >= nblk issues a dummy load (every lane reads the pair's first row) so
  // the pipeline never branches around its loads
  auto issue = [&](int slot, int j) {
    const bool real = j < nblk;
    // a caller's entry outside [0, nb) is clamped to a valid block: every
    // read stays inside the pair's rows (the result is then unspecified)
    const int t0 = min(max(list[real ? j : 0], 0), (N - 1) >> 6) * 64 + tile0;
    const uint32_t koff = real ? (uint32_t)min(t0 + l16, N - 1) * (D * 2) + j4 * 16 : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kbuf[slot][ks] = ld_stream(reinterpret_cast<const uint4*>(kb + koff + (real ? ks * 64 : 0)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t voff = real ? (uint32_t)min(t0 + 4 * j4 + r, N - 1) * (D * 2) + l16 * 8 : 0u;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vbuf[slot][nb][r] = ld_stream(reinterpret_cast<const uint2*>(vb + voff + (real ? nb * 128 : 0)));
    }
  };
  uint2* vt = vt_lds[wave];
  auto compute = [&](int slot, int j) {
    const int t0 = list[j] * 64 + tile0;
    f32x4v sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kbuf[slot][ks]), as_bf16x8(qf[ks]),
                                                   sc, 0, 0, 0);
    // V^T: lane (j4, l16) holds tokens 4*j4 .. +3 x columns 64*nb + 4*l16 .. +3
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
        const uint2* rw = vbuf[slot][nb];
        const uint32_t w0 = (d < 2) ? rw[0].x : rw[0].y, w1 = (d < 2) ? rw[1].x : rw[1].y;
        const uint32_t w2 = (d < 2) ? rw[2].x : rw[2].y, w3 = (d < 2) ? rw[3].x : rw[3].y;
        vt[vt_row(64 * nb + 4 * l16 + d) * 4 + j4] = make_uint2(pick16(w0, w1, sel), pick16(w2, w3, sel));
      }
    wave_lds_sync();
    softmax_pv<NC>(sc, scale_log2, N - (t0 + 4 * j4), 1.f, vt, l16, j4, m_run, l_run, acc);
    wave_lds_sync();  // the next tile's V^T writes follow this tile's reads
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
  decode_finish<D, G>(m_run, l_run, acc, m_lds, o_lds, wave, tid,
                      ((int64_t)pair * n_splits + split) * G, part_o, part_ml);
}

// FP8 (OCP E4M3) cache variant of decode_kernel.  K and V rows are one byte
// per value with one fp32 scale per (b, kv head, 64-token block) each; the
// E4M3 values convert exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8 with a
// unit scale, two values per instruction), the K scale multiplies the block's logits and the V scale the
// weights PV reads, so the arithmetic is that of the bf16 kernel on the
// dequantized cache.  Half the bytes per block, so P is one deeper.  The QK
// k order is permuted so a lane's 8*KS key bytes are contiguous: lane l holds
// dims [8*KS*(l/16) + 8*ks, +8) of k-step ks, on both operands.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  // two E4M3 values (bytes 2*HI, 2*HI + 1 of w) -> two bf16 in one instruction
  // (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, E4M3 fits bf16)
  typedef __bf16 b2v __attribute__((ext_vector_type(2)));
  const b2v r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

template <int D, int G, int P>
__global__ __launch_bounds__(256, 1) void decode_fp8_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const float* __restrict__ ksc, const float* __restrict__ vsc, int sstride,
    const int32_t* __restrict__ idx, int n_keep, int Hq, int Hkv, int N, int stride,
    float scale_log2, int bps, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int KS = D / 32;  // QK k-steps over the head dim
  constexpr int KB = KS / 2;  // 16-byte key loads per lane per tile
  constexpr int VW = D / 64;  // 4-byte words of a V row per lane (16 lanes span the row)
  constexpr int NC = D / 16;
  static_assert(G <= 16 && D % 64 == 0, "16 heads per MFMA tile, head dim a multiple of 64");
  __shared__ __align__(16) uint2 vt_lds[DEC_WAVES][D * 4];
  __shared__ __align__(16) float m_lds[DEC_WAVES][G][2];
  __shared__ __align__(16) float o_lds[DEC_WAVES][G][D];

  const int split = blockIdx.x;
  const int pair = blockIdx.y;
  const int b = pair / Hkv, kvh = pair % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, j4 = lane >> 4;

  // q^T fragments in the permuted k order
  uint4 qf[KS];
  {
    const uint4* qs = reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + (int64_t)kvh * G) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = (l16 < G) ? qs[l16 * (D / 8) + j4 * KS + ks] : make_uint4(0, 0, 0, 0);
  }

  const int blk0 = split * bps;
  const int32_t* list = idx + (int64_t)pair * n_keep + blk0;
  const int nblk = split_blocks(list, n_keep, blk0, bps);
  const uint8_t* kb = k + (int64_t)pair * stride * D;
  const uint8_t* vb = v + (int64_t)pair * stride * D;
  const float* ks_row = ksc + (int64_t)pair * sstride;
  const float* vs_row = vsc + (int64_t)pair * sstride;
  const int tile0 = 16 * wave;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4v acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = f32x4v{0.f, 0.f, 0.f, 0.f};

  // K: token l16, bytes 8*KS*j4 .. ; V: rows 4*j4 + r, bytes 4*VW*l16 .. +4*VW
  uint4 kbuf[P][KB];
  uint32_t vbuf[P][4][VW];
  float skb[P], svb[P];
  // Dummy loads (j >= nblk) use block 0's scales and a K/V offset masked to
  // an opaque lane-varying zero, computed without a branch: with a provably
  // uniform address the compiler turns the dummy into a scalar load on a
  // path of its own, and the wait counts after the merge then keep too few
  // tiles in flight.
  int vzero = 0;
  asm volatile("" : "+v"(vzero));
  auto issue = [&](int slot, int j) {
    const uint32_t m = (j < nblk) ? 0xffffffffu : 0u;  // uniform
    // clamped to a valid block as in the bf16 kernel (rows and scales)
    const int blk = min(max(list[max(min(j, nblk - 1), 0)], 0), (N - 1) >> 6) & (int)m;
    const int t0 = blk * 64 + tile0;
    const uint32_t koff = (((uint32_t)min(t0 + l16, N - 1) * D + j4 * (8 * KS)) & m) + vzero;
#pragma unroll
    for (int u = 0; u < KB; ++u)
      kbuf[slot][u] = ld_stream(reinterpret_cast<const uint4*>(kb + koff + ((u * 16) & m)));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t voff =
          (((uint32_t)min(t0 + 4 * j4 + r, N - 1) * D + l16 * (4 * VW)) & m) + vzero;
      if constexpr (VW == 2) {
        const uint2 w = ld_stream(reinterpret_cast<const uint2*>(vb + voff));
        vbuf[slot][r][0] = w.x;
        vbuf[slot][r][1] = w.y;
      } else {
        vbuf[slot][r][0] = *reinterpret_cast<const uint32_t*>(vb + voff);
      }
    }
    // vector loads (the opaque zero keeps them off the scalar unit): they
    // retire in order with this tile's K/V loads, whereas a scalar load
    // would make every later LDS wait also wait for it
    skb[slot] = ks_row[blk + vzero];
    svb[slot] = vs_row[blk + vzero];
  };
  uint2* vt = vt_lds[wave];
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
    // V^T: per pair of columns (2p, 2p+1) of a word, gather the 4 tokens'
    // bytes (tokens 0,1 and 2,3), then decode each byte pair to a bf16 pair
#pragma unroll
    for (int w = 0; w < VW; ++w)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const uint32_t sel = pp ? 0x07030602u : 0x05010400u;
        const uint32_t t01 = __builtin_amdgcn_perm(vbuf[slot][1][w], vbuf[slot][0][w], sel);
        const uint32_t t23 = __builtin_amdgcn_perm(vbuf[slot][3][w], vbuf[slot][2][w], sel);
        const int col = 4 * (VW * l16 + w) + 2 * pp;
        vt[vt_row(col) * 4 + j4] =
            make_uint2(fp8x2_to_bf16x2<false>(t01), fp8x2_to_bf16x2<false>(t23));
        vt[vt_row(col + 1) * 4 + j4] =
            make_uint2(fp8x2_to_bf16x2<true>(t01), fp8x2_to_bf16x2<true>(t23));
      }
    wave_lds_sync();
    // the block's K scale folds into the logits, its V scale into the weights
    softmax_pv<NC>(sc, scale_log2 * skb[slot], N - (t0 + 4 * j4), svb[slot], vt, l16, j4, m_run,
                   l_run, acc);
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
  decode_finish<D, G>(m_run, l_run, acc, m_lds, o_lds, wave, tid,
                      ((int64_t)pair * n_splits + split) * G, part_o, part_ml);
}

// Exact merge of the splits of one (batch, query head): M = max m_s,
// L = sum 2^(m_s - M) l_s, o = sum 2^(m_s - M) o_s / L, lse = (M + log2 L) ln 2.
// One workgroup of D threads (one value column each) per (batch, query head).
// The first MERGE_CHUNK splits' columns are requested together with the
// (m, l) pairs (lane s of every wave holds split s), so the common case is a
// single memory round trip; the split weights reach the columns by
// cross-lane reads, with no LDS and no barrier.  A separate launch: the
// kernel boundary makes the partials of all workgroups visible (an
// agent-scope fence per workgroup is far more costly on a multi-XCD part).
constexpr int MERGE_CHUNK = 16;

template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         int G, int Hq, int Hkv, int S,
                                                         float* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq;
  const int pair = b * Hkv + h / G, hh = h % G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t r0 = (int64_t)pair * S * G + hh;  // row of split s: r0 + s * G
  const float2* ml2 = reinterpret_cast<const float2*>(part_ml);
  float ov[MERGE_CHUNK];
#pragma unroll
  for (int i = 0; i < MERGE_CHUNK; ++i)
    ov[i] = (i < S) ? part_o[(r0 + (int64_t)i * G) * D + tid] : 0.f;
  // the first 64 splits' (m, l) stay in registers for the weights below
  const float2 ml0 = (lane < S) ? ml2[r0 + (int64_t)lane * G] : make_float2(-INFINITY, 0.f);
  float M = ml0.x;
  for (int s2 = lane + 64; s2 < S; s2 += 64) M = fmaxf(M, ml2[r0 + (int64_t)s2 * G].x);
  M = wave_max(M);
  float L = 0.f, o = 0.f;
  for (int sb = 0; sb < S; sb += 64) {
    const int s2 = sb + lane;
    float w = 0.f;
    if (s2 < S) {
      const float2 ml = (sb == 0) ? ml0 : ml2[r0 + (int64_t)s2 * G];
      w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      L = fmaf(w, ml.y, L);
    }
    const int ns = min(64, S - sb);
    for (int cb = 0; cb < ns; cb += MERGE_CHUNK) {
      if (sb + cb > 0) {  // later chunks (more than MERGE_CHUNK splits)
#pragma unroll
        for (int i = 0; i < MERGE_CHUNK; ++i)
          ov[i] = (cb + i < ns) ? part_o[(r0 + (int64_t)(sb + cb + i) * G) * D + tid] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < MERGE_CHUNK; ++i)
        o = fmaf(readlane(w, min(cb + i, 63)), ov[i], o);  // ov is 0 past the splits
    }
  }
  L = wave_sum(L);
  out[(int64_t)bh * D + tid] = o / L;
  if (lse && tid == 0) lse[bh] = (M + log2f(L)) * LN2;
}

// The plan aims at one round of 256 workgroups, one per CU of the MI355X:
// splits per pair = round(256 / pairs), each split a contiguous run of the
// kept-block list; more pairs than that, one split per pair.  Two workgroups
// of 4 waves would fit per CU, but measured, one longer split per CU is
// faster at every shape (128K: 40.1 against 41.7 us for S4; 1M: 72.6 against
// 74.2): each workgroup pays its start-up (list, then first-tile latency) and
// its epilogue once over twice the blocks, and the merge reads half the
// partials.  A round that is not whole (384 or 640 workgroups) is slower still.
constexpr int DEC_TARGET_WGS = 256;

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

// partials at the front of the workspace: [pairs][splits][g][2] (m, l), then
// [pairs][splits][g][d] o
struct DecodeWs {
  float* ml;
  float* o;
};
static DecodeWs decode_ws(float* ws, int64_t pairs, int d, const DecodePlan& p) {
  return {ws, ws + (size_t)pairs * p.n_splits * p.g * 2};
}

template <int D, int G>
static void launch_partials_t(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int N,
                              int stride, float scale, const DecodePlan& plan, float* ws,
                              hipStream_t st) {
  const int64_t pairs = (int64_t)B * Hkv;
  const DecodeWs w = decode_ws(ws, pairs, D, plan);
  dim3 grid(plan.n_splits, (unsigned)pairs);
  decode_kernel<D, G, DEC_STAGES><<<grid, 256, 0, st>>>(
      q, k, v, idx, n_keep, Hq, Hkv, N, stride, scale * LOG2E, plan.bps, plan.n_splits, w.o,
      w.ml);
}

template <int D, int G>
static void launch_select_partials_t(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const FusedSelect& fs, int n_keep, int B, int Hq, int Hkv,
                                     int N, int stride, float scale, const DecodePlan& plan,
                                     float* ws, hipStream_t st) {
  const int64_t pairs = (int64_t)B * Hkv;
  const DecodeWs w = decode_ws(ws, pairs, D, plan);
  dim3 grid(plan.n_splits, (unsigned)pairs);
  if (fs.c1 - fs.c0 <= 256 * 8)  // 8 candidates per thread, else 16
    decode_kernel<D, G, DEC_STAGES, 8><<<grid, 256, 0, st>>>(
        q, k, v, nullptr, n_keep, Hq, Hkv, N, stride, scale * LOG2E, plan.bps, plan.n_splits,
        w.o, w.ml, fs);
  else
    decode_kernel<D, G, DEC_STAGES, DEC_SEL_KPT><<<grid, 256, 0, st>>>(
        q, k, v, nullptr, n_keep, Hq, Hkv, N, stride, scale * LOG2E, plan.bps, plan.n_splits,
        w.o, w.ml, fs);
}

template <int D, int G>
static void launch_partials_fp8_t(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                                  const float* ksc, const float* vsc, int sstride,
                                  const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int N,
                                  int stride, float scale, const DecodePlan& plan, float* ws,
                                  hipStream_t st) {
  const int64_t pairs = (int64_t)B * Hkv;
  const DecodeWs w = decode_ws(ws, pairs, D, plan);
  dim3 grid(plan.n_splits, (unsigned)pairs);
  decode_fp8_kernel<D, G, DEC_STAGES_FP8><<<grid, 256, 0, st>>>(
      q, k, v, ksc, vsc, sstride, idx, n_keep, Hq, Hkv, N, stride, scale * LOG2E, plan.bps,
      plan.n_splits, w.o, w.ml);
}

void launch_decode_merge(int B, int Hq, int Hkv, int d, const DecodePlan& plan, const float* ws,
                         float* out, float* lse, hipStream_t st) {
  const DecodeWs w = decode_ws(const_cast<float*>(ws), (int64_t)B * Hkv, d, plan);
  if (d == 128)
    decode_merge_kernel<128><<<(unsigned)(B * Hq), 128, 0, st>>>(w.o, w.ml, plan.g, Hq, Hkv,
                                                                 plan.n_splits, out, lse);
  else
    decode_merge_kernel<64><<<(unsigned)(B * Hq), 64, 0, st>>>(w.o, w.ml, plan.g, Hq, Hkv,
                                                               plan.n_splits, out, lse);
}

bool decode_select_fusable(int d, int g, int n_cand, int n_keep) {
  return d == 128 && n_cand <= DEC_SEL_MAX_CAND && n_keep <= DEC_SEL_MAX_KEEP &&
         (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
}

void launch_decode_select_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const float* scores, int nb, int c0, int c1, int top_k,
                                   int32_t* idx_out, int n_keep, int B, int Hq, int Hkv, int N,
                                   int stride, float scale, const DecodePlan& plan, float* ws,
                                   hipStream_t st) {
  const FusedSelect fs{scores, nb, c0, c1, top_k, idx_out};
#define BSA_DEC(GG)                                                                            \
  if (plan.g == GG)                                                                            \
    return launch_select_partials_t<128, GG>(q, k, v, fs, n_keep, B, Hq, Hkv, N, stride, scale, \
                                             plan, ws, st);
  BSA_DEC(1) BSA_DEC(2) BSA_DEC(4) BSA_DEC(8) BSA_DEC(16)
#undef BSA_DEC
}

void launch_decode_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int d, int N,
                            int stride, float scale, const DecodePlan& plan, float* ws,
                            hipStream_t st) {
#define BSA_DEC(DD, GG)                                                                       \
  if (d == DD && plan.g == GG)                                                                \
    return launch_partials_t<DD, GG>(q, k, v, idx, n_keep, B, Hq, Hkv, N, stride, scale, plan, \
                                     ws, st);
  BSA_DEC(128, 1) BSA_DEC(128, 2) BSA_DEC(128, 4) BSA_DEC(128, 8) BSA_DEC(128, 16)
  BSA_DEC(64, 1) BSA_DEC(64, 2) BSA_DEC(64, 4) BSA_DEC(64, 8) BSA_DEC(64, 16)
#undef BSA_DEC
}

void launch_decode_partials_fp8(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                                const float* ksc, const float* vsc, int sstride,
                                const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int d,
                                int N, int stride, float scale, const DecodePlan& plan, float* ws,
                                hipStream_t st) {
#define BSA_DEC(DD, GG)                                                                        \
  if (d == DD && plan.g == GG)                                                                 \
    return launch_partials_fp8_t<DD, GG>(q, k, v, ksc, vsc, sstride, idx, n_keep, B, Hq, Hkv, \
                                         N, stride, scale, plan, ws, st);
  BSA_DEC(128, 1) BSA_DEC(128, 2) BSA_DEC(128, 4) BSA_DEC(128, 8) BSA_DEC(128, 16)
  BSA_DEC(64, 1) BSA_DEC(64, 2) BSA_DEC(64, 4) BSA_DEC(64, 8) BSA_DEC(64, 16)
#undef BSA_DEC
}

}  // namespace bsa
