/* oracle.c -- plain CPU reference of block-summary sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY: the definition the HIP library is checked
 * against.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load it.  It shares no code with the HIP library.
 *
 * Everything is plain loops in fp64 over bf16 inputs.  No blocking, fusion or
 * reordering beyond what each definition below states.
 *
 * Sources (web pages; section names as printed on them):
 *  [KV]  hotdry.top post "claude-opus-long-context-kv-cache-sparse-attention":
 *        section "稀疏注意力与 KV Cache 压缩的工程实现" (64-token blocks as the
 *        unit of scoring and retention, attention-sink block, ~128-token local
 *        window, importance selection of the middle blocks) and the parameter
 *        table under "可落地的配置参数与监控要点" (block 64, 1 sink block,
 *        2 local blocks, 10-20 % kept).
 *  [CSA] "CSA + HCA 混合注意力机制": section 2.1 (scaled dot-product attention
 *        softmax(QK^T/sqrt(d))V), 2.3 (decode chain: append K/V, then read),
 *        4.1 (every m consecutive tokens become one compressed entry, mean
 *        pooling as the parameter-free choice), 4.3 (sliding window of the
 *        last n_win raw tokens), 4.4 (score every block, keep the top-k,
 *        attend over the kept ones only), 5.1/5.2 (m'=128 compression, dense
 *        attention over all compressed entries).
 *  [CMP] "Claude Code压缩上下文窗口的底层原理与性能优化实践", section
 *        关键代码实现 (mean pooling of token groups).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - summary = arithmetic mean of the block's key rows;
 *  - block score = (sum of the group's query heads) . summary, no scale;
 *  - top-k = highest scores, ties broken towards the lower index;
 *  - kept = sink blocks U top-k of the middle U local blocks, ascending;
 *  - keep ratio r: total kept = floor(r*nb + 0.5), k = total - sink - local;
 *  - prefill: streams cover only the P prior tokens; window = [p-W+1, p];
 *    a tile of q_tile consecutive queries shares one branch-A selection;
 *    the three branch outputs are averaged.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

uint16_t oracle_round_bf16(double x) {
  /* direct fp64 -> bf16 rounding (8 significant bits), ties to even */
  if (x == 0.0 || isnan(x) || isinf(x)) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
  }
  double a = fabs(x);
  int e;
  double m = frexp(a, &e);           /* a = m * 2^e, m in [0.5, 1) */
  double r;
  if (e - 1 < -126) {                /* bf16 subnormal: spacing 2^-133 */
    r = ldexp(rint(ldexp(a, 133)), -133);
  } else {
    double s = ldexp(m, 8);          /* [128, 256) */
    double ri = rint(s);             /* default rounding mode: ties to even */
    r = ldexp(ri, e - 8);
  }
  float f = (float)(x < 0 ? -r : r); /* exact: at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

int32_t oracle_num_blocks(int32_t n, int32_t m) {
  if (n < 0 || m <= 0) return -1;
  return (int32_t)(((int64_t)n + m - 1) / m);
}

int32_t oracle_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* candidate range [c0, c1) and |sink U local| for nb blocks */
static void ranges(int32_t nb, int32_t n_sink, int32_t n_local, int32_t* c0, int32_t* c1,
                   int32_t* fixed) {
  int32_t s_end = n_sink < nb ? n_sink : nb;          /* sink = [0, s_end) */
  int32_t l_beg = nb - n_local > 0 ? nb - n_local : 0; /* local = [l_beg, nb) */
  *c0 = s_end;
  *c1 = l_beg > s_end ? l_beg : s_end;
  *fixed = (l_beg > s_end) ? s_end + (nb - l_beg) : nb;
}

static int32_t k_of(int32_t nb, int32_t n_sink, int32_t n_local, int32_t top_k,
                    double keep_ratio, int32_t n_cand) {
  int64_t k;
  if (top_k >= 0)
    k = top_k;
  else
    k = (int64_t)floor(keep_ratio * (double)nb + 0.5) - n_sink - n_local;
  if (k < 0) k = 0;
  if (k > n_cand) k = n_cand;
  return (int32_t)k;
}

int32_t oracle_num_kept(int32_t nb, int32_t n_sink, int32_t n_local, int32_t top_k,
                        double keep_ratio) {
  if (nb < 0 || n_sink < 0 || n_local < 0) return -1;
  int32_t c0, c1, fixed;
  ranges(nb, n_sink, n_local, &c0, &c1, &fixed);
  return fixed + k_of(nb, n_sink, n_local, top_k, keep_ratio, c1 - c0);
}

/* ---- block summaries: [KV] block-level evaluation unit; [CSA] 4.1 mean pool */
int oracle_block_summaries(const uint16_t* x, int32_t B, int32_t H, int32_t N,
                           int32_t stride, int32_t d, int32_t bs, double* out) {
  if (!x || !out || B < 0 || H < 0 || N < 0 || d <= 0 || bs <= 0 || stride < N) return -1;
  int32_t nb = oracle_num_blocks(N, bs);
  int64_t nbh = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < nbh; ++bh) {
    const uint16_t* xs = x + bh * (int64_t)stride * d;
    for (int32_t j = 0; j < nb; ++j) {
      int32_t t0 = j * bs;
      int32_t t1 = t0 + bs < N ? t0 + bs : N;
      double* o = out + (bh * nb + j) * (int64_t)d;
      for (int32_t c = 0; c < d; ++c) {
        double s = 0.0;
        for (int32_t t = t0; t < t1; ++t) s += bf(xs[(int64_t)t * d + c]);
        o[c] = s / (double)(t1 - t0);
      }
    }
  }
  return 0;
}

/* ---- the fp32 summary: [KV] block-level evaluation unit; [CSA] 4.1 mean
 * pool.  The pages fix the mean, not its fp32 evaluation; the reading taken
 * here is the plainest loop: an fp32 running sum in token order, then an fp32
 * division by the count (C on x86-64 evaluates float expressions in float,
 * and the build disables contraction). */
int oracle_block_summaries_f32(const uint16_t* x, int32_t B, int32_t H, int32_t N,
                               int32_t stride, int32_t d, int32_t bs, float* out) {
  if (!x || !out || B < 0 || H < 0 || N < 0 || d <= 0 || bs <= 0 || stride < N) return -1;
  int32_t nb = oracle_num_blocks(N, bs);
  int64_t nbh = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < nbh; ++bh) {
    const uint16_t* xs = x + bh * (int64_t)stride * d;
    for (int32_t j = 0; j < nb; ++j) {
      int32_t t0 = j * bs;
      int32_t t1 = t0 + bs < N ? t0 + bs : N;
      float* o = out + (bh * nb + j) * (int64_t)d;
      for (int32_t c = 0; c < d; ++c) {
        float s = 0.0f;
        for (int32_t t = t0; t < t1; ++t)
          s = s + (float)bf(xs[(int64_t)t * d + c]); /* the conversion is exact */
        o[c] = s / (float)(t1 - t0);
      }
    }
  }
  return 0;
}

/* ---- selection order: higher score first, lower index on equal scores */
typedef struct {
  double s;
  int32_t j;
} scored;

static int by_score_desc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

/* keep the first k of `cand` (n entries) under by_score_desc; marks keep[j] */
static void top_k_mark(scored* cand, int32_t n, int32_t k, unsigned char* keep) {
  qsort(cand, (size_t)n, sizeof(scored), by_score_desc);
  for (int32_t i = 0; i < k; ++i) keep[cand[i].j] = 1;
}

/* ---- [KV] sink + local + importance selection; [CSA] 4.4 score then top-k */
int oracle_select_blocks(const uint16_t* q, const double* summaries, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t d, int32_t nb, int32_t n_sink,
                         int32_t n_local, int32_t top_k, double keep_ratio,
                         int32_t* idx_out, double* scores_out) {
  if (!q || !summaries || !idx_out || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 ||
      nb < 0 || n_sink < 0 || n_local < 0)
    return -1;
  int32_t g = Hq / Hkv;
  int32_t c0, c1, fixed;
  ranges(nb, n_sink, n_local, &c0, &c1, &fixed);
  int32_t k = k_of(nb, n_sink, n_local, top_k, keep_ratio, c1 - c0);
  int32_t n_keep = fixed + k;
  int64_t npair = (int64_t)B * Hkv;
  int bad = 0;
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < npair; ++p) {
    int64_t b = p / Hkv, kvh = p % Hkv;
    double* qbar = (double*)calloc((size_t)d, sizeof(double));
    scored* cand = (scored*)malloc(sizeof(scored) * (size_t)(c1 - c0 + 1));
    unsigned char* keep = (unsigned char*)calloc((size_t)nb + 1, 1);
    /* pooled query: sum over the query heads that read this kv head */
    for (int32_t h = (int32_t)kvh * g; h < (int32_t)kvh * g + g; ++h)
      for (int32_t c = 0; c < d; ++c) qbar[c] += bf(q[(b * Hq + h) * (int64_t)d + c]);
    const double* sm = summaries + p * (int64_t)nb * d;
    for (int32_t j = c0; j < c1; ++j) {
      double s = 0.0;
      for (int32_t c = 0; c < d; ++c) s += qbar[c] * sm[(int64_t)j * d + c];
      cand[j - c0].s = s;
      cand[j - c0].j = j;
    }
    if (scores_out) {
      double* so = scores_out + p * (int64_t)nb;
      for (int32_t j = 0; j < nb; ++j) so[j] = NAN;
      for (int32_t j = c0; j < c1; ++j) so[j] = cand[j - c0].s;
    }
    top_k_mark(cand, c1 - c0, k, keep);
    for (int32_t j = 0; j < nb; ++j)
      if (j < c0 || j >= c1) keep[j] = 1; /* sink and local blocks */
    int32_t w = 0;
    for (int32_t j = 0; j < nb; ++j)
      if (keep[j]) {
        if (w < n_keep) idx_out[p * n_keep + w] = j;
        ++w;
      }
    if (w != n_keep) {
#pragma omp atomic write
      bad = 1;
    }
    free(qbar);
    free(cand);
    free(keep);
  }
  return bad ? -1 : 0;
}

/* ---- [KV] "锚点动态选择" / "动态重要性选择（Top-P Selection）": the sink and
 * local blocks are anchors; the threshold is tau = a_max + margin * (a_max -
 * a_min) over the anchors' scores; k = #(candidates scoring above tau),
 * clamped so that the kept total lies in [ratio_min * nb, ratio_max * nb]
 * (rounded as k_of does); the kept list is sink + top-k + local, ascending,
 * padded with -1 to the widest list. */
int32_t oracle_adaptive_bounds(int32_t nb, int32_t n_sink, int32_t n_local, double ratio_min,
                               double ratio_max, int32_t* k_lo, int32_t* k_hi) {
  if (nb < 0 || n_sink < 0 || n_local < 0 || !(ratio_min >= 0.0) || !(ratio_max >= ratio_min))
    return -1;
  int32_t c0, c1, fixed;
  ranges(nb, n_sink, n_local, &c0, &c1, &fixed);
  int32_t n_cand = c1 - c0;
  int64_t lo = (int64_t)floor(ratio_min * (double)nb + 0.5) - fixed;
  int64_t hi = (int64_t)floor(ratio_max * (double)nb + 0.5) - fixed;
  if (lo < 0) lo = 0;
  if (lo > n_cand) lo = n_cand;
  if (hi < lo) hi = lo;
  if (hi > n_cand) hi = n_cand;
  *k_lo = (int32_t)lo;
  *k_hi = (int32_t)hi;
  return fixed + (int32_t)hi; /* the widest list */
}

int oracle_select_blocks_adaptive(const uint16_t* q, const double* summaries, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t d, int32_t nb, int32_t n_sink,
                                  int32_t n_local, double ratio_min, double ratio_max,
                                  double margin, int32_t* idx_out, int32_t* count_out,
                                  double* scores_out) {
  int32_t k_lo, k_hi;
  int32_t width = oracle_adaptive_bounds(nb, n_sink, n_local, ratio_min, ratio_max, &k_lo, &k_hi);
  if (!q || !summaries || !idx_out || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 ||
      width < 0)
    return -1;
  int32_t g = Hq / Hkv;
  int32_t c0, c1, fixed;
  ranges(nb, n_sink, n_local, &c0, &c1, &fixed);
  int64_t npair = (int64_t)B * Hkv;
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < npair; ++p) {
    int64_t b = p / Hkv, kvh = p % Hkv;
    double* qbar = (double*)calloc((size_t)d, sizeof(double));
    double* sc = (double*)malloc(sizeof(double) * ((size_t)nb + 1));
    scored* cand = (scored*)malloc(sizeof(scored) * (size_t)(c1 - c0 + 1));
    unsigned char* keep = (unsigned char*)calloc((size_t)nb + 1, 1);
    for (int32_t h = (int32_t)kvh * g; h < (int32_t)kvh * g + g; ++h)
      for (int32_t c = 0; c < d; ++c) qbar[c] += bf(q[(b * Hq + h) * (int64_t)d + c]);
    const double* sm = summaries + p * (int64_t)nb * d;
    /* every block is scored: the candidates and the anchors */
    for (int32_t j = 0; j < nb; ++j) {
      double s = 0.0;
      for (int32_t c = 0; c < d; ++c) s += qbar[c] * sm[(int64_t)j * d + c];
      sc[j] = s;
    }
    double a_max = -INFINITY, a_min = INFINITY;
    for (int32_t j = 0; j < nb; ++j)
      if (j < c0 || j >= c1) {
        if (sc[j] > a_max) a_max = sc[j];
        if (sc[j] < a_min) a_min = sc[j];
      }
    /* no anchor block: every candidate counts */
    double tau = fixed > 0 ? a_max + margin * (a_max - a_min) : -INFINITY;
    int32_t above = 0;
    for (int32_t j = c0; j < c1; ++j) {
      cand[j - c0].s = sc[j];
      cand[j - c0].j = j;
      if (sc[j] > tau) ++above;
    }
    int32_t k = above < k_lo ? k_lo : (above > k_hi ? k_hi : above);
    top_k_mark(cand, c1 - c0, k, keep);
    for (int32_t j = 0; j < nb; ++j)
      if (j < c0 || j >= c1) keep[j] = 1;
    int32_t w = 0;
    for (int32_t j = 0; j < nb; ++j)
      if (keep[j]) idx_out[p * width + w++] = j;
    for (; w < width; ++w) idx_out[p * width + w] = -1;
    if (count_out) count_out[p] = fixed + k;
    if (scores_out)
      for (int32_t j = 0; j < nb; ++j) scores_out[p * (int64_t)nb + j] = sc[j];
    free(qbar);
    free(sc);
    free(cand);
    free(keep);
  }
  return 0;
}

/* ---- FP8 KV cache (aicoding.csdn.net page, 二.2 (3) FP8量化与无损压缩; the
 * format is not fixed there: OCP E4M3, one fp32 scale per (pair, block)).
 * E4M3: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no infinities,
 * 0x7F / 0xFF are NaN, the largest finite magnitude 448 = 1.75 * 2^8. */
double oracle_e4m3_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return s ? -v : v;
}

/* the nearest E4M3 code, ties to the even code; magnitudes >= 448 saturate */
uint8_t oracle_e4m3_encode(double y) {
  uint8_t s = signbit(y) ? 0x80 : 0;
  double a = fabs(y);
  if (a >= 448.0) return s | 0x7E;
  if (a == 0.0) return s;
  int e;
  frexp(a, &e);            /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  if (E < -6) E = -6;      /* the subnormal codes share exponent -6's spacing */
  double r = rint(a / ldexp(1.0, E - 3)); /* spacing 2^(E-3): 3 mantissa bits */
  int code;
  if (E == -6 && r < 8.0) {
    code = (int)r;         /* subnormal: exponent field 0 */
  } else {
    if (r >= 16.0) { /* rounded up to the next power of two */
      r = 8.0;
      E += 1;
    }
    code = ((E + 7) << 3) | ((int)r - 8);
  }
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(s | code);
}

/* per (pair, block j): amax = max |x| over the valid tokens; scale = amax /
 * 448 and inv = 448 / amax in fp32; code = E4M3(clamp(x * inv, +-448)) with
 * the product in fp32.  out [B][H][stride][d] (rows < N), scales [B][H][sstride] */
int oracle_quantize_fp8(const uint16_t* x, int32_t B, int32_t H, int32_t N, int32_t stride,
                        int32_t d, int32_t bs, int32_t sstride, uint8_t* out, float* scales) {
  if (!x || !out || !scales || B < 0 || H < 0 || N < 0 || d <= 0 || bs <= 0 || stride < N)
    return -1;
  int32_t nb = oracle_num_blocks(N, bs);
  if (sstride < nb) return -1;
  int64_t np = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t p = 0; p < np; ++p) {
    for (int32_t j = 0; j < nb; ++j) {
      int32_t t0 = j * bs, t1 = t0 + bs < N ? t0 + bs : N;
      float amax = 0.0f;
      for (int32_t t = t0; t < t1; ++t)
        for (int32_t c = 0; c < d; ++c) {
          float a = (float)fabs(bf(x[(p * stride + t) * (int64_t)d + c]));
          if (a > amax) amax = a;
        }
      float sc = amax / 448.0f;
      float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
      for (int32_t t = t0; t < t1; ++t)
        for (int32_t c = 0; c < d; ++c) {
          int64_t o = (p * stride + t) * (int64_t)d + c;
          float y = (float)bf(x[o]) * inv;
          if (y > 448.0f) y = 448.0f;
          if (y < -448.0f) y = -448.0f;
          out[o] = oracle_e4m3_encode((double)y);
        }
      scales[p * sstride + j] = sc;
    }
  }
  return 0;
}

/* exact softmax attention over the kept blocks of a quantized cache: each
 * key / value entry is scale[block] * E4M3(code), in fp64 */
int oracle_sparse_decode_attn_fp8(const uint16_t* q, const uint8_t* k8, const uint8_t* v8,
                                  const float* kscales, const float* vscales, const int32_t* idx,
                                  int32_t n_keep, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                  int32_t N, int32_t stride, int32_t bs, int32_t sstride,
                                  double scale, double* out, double* lse) {
  if (!q || !k8 || !v8 || !kscales || !vscales || !idx || !out || B < 0 || Hq <= 0 ||
      Hkv <= 0 || Hq % Hkv || d <= 0 || N < 1 || stride < N || bs <= 0 || n_keep < 1)
    return -1;
  int32_t g = Hq / Hkv;
  int32_t nb = oracle_num_blocks(N, bs);
  if (sstride < nb) return -1;
  for (int64_t p = 0; p < (int64_t)B * Hkv; ++p) {
    const int32_t* li = idx + p * n_keep;
    int32_t used = n_keep;
    for (int32_t i = 0; i < n_keep; ++i) {
      if (li[i] == -1) {
        used = i;
        break;
      }
      if (li[i] < 0 || li[i] >= nb || (i && li[i] <= li[i - 1])) return -1;
    }
    if (used == 0) return -1;
    for (int32_t i = used; i < n_keep; ++i)
      if (li[i] != -1) return -1;
  }
  if (scale == 0.0) scale = 1.0 / sqrt((double)d);
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = oracle_e4m3_value((uint8_t)c);
  int64_t nqh = (int64_t)B * Hq;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < nqh; ++bh) {
    int64_t b = bh / Hq, h = bh % Hq, kvh = h / g, p = b * Hkv + kvh;
    const int32_t* list = idx + p * n_keep;
    double* z = (double*)malloc(sizeof(double) * ((size_t)n_keep * bs + 1));
    int64_t* row = (int64_t*)malloc(sizeof(int64_t) * ((size_t)n_keep * bs + 1));
    double* vs = (double*)malloc(sizeof(double) * ((size_t)n_keep * bs + 1));
    int32_t n = 0;
    double zmax = -INFINITY;
    for (int32_t i = 0; i < n_keep && list[i] >= 0; ++i) {
      int32_t blk = list[i], t0 = blk * bs, t1 = t0 + bs < N ? t0 + bs : N;
      double ks = (double)kscales[p * sstride + blk];
      for (int32_t t = t0; t < t1; ++t) {
        const uint8_t* kr = k8 + (p * stride + t) * (int64_t)d;
        double sdot = 0.0;
        for (int32_t c = 0; c < d; ++c) sdot += bf(q[bh * d + c]) * (ks * lut[kr[c]]);
        z[n] = sdot * scale;
        row[n] = (p * stride + t) * (int64_t)d;
        vs[n] = (double)vscales[p * sstride + blk];
        if (z[n] > zmax) zmax = z[n];
        ++n;
      }
    }
    double l = 0.0;
    for (int32_t t = 0; t < n; ++t) {
      z[t] = exp(z[t] - zmax);
      l += z[t];
    }
    double* o = out + bh * d;
    for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int32_t t = 0; t < n; ++t) {
      double pw = z[t] / l;
      for (int32_t c = 0; c < d; ++c) o[c] += pw * (vs[t] * lut[v8[row[t] + c]]);
    }
    if (lse) lse[bh] = zmax + log(l);
    free(z);
    free(row);
    free(vs);
  }
  return 0;
}

/* ---- [CSA] 2.1 / 4.4: exact softmax(q K^T / sqrt(d)) V over a token list.
 * Writes o[d] and returns lse; w (optional) receives the weights. */
static double attend(const uint16_t* qh, const double* qd, int32_t d, int32_t n,
                     const int64_t* rows_k, const int64_t* rows_v, const uint16_t* kb,
                     const uint16_t* vb, const float* kf, const float* vf, double scale,
                     double* z, double* o, double* w) {
  /* z_t = scale * q . K_t */
  double zmax = -INFINITY;
  for (int32_t t = 0; t < n; ++t) {
    double s = 0.0;
    for (int32_t c = 0; c < d; ++c) {
      double qc = qh ? bf(qh[c]) : qd[c];
      double kc = kb ? bf(kb[rows_k[t] + c]) : (double)kf[rows_k[t] + c];
      s += qc * kc;
    }
    z[t] = s * scale;
    if (z[t] > zmax) zmax = z[t];
  }
  double l = 0.0;
  for (int32_t t = 0; t < n; ++t) {
    z[t] = exp(z[t] - zmax);
    l += z[t];
  }
  for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
  for (int32_t t = 0; t < n; ++t) {
    double p = z[t] / l;
    if (w) w[t] = p;
    for (int32_t c = 0; c < d; ++c) {
      double vc = vb ? bf(vb[rows_v[t] + c]) : (double)vf[rows_v[t] + c];
      o[c] += p * vc;
    }
  }
  return zmax + log(l);
}

int oracle_sparse_decode_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, int32_t n_keep, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t d, int32_t N, int32_t stride,
                              int32_t bs, double scale, double* out, double* lse,
                              double* weights) {
  if (!q || !k || !v || !idx || !out || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv ||
      d <= 0 || N < 0 || stride < N || bs <= 0 || n_keep < 0)
    return -1;
  int32_t g = Hq / Hkv;
  int32_t nb = oracle_num_blocks(N, bs);
  /* each list: ascending block indices without repeats, optionally ended by
   * a run of -1 (the absent entries of an adaptive selection), >= 1 block */
  for (int64_t p = 0; p < (int64_t)B * Hkv && n_keep > 0; ++p) {
    const int32_t* li = idx + p * n_keep;
    int32_t used = n_keep;
    for (int32_t i = 0; i < n_keep; ++i) {
      if (li[i] == -1) {
        used = i;
        break;
      }
      if (li[i] < 0 || li[i] >= nb) return -1;
      if (i && li[i] <= li[i - 1]) return -1;
    }
    if (used == 0) return -1;
    for (int32_t i = used; i < n_keep; ++i)
      if (li[i] != -1) return -1;
  }
  if (scale == 0.0) scale = 1.0 / sqrt((double)d);
  int64_t nqh = (int64_t)B * Hq;
#pragma omp parallel for schedule(dynamic)
  for (int64_t bh = 0; bh < nqh; ++bh) {
    int64_t b = bh / Hq, h = bh % Hq, kvh = h / g;
    const int32_t* list = idx + (b * Hkv + kvh) * (int64_t)n_keep;
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * ((size_t)n_keep * bs + 1));
    int32_t* slot = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n_keep * bs + 1));
    double* z = (double*)malloc(sizeof(double) * ((size_t)n_keep * bs + 1));
    double* wt = (double*)malloc(sizeof(double) * ((size_t)n_keep * bs + 1));
    int32_t n = 0;
    int64_t base = (b * Hkv + kvh) * (int64_t)stride * d;
    for (int32_t i = 0; i < n_keep && list[i] >= 0; ++i) {
      int32_t t0 = list[i] * bs;
      int32_t t1 = t0 + bs < N ? t0 + bs : N;
      for (int32_t t = t0; t < t1; ++t) {
        rows[n] = base + (int64_t)t * d;
        slot[n] = i * bs + (t - t0);
        ++n;
      }
    }
    double l = attend(q + bh * d, NULL, d, n, rows, rows, k, v, NULL, NULL, scale, z,
                      out + bh * d, wt);
    if (lse) lse[bh] = l;
    if (weights) {
      double* wo = weights + bh * (int64_t)n_keep * bs;
      for (int64_t i = 0; i < (int64_t)n_keep * bs; ++i) wo[i] = 0.0;
      for (int32_t t = 0; t < n; ++t) wo[slot[t]] = wt[t];
    }
    free(rows);
    free(slot);
    free(z);
    free(wt);
  }
  return 0;
}

/* ---- chunked prefill: [CSA] 4.1-4.4 (branch A), 5.1-5.2 (branch B),
 * 4.3 (branch C); outputs averaged. */
int oracle_sparse_prefill_attn(const uint16_t* q, int32_t C, const uint16_t* k,
                               const uint16_t* v, int32_t B, int32_t P, int32_t Hq,
                               int32_t Hkv, int32_t d, int32_t stride, int32_t m_sparse,
                               int32_t top_k, int32_t m_dense, int32_t window,
                               int32_t q_tile, double scale, const int32_t* sel_in,
                               const int32_t* rows, int32_t n_rows, int32_t combine,
                               int32_t indexer, const double* sink_logits, double* out,
                               double* branch_out, double* lse3, int32_t* sel_out,
                               double* sel_scores) {
  if (!q || !k || !v || !out || C <= 0 || B <= 0 || P < 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv || d <= 0 || stride < P + C || m_sparse <= 0 || top_k < 0 || m_dense <= 0 ||
      window <= 0 || q_tile <= 0 || d > 512 || (combine != 0 && combine != 1) ||
      (indexer != 0 && indexer != 1))
    return -1;
  if (!rows) n_rows = C;
  if (n_rows < 0) return -1;
  for (int32_t r = 0; rows && r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= C) return -1;
  if (scale == 0.0) scale = 1.0 / sqrt((double)d);
  int32_t g = Hq / Hkv;
  int32_t E4 = oracle_num_blocks(P, m_sparse);
  int32_t E128 = oracle_num_blocks(P, m_dense);
  int32_t kk = top_k < E4 ? top_k : E4;
  int32_t n_tiles = oracle_num_blocks(C, q_tile);
  int64_t npair = (int64_t)B * Hkv;
  if (sel_in)
    for (int64_t i = 0; i < (int64_t)B * n_tiles * Hkv * kk; ++i)
      if (sel_in[i] < 0 || sel_in[i] >= E4) return -1;

  /* compressed streams over the prior tokens: bf16-rounded means for
   * attention (the stored compressed cache is bf16); the scoring keys below */
  double* ks_exact = (double*)malloc(sizeof(double) * (size_t)(npair * E4 * d + 1));
  double* tmp4 = (double*)malloc(sizeof(double) * (size_t)(npair * E4 * d + 1));
  double* tmp128 = (double*)malloc(sizeof(double) * (size_t)(npair * E128 * d + 1));
  float* k4 = (float*)malloc(sizeof(float) * (size_t)(npair * E4 * d + 1));
  float* v4 = (float*)malloc(sizeof(float) * (size_t)(npair * E4 * d + 1));
  float* k128 = (float*)malloc(sizeof(float) * (size_t)(npair * E128 * d + 1));
  float* v128 = (float*)malloc(sizeof(float) * (size_t)(npair * E128 * d + 1));
  oracle_block_summaries(k, B, Hkv, P, stride, d, m_sparse, ks_exact);
  for (int64_t i = 0; i < npair * E4 * d; ++i) k4[i] = (float)bf(oracle_round_bf16(ks_exact[i]));
  oracle_block_summaries(v, B, Hkv, P, stride, d, m_sparse, tmp4);
  for (int64_t i = 0; i < npair * E4 * d; ++i) v4[i] = (float)bf(oracle_round_bf16(tmp4[i]));
  oracle_block_summaries(k, B, Hkv, P, stride, d, m_dense, tmp128);
  for (int64_t i = 0; i < npair * E128 * d; ++i) k128[i] = (float)bf(oracle_round_bf16(tmp128[i]));
  oracle_block_summaries(v, B, Hkv, P, stride, d, m_dense, tmp128);
  for (int64_t i = 0; i < npair * E128 * d; ++i) v128[i] = (float)bf(oracle_round_bf16(tmp128[i]));
  free(tmp4);
  free(tmp128);
  /* the keys the selection scores against ([CSA] 4.2: the indexer scores the
   * compressed entries, at low precision, its recall measured against a BF16
   * indexer).  indexer 0: the bf16 compressed keys as the stream holds them,
   * the bf16 rounding (ties to even) of the fp32 mean in token order;
   * indexer 1: the exact means */
  double* ks_b16 = NULL;
  if (indexer == 0) {
    float* f32 = (float*)malloc(sizeof(float) * (size_t)(npair * E4 * d + 1));
    ks_b16 = (double*)malloc(sizeof(double) * (size_t)(npair * E4 * d + 1));
    oracle_block_summaries_f32(k, B, Hkv, P, stride, d, m_sparse, f32);
    for (int64_t i = 0; i < npair * E4 * d; ++i) ks_b16[i] = bf(oracle_round_bf16((double)f32[i]));
    free(f32);
  }
  const double* keys = indexer == 0 ? ks_b16 : ks_exact;

  /* which tiles need a selection: all of them when the selection or its
   * scores are requested, else those holding a requested row (unless the
   * caller supplies the selection) */
  unsigned char* need = (unsigned char*)calloc((size_t)B * n_tiles + 1, 1);
  for (int64_t i = 0; i < (int64_t)B * n_tiles; ++i) need[i] = (sel_out || sel_scores) ? 1 : 0;
  if (!sel_in)
    for (int32_t b = 0; b < B; ++b)
      for (int32_t r = 0; r < n_rows; ++r) need[b * n_tiles + (rows ? rows[r] : r) / q_tile] = 1;
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)((int64_t)B * n_tiles * Hkv * kk + 1));
  int64_t nprob = (int64_t)B * n_tiles * Hkv;
#pragma omp parallel for schedule(dynamic)
  for (int64_t pr = 0; pr < nprob; ++pr) {
    int64_t b = pr / ((int64_t)n_tiles * Hkv);
    int64_t tile = (pr / Hkv) % n_tiles, kvh = pr % Hkv;
    if (!need[b * n_tiles + tile]) continue;
    double* qbar = (double*)calloc((size_t)d, sizeof(double));
    scored* cand = (scored*)malloc(sizeof(scored) * ((size_t)E4 + 1));
    unsigned char* keep = (unsigned char*)calloc((size_t)E4 + 1, 1);
    int32_t i0 = (int32_t)tile * q_tile;
    int32_t i1 = i0 + q_tile < C ? i0 + q_tile : C;
    /* pooled query of the tile: every (query, head) pair reading this kv head */
    for (int32_t i = i0; i < i1; ++i)
      for (int32_t h = (int32_t)kvh * g; h < (int32_t)kvh * g + g; ++h)
        for (int32_t c = 0; c < d; ++c)
          qbar[c] += bf(q[(((int64_t)b * C + i) * Hq + h) * d + c]);
    const double* ks = keys + (b * Hkv + kvh) * (int64_t)E4 * d;
    for (int32_t j = 0; j < E4; ++j) {
      double s = 0.0;
      for (int32_t c = 0; c < d; ++c) s += qbar[c] * ks[(int64_t)j * d + c];
      cand[j].s = s;
      cand[j].j = j;
      if (sel_scores) sel_scores[pr * E4 + j] = s;
    }
    top_k_mark(cand, E4, kk, keep);
    int32_t w = 0;
    for (int32_t j = 0; j < E4; ++j)
      if (keep[j]) sel[pr * kk + w++] = j;
    if (sel_out) memcpy(sel_out + pr * kk, sel + pr * kk, sizeof(int32_t) * (size_t)kk);
    free(qbar);
    free(cand);
    free(keep);
  }
  const int32_t* use = sel_in ? sel_in : sel;

  int64_t nwork = (int64_t)B * n_rows * Hq;
  int32_t maxn = kk;
  if (E128 > maxn) maxn = E128;
  if (window > maxn) maxn = window;
  int32_t max_all = kk + E128 + window + 1; /* concatenated logits (+ the sink) */
#pragma omp parallel for schedule(dynamic)
  for (int64_t wi = 0; wi < nwork; ++wi) {
    int64_t b = wi / ((int64_t)n_rows * Hq);
    int32_t r = (int32_t)((wi / Hq) % n_rows);
    int32_t h = (int32_t)(wi % Hq), kvh = h / g;
    int32_t i = rows ? rows[r] : r;
    int32_t tile = i / q_tile;
    const uint16_t* qh = q + (((int64_t)b * C + i) * Hq + h) * d;
    int64_t* rk = (int64_t*)malloc(sizeof(int64_t) * ((size_t)maxn + 1));
    double* z = (double*)malloc(sizeof(double) * ((size_t)maxn + 1));
    double o[3][512];
    double l[3];
    int64_t pair = b * Hkv + kvh;
    /* branch A: the tile's selected m_sparse entries */
    const int32_t* list = use + ((b * n_tiles + tile) * Hkv + kvh) * (int64_t)kk;
    for (int32_t t = 0; t < kk; ++t) rk[t] = (pair * E4 + list[t]) * (int64_t)d;
    l[0] = attend(qh, NULL, d, kk, rk, rk, NULL, NULL, k4, v4, scale, z, o[0], NULL);
    /* branch B: every m_dense entry */
    for (int32_t t = 0; t < E128; ++t) rk[t] = (pair * E128 + t) * (int64_t)d;
    l[1] = attend(qh, NULL, d, E128, rk, rk, NULL, NULL, k128, v128, scale, z, o[1], NULL);
    /* branch C: raw tokens [p - window + 1, p], p = P + i */
    int32_t p = P + i;
    int32_t t0 = p - window + 1 > 0 ? p - window + 1 : 0;
    int32_t n = 0;
    for (int32_t t = t0; t <= p; ++t) rk[n++] = (pair * stride + t) * (int64_t)d;
    l[2] = attend(qh, NULL, d, n, rk, rk, k, v, NULL, NULL, scale, z, o[2], NULL);
    double* dst = out + wi * d;
    int has_sink = sink_logits != NULL;
    double zs = has_sink ? sink_logits[h] : 0.0;
    if (combine == 0) {
      /* average of the three branch outputs; with a sink logit each branch's
       * softmax also holds one extra logit zs whose value vector is zero
       * ("CSA + HCA 混合注意力机制" §5.4) */
      for (int32_t c = 0; c < d; ++c) dst[c] = 0.0;
      for (int32_t br = 0; br < 3; ++br) {
        double keep = has_sink ? 1.0 / (1.0 + exp(zs - l[br])) : 1.0;
        for (int32_t c = 0; c < d; ++c) dst[c] += o[br][c] * keep;
      }
      for (int32_t c = 0; c < d; ++c) dst[c] /= 3.0;
    } else {
      /* one softmax over the concatenated logits of A, B and C (and the sink
       * logit, value zero): §4.3 attends the compressed entries, the window
       * and the tail together */
      int64_t* rka = (int64_t*)malloc(sizeof(int64_t) * ((size_t)max_all + 1));
      double* za = (double*)malloc(sizeof(double) * ((size_t)max_all + 1));
      int32_t src[3] = {0, 0, 0}, na = 0;
      /* logits of each branch in order */
      for (int32_t t = 0; t < kk; ++t) rka[na++] = (pair * E4 + list[t]) * (int64_t)d;
      src[0] = na;
      for (int32_t t = 0; t < E128; ++t) rka[na++] = (pair * E128 + t) * (int64_t)d;
      src[1] = na;
      for (int32_t t = t0; t <= p; ++t) rka[na++] = (pair * stride + t) * (int64_t)d;
      src[2] = na;
      double zmax = has_sink ? zs : -INFINITY;
      for (int32_t t = 0; t < na; ++t) {
        double sdot = 0.0;
        for (int32_t c = 0; c < d; ++c) {
          double kc = t < src[0]   ? (double)k4[rka[t] + c]
                      : t < src[1] ? (double)k128[rka[t] + c]
                                   : bf(k[rka[t] + c]);
          sdot += bf(qh[c]) * kc;
        }
        za[t] = sdot * scale;
        if (za[t] > zmax) zmax = za[t];
      }
      double den = has_sink ? exp(zs - zmax) : 0.0;
      for (int32_t t = 0; t < na; ++t) {
        za[t] = exp(za[t] - zmax);
        den += za[t];
      }
      for (int32_t c = 0; c < d; ++c) dst[c] = 0.0;
      for (int32_t t = 0; t < na; ++t) {
        double pw = za[t] / den;
        for (int32_t c = 0; c < d; ++c) {
          double vc = t < src[0]   ? (double)v4[rka[t] + c]
                      : t < src[1] ? (double)v128[rka[t] + c]
                                   : bf(v[rka[t] + c]);
          dst[c] += pw * vc;
        }
      }
      free(rka);
      free(za);
    }
    int64_t nb3 = (int64_t)B * n_rows * Hq;
    for (int32_t br = 0; br < 3; ++br) {
      if (branch_out)
        for (int32_t c = 0; c < d; ++c) branch_out[(br * nb3 + wi) * d + c] = o[br][c];
      if (lse3) lse3[br * nb3 + wi] = l[br];
    }
    free(rk);
    free(z);
  }
  free(need);
  free(sel);
  free(ks_exact);
  free(ks_b16);
  free(k4);
  free(v4);
  free(k128);
  free(v128);
  return 0;
}
