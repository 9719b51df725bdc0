/* oracle.h -- plain CPU reference of block-summary sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and oracle.c are the slow, obviously
 * correct definition that the HIP library is checked against.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Inputs are bf16 bit patterns (uint16_t); every computation is carried out in
 * fp64 (except oracle_block_summaries_f32, which states its fp32 steps);
 * outputs are fp64.  Layouts (row-major):
 *   q (decode)   [B][Hq][d]
 *   q (prefill)  [B][C][Hq][d]
 *   K, V         [B][Hkv][stride][d]   (stride = cache capacity in tokens)
 * Query head h reads kv head h / (Hq/Hkv).
 *
 * Return value: 0 on success, -1 on an invalid argument (nothing is written).
 */
#ifndef BSA_ORACLE_H
#define BSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* number of blocks (or compressed entries) covering n tokens: ceil(n / m) */
int32_t oracle_num_blocks(int32_t n, int32_t m);

/* kept-block count for nb blocks: |sink U local| + k (see oracle.c) */
int32_t oracle_num_kept(int32_t nb, int32_t n_sink, int32_t n_local, int32_t top_k,
                        double keep_ratio);

/* threads the oracle's parallel loops use, and a way to change it (n >= 1) */
int32_t oracle_num_threads(void);
void oracle_set_threads(int32_t n);

/* block summaries: out[b][h][j][c] = mean of x over the tokens of block j */
int oracle_block_summaries(const uint16_t* x, int32_t B, int32_t H, int32_t N,
                           int32_t stride, int32_t d, int32_t bs, double* out);

/* the same mean as a stored fp32 summary: the block's values added one token
 * at a time in fp32 (ascending token order, from 0), then one correctly
 * rounded fp32 division by the token count.  The one place the oracle works
 * in fp32: it fixes the fp32 summary bit for bit. */
int oracle_block_summaries_f32(const uint16_t* x, int32_t B, int32_t H, int32_t N,
                               int32_t stride, int32_t d, int32_t bs, float* out);

/* per (b, kv head) block selection; idx_out [B][Hkv][n_keep] ascending,
 * scores_out [B][Hkv][nb] (candidates only; others set to NaN) or NULL */
int oracle_select_blocks(const uint16_t* q, const double* summaries, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t d, int32_t nb, int32_t n_sink,
                         int32_t n_local, int32_t top_k, double keep_ratio,
                         int32_t* idx_out, double* scores_out);

/* anchor-adaptive selection: tau = a_max + margin * (a_max - a_min) over the
 * scores of the sink and local (anchor) blocks; k = #(candidates scoring above
 * tau) clamped to [k_lo, k_hi], where the kept totals ratio_min * nb and
 * ratio_max * nb are rounded as for keep_ratio; kept = sink + top-k + local,
 * ascending, padded with -1 to the widest list (returned by
 * oracle_adaptive_bounds, which also gives k_lo and k_hi; -1 on bad input).
 * idx_out [B][Hkv][width]; count_out [B][Hkv] or NULL; scores_out [B][Hkv][nb]
 * (every block) or NULL.  Without anchor blocks every candidate counts. */
int32_t oracle_adaptive_bounds(int32_t nb, int32_t n_sink, int32_t n_local, double ratio_min,
                               double ratio_max, int32_t* k_lo, int32_t* k_hi);
int oracle_select_blocks_adaptive(const uint16_t* q, const double* summaries, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t d, int32_t nb, int32_t n_sink,
                                  int32_t n_local, double ratio_min, double ratio_max,
                                  double margin, int32_t* idx_out, int32_t* count_out,
                                  double* scores_out);

/* exact softmax attention over the tokens of the listed blocks.
 * idx [B][Hkv][n_keep] (a list may end in a run of -1: absent entries);
 * out [B][Hq][d]; lse [B][Hq] or NULL;
 * weights [B][Hq][n_keep*bs] or NULL (softmax weight of each listed token in
 * list order; slots past the end of a partial block are 0).
 * scale 0 selects 1/sqrt(d). */
int oracle_sparse_decode_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, int32_t n_keep, int32_t B, int32_t Hq,
                              int32_t Hkv, int32_t d, int32_t N, int32_t stride,
                              int32_t bs, double scale, double* out, double* lse,
                              double* weights);

/* chunked prefill with three branches, combined by `combine`:
 *   A: top_k entries of the m_sparse mean-pooled stream, chosen per
 *      (query tile of q_tile queries, kv head);
 *   B: all entries of the m_dense mean-pooled stream;
 *   C: the last `window` raw tokens up to and including the query.
 * The compressed streams cover the P prior tokens; the chunk's own K/V sit at
 * [P, P+C).  rows: the chunk query indices to evaluate (NULL = all C, in
 * order); out [B][n_rows][Hq][d]; branch_out [3][B][n_rows][Hq][d] or NULL;
 * lse3 [3][B][n_rows][Hq] or NULL; sel_in [B][n_tiles][Hkv][top_k'] or NULL
 * (use this selection for branch A instead of the oracle's own);
 * sel_out [B][n_tiles][Hkv][top_k'] or NULL (every tile);
 * sel_scores [B][n_tiles][Hkv][E_sparse] or NULL (every tile).
 * top_k' = min(top_k, E_sparse).
 * combine 0: out = mean of the three branch softmax outputs; 1: one softmax
 * over the concatenated logits of all three branches.  sink_logits [Hq] or
 * NULL: one extra logit per head (natural-log units) with a zero value vector,
 * in each branch's softmax (combine 0) or in the concatenated one (combine 1).
 * branch_out and lse3 always describe the branches without the sink.
 * indexer 0: the selection scores the pooled query against the bf16 compressed
 * keys (bf16 rounding of the fp32 token-order mean, as the stored stream holds
 * them); 1: against the exact means. */
int oracle_sparse_prefill_attn(const uint16_t* q, int32_t C, const uint16_t* k,
                               const uint16_t* v, int32_t B, int32_t P, int32_t Hq,
                               int32_t Hkv, int32_t d, int32_t stride, int32_t m_sparse,
                               int32_t top_k, int32_t m_dense, int32_t window,
                               int32_t q_tile, double scale, const int32_t* sel_in,
                               const int32_t* rows, int32_t n_rows, int32_t combine,
                               int32_t indexer, const double* sink_logits, double* out,
                               double* branch_out, double* lse3, int32_t* sel_out,
                               double* sel_scores);

/* FP8 KV cache: OCP E4M3 codes with one fp32 scale per (pair, block).
 * oracle_e4m3_value: the value of a code (NaN for 0x7F / 0xFF);
 * oracle_e4m3_encode: the nearest code, ties to even, |y| >= 448 saturates;
 * oracle_quantize_fp8: amax per block, scale = amax / 448 and inv = 448 / amax
 *   in fp32, code = encode(clamp(x * inv in fp32, +-448)); out [B][H][stride][d]
 *   for rows < N, scales [B][H][sstride] (sstride >= nb);
 * oracle_sparse_decode_attn_fp8: exact softmax attention over the kept blocks
 *   of the dequantized cache (scale * value), lists as oracle_sparse_decode_attn. */
double oracle_e4m3_value(uint8_t c);
uint8_t oracle_e4m3_encode(double y);
int oracle_quantize_fp8(const uint16_t* x, int32_t B, int32_t H, int32_t N, int32_t stride,
                        int32_t d, int32_t bs, int32_t sstride, uint8_t* out, float* scales);
int oracle_sparse_decode_attn_fp8(const uint16_t* q, const uint8_t* k8, const uint8_t* v8,
                                  const float* kscales, const float* vscales, const int32_t* idx,
                                  int32_t n_keep, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                  int32_t N, int32_t stride, int32_t bs, int32_t sstride,
                                  double scale, double* out, double* lse);

/* round an fp64 value to the nearest bf16 (ties to even); returns bits */
uint16_t oracle_round_bf16(double x);

#ifdef __cplusplus
}
#endif
#endif
