// bsa_launch.h -- internal launch wrappers of libbsa (host side).
// The C ABI in bsa_api.hip validates arguments and plans launches; these
// functions only enqueue kernels on the given stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// mean of the blocks [j0, nb) of `bs` tokens: x [pairs][stride][d] -> [pairs][ostride][d]
void launch_summaries(const uint16_t* x, int64_t pairs, int N, int stride, int d, int bs,
                      int j0, int ostride, float* out_f32, uint16_t* out_bf16, hipStream_t st);

// copy src [pairs][n_new][d] to dst [pairs][stride][d] at rows [N, N + n_new)
void launch_append(const uint16_t* src, uint16_t* dst, int64_t pairs, int n_new, int N,
                   int stride, int d, hipStream_t st);

// append n_new K/V rows at N and refresh the summaries of the blocks they land in
constexpr int APPEND_MAX_BS = 128;  // block sizes the fused refresh stages in LDS
void launch_append_update(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                          uint16_t* v_cache, int64_t pairs, int n_new, int N, int stride, int d,
                          int bs, int ostride, float* out_f32, uint16_t* out_bf16,
                          hipStream_t st);

// OCP E4M3 copy of a cache [pairs][stride][d] with one scale per (pair, block)
void launch_quantize_fp8(const uint16_t* x, uint8_t* out, float* scales, int64_t pairs, int N,
                         int stride, int d, int bs, int sstride, hipStream_t st);

// candidate scores s[pair][j] = qbar . summary_j for j in [c0, c1); summaries
// (fp32, or bf16 when summ_bf16) rows are sstride blocks apart, scores rows nb apart
void launch_scores(const uint16_t* q, const void* summ, bool summ_bf16, int B, int Hq, int Hkv,
                   int d, int nb, int sstride, int c0, int c1, float* scores, hipStream_t st);

// per pair: sink [0,c0) + top-k of scores[c0,c1) + local [c1,nb), ascending.
// adaptive: k per pair from the anchors' scores, clamped to [k_lo, k_hi], the
// list padded with -1 to n_keep
void launch_topk(const float* scores, int64_t pairs, int nb, int c0, int c1, int k, int n_keep,
                 int32_t* idx_out, hipStream_t st, bool adaptive = false, int k_lo = 0,
                 int k_hi = 0, float margin = 0.f);

struct DecodePlan {
  int g;           // query heads per kv head
  int bps;         // kept blocks per split (one workgroup per split)
  int n_splits;    // splits per (batch, kv head)
};
DecodePlan plan_decode(int64_t pairs, int n_keep, int g, int n_splits_req);
size_t decode_workspace_bytes(int64_t pairs, int d, const DecodePlan& p);

// S4: split-K partials into the workspace: [pairs][splits][g][2] (m, l), then
// [pairs][splits][g][d] o
// S3 + S4 in one launch: each workgroup selects its pair's kept blocks from the
// block scores (candidates [c0, c1)) before it attends; split 0 writes the list
// to idx_out.  Fusable for d = 128, up to 4096 candidates and 4160 kept blocks.
bool decode_select_fusable(int d, int g, int n_cand, int n_keep);
void launch_decode_select_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const float* scores, int nb, int c0, int c1, int top_k,
                                   int32_t* idx_out, int n_keep, int B, int Hq, int Hkv, int N,
                                   int stride, float scale, const DecodePlan& plan, float* ws,
                                   hipStream_t st);
void launch_decode_partials(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int d, int N,
                            int stride, float scale, const DecodePlan& plan, float* ws,
                            hipStream_t st);
// the same over an E4M3 cache with per-(pair, block) K and V scales [pairs][sstride]
void launch_decode_partials_fp8(const uint16_t* q, const uint8_t* k, const uint8_t* v,
                                const float* ksc, const float* vsc, int sstride,
                                const int32_t* idx, int n_keep, int B, int Hq, int Hkv, int d,
                                int N, int stride, float scale, const DecodePlan& plan, float* ws,
                                hipStream_t st);
// S5: exact log-sum-exp merge of the partials -> out [B][Hq][d], lse [B][Hq] (or null)
void launch_decode_merge(int B, int Hq, int Hkv, int d, const DecodePlan& plan, const float* ws,
                         float* out, float* lse, hipStream_t st);

// chunked prefill: pooled queries, scores, top-k, three-branch attention
struct PrefillLaunch {
  const uint16_t* q;      // [B][C][Hq][128]
  const uint16_t* k;      // [B][Hkv][stride][128]
  const uint16_t* v;
  const float* k4f;       // [B][Hkv][E4][128] fp32 (scoring copy, BSA_INDEXER_F32)
  const uint16_t* k4b;    // [B][Hkv][E4][128] bf16
  const uint16_t* v4b;
  const uint16_t* k128b;  // [B][Hkv][E128][128] bf16
  const uint16_t* v128b;
  float* out;             // [B][C][Hq][128]
  float* lse3;            // [3][B][C][Hq] or null
  const float* sink;      // [Hq] sink logits or null
  void* workspace;        // pooled queries + scores (R2 only)
  int B, C, Hq, Hkv, P, stride, E4, E128, ksel, window, q_tile, n_tiles;
  int combine;            // 0 average, 1 concatenated softmax
  int indexer_f32;        // 1: R2 scores against k4f, 0: against k4b
  float scale;
};
constexpr int PREFILL_MAX_E4 = 131072;  // entries of the selected stream per (b, kv head)
constexpr int PREFILL_MAX_SEL = 4096;   // selected entries per (tile, kv head)
size_t prefill_workspace_bytes(int B, int Hkv, int D, int n_tiles, int E4, int ksel, bool need_sel);
// R2 (pooled queries, scores, top-k) -> sel [B][n_tiles][Hkv][ksel]
bool launch_prefill_select(const PrefillLaunch& L, int32_t* sel, hipStream_t st);
// R3-R6 over sel
bool launch_prefill_attend(const PrefillLaunch& L, const int32_t* sel, hipStream_t st);

}  // namespace bsa
