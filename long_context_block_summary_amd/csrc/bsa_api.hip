// bsa_api.hip -- the extern "C" entry points declared in include/bsa.h.
// Every argument check runs before any launch; kernels are only enqueued on
// the caller's stream.
#include <math.h>
#include <algorithm>
#include <cmath>
#include <stdint.h>

#include "../../include/bsa.h"
#include "bsa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(const bsa_shape* s) {
  return s && s->batch >= 1 && s->n_q_heads >= 1 && s->n_kv_heads >= 1 &&
         s->n_q_heads % s->n_kv_heads == 0 && s->head_dim >= 1 && s->seq_len >= 0 &&
         s->seq_stride >= s->seq_len && s->summary_stride >= 0;
}

bool dim_supported(int d) { return d == 64 || d == 128; }

bool group_supported(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// candidate range [c0, c1) and |sink U local|
void kept_ranges(int nb, int n_sink, int n_local, int* c0, int* c1, int* fixed) {
  const int s_end = n_sink < nb ? n_sink : nb;
  const int l_beg = nb - n_local > 0 ? nb - n_local : 0;
  *c0 = s_end;
  *c1 = l_beg > s_end ? l_beg : s_end;
  *fixed = l_beg > s_end ? s_end + (nb - l_beg) : nb;
}

int middle_k(int nb, const bsa_select_cfg* cfg, int n_cand) {
  int64_t k;
  if (cfg->top_k >= 0)
    k = cfg->top_k;
  else
    k = (int64_t)floor(cfg->keep_ratio * (double)nb + 0.5) - cfg->n_sink_blocks -
        cfg->n_local_blocks;
  if (k < 0) k = 0;
  if (k > n_cand) k = n_cand;
  return (int)k;
}

bool select_cfg_ok(const bsa_select_cfg* c) {
  if (!c || c->block_size < 1 || c->n_sink_blocks < 0 || c->n_local_blocks < 0) return false;
  if (c->summaries_bf16 != 0 && c->summaries_bf16 != 1) return false;
  if (c->adaptive) {
    return c->adaptive == 1 && c->keep_ratio >= 0.0 && c->keep_ratio <= c->keep_ratio_max &&
           c->keep_ratio_max <= 1.0 && std::isfinite((float)c->anchor_margin);
  }
  return c->top_k >= 0 || (c->keep_ratio >= 0.0 && c->keep_ratio <= 1.0);
}

// adaptive selection: the middle-block count lies in [k_lo, k_hi] (the kept
// totals keep_ratio * nb and keep_ratio_max * nb, rounded as middle_k rounds)
void adaptive_bounds(int nb, const bsa_select_cfg* cfg, int fixed, int n_cand, int* k_lo,
                     int* k_hi) {
  int64_t lo = (int64_t)floor(cfg->keep_ratio * (double)nb + 0.5) - fixed;
  int64_t hi = (int64_t)floor(cfg->keep_ratio_max * (double)nb + 0.5) - fixed;
  lo = lo < 0 ? 0 : (lo > n_cand ? n_cand : lo);
  hi = hi < lo ? lo : (hi > n_cand ? n_cand : hi);
  *k_lo = (int)lo;
  *k_hi = (int)hi;
}

// middle blocks per list: k (fixed mode) or k_hi (adaptive: the widest list)
int list_k(int nb, const bsa_select_cfg* cfg, int c0, int c1, int fixed) {
  if (!cfg->adaptive) return middle_k(nb, cfg, c1 - c0);
  int lo, hi;
  adaptive_bounds(nb, cfg, fixed, c1 - c0, &lo, &hi);
  return hi;
}

// blocks between consecutive (b, kv head) rows of a summaries buffer, or -1
// when the shape's summary_stride is below the blocks in use
int summary_stride(const bsa_shape* s, int bs) {
  const int nb = bsa_num_blocks(s->seq_len, bs);
  if (s->summary_stride == 0) return nb;
  return s->summary_stride >= nb ? s->summary_stride : -1;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_HIP_ERROR;
}

}  // namespace

extern "C" {

int32_t bsa_num_blocks(int32_t n, int32_t m) {
  if (n < 0 || m <= 0) return -1;
  return (int32_t)(((int64_t)n + m - 1) / m);
}

int32_t bsa_num_kept(int32_t nb, const bsa_select_cfg* cfg) {
  if (nb < 0 || !select_cfg_ok(cfg)) return -1;
  int c0, c1, fixed;
  kept_ranges(nb, cfg->n_sink_blocks, cfg->n_local_blocks, &c0, &c1, &fixed);
  return fixed + list_k(nb, cfg, c0, c1, fixed);
}

size_t bsa_select_workspace_size(const bsa_shape* shape, const bsa_select_cfg* cfg) {
  if (!shape_ok(shape) || !select_cfg_ok(cfg)) return SIZE_MAX;
  const int nb = bsa_num_blocks(shape->seq_len, cfg->block_size);
  return (size_t)shape->batch * shape->n_kv_heads * (size_t)nb * sizeof(float);
}

size_t bsa_decode_step_workspace_size(const bsa_shape* shape, const bsa_select_cfg* cfg) {
  if (!shape_ok(shape) || !select_cfg_ok(cfg)) return SIZE_MAX;
  const int n_keep = bsa_num_kept(bsa_num_blocks(shape->seq_len, cfg->block_size), cfg);
  const size_t dec = bsa_decode_workspace_size(shape, n_keep < 1 ? 1 : n_keep, cfg->block_size, 0);
  if (dec == SIZE_MAX) return SIZE_MAX;
  return (bsa_select_workspace_size(shape, cfg) + 255) / 256 * 256 + dec;
}
size_t bsa_decode_workspace_size(const bsa_shape* shape, int32_t n_keep, int32_t block_size,
                                 int32_t n_splits) {
  if (!shape_ok(shape) || n_keep < 1 || block_size < 1 || n_splits < 0) return SIZE_MAX;
  const int g = shape->n_q_heads / shape->n_kv_heads;
  const int64_t pairs = (int64_t)shape->batch * shape->n_kv_heads;
  bsa::DecodePlan p = bsa::plan_decode(pairs, n_keep, g, n_splits);
  return bsa::decode_workspace_bytes(pairs, shape->head_dim, p);
}

const char* bsa_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_INVALID_ARG: return "invalid argument";
    case BSA_UNSUPPORTED: return "unsupported configuration";
    case BSA_WORKSPACE_TOO_SMALL: return "workspace too small";
    case BSA_HIP_ERROR: return "HIP launch error";
    default: return "unknown status";
  }
}

int update_block_summaries(const void* x, const bsa_shape* shape, int32_t block_size,
                           int32_t first_token, float* out_f32, void* out_bf16,
                           void* hip_stream) {
  if (!x || !shape_ok(shape) || block_size < 1 || (!out_f32 && !out_bf16)) return BSA_INVALID_ARG;
  if (!aligned16(x) || (out_f32 && !aligned16(out_f32)) || (out_bf16 && !aligned16(out_bf16)))
    return BSA_INVALID_ARG;
  if (!dim_supported(shape->head_dim)) return BSA_UNSUPPORTED;
  const int nb = bsa_num_blocks(shape->seq_len, block_size);
  const int ss = summary_stride(shape, block_size);
  if (ss < 0 || first_token < 0 || first_token > shape->seq_len) return BSA_INVALID_ARG;
  if (shape->seq_len == 0 || first_token == shape->seq_len) return BSA_OK;
  const int j0 = first_token / block_size;
  if (j0 >= nb) return BSA_OK;
  bsa::launch_summaries(static_cast<const uint16_t*>(x),
                        (int64_t)shape->batch * shape->n_kv_heads, shape->seq_len,
                        shape->seq_stride, shape->head_dim, block_size, j0, ss, out_f32,
                        static_cast<uint16_t*>(out_bf16), static_cast<hipStream_t>(hip_stream));
  return launch_status();
}

int build_block_summaries(const void* x, const bsa_shape* shape, int32_t block_size,
                          float* out_f32, void* out_bf16, void* hip_stream) {
  return update_block_summaries(x, shape, block_size, 0, out_f32, out_bf16, hip_stream);
}

int append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              const bsa_shape* shape, int32_t n_new, int32_t block_size, float* summaries_f32,
              void* summaries_bf16, void* hip_stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !shape_ok(shape) || n_new < 0)
    return BSA_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return BSA_INVALID_ARG;
  if (!dim_supported(shape->head_dim)) return BSA_UNSUPPORTED;
  if ((int64_t)shape->seq_len + n_new > shape->seq_stride) return BSA_INVALID_ARG;
  const bool refresh = summaries_f32 || summaries_bf16;
  bsa_shape after = *shape;
  after.seq_len = shape->seq_len + n_new;
  int ss = 0;
  if (refresh) {
    if (block_size < 1 || (summaries_f32 && !aligned16(summaries_f32)) ||
        (summaries_bf16 && !aligned16(summaries_bf16)))
      return BSA_INVALID_ARG;
    ss = summary_stride(&after, block_size);
    if (ss < 0) return BSA_INVALID_ARG;
  }
  if (n_new == 0) return BSA_OK;
  const int64_t pairs = (int64_t)shape->batch * shape->n_kv_heads;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (refresh && block_size <= bsa::APPEND_MAX_BS) {
    bsa::launch_append_update(static_cast<const uint16_t*>(k_new),
                              static_cast<const uint16_t*>(v_new),
                              static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                              pairs, n_new, shape->seq_len, shape->seq_stride, shape->head_dim,
                              block_size, ss, summaries_f32,
                              static_cast<uint16_t*>(summaries_bf16), st);
    return launch_status();
  }
  bsa::launch_append(static_cast<const uint16_t*>(k_new), static_cast<uint16_t*>(k_cache), pairs,
                     n_new, shape->seq_len, shape->seq_stride, shape->head_dim, st);
  bsa::launch_append(static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(v_cache), pairs,
                     n_new, shape->seq_len, shape->seq_stride, shape->head_dim, st);
  if (refresh)
    bsa::launch_summaries(static_cast<const uint16_t*>(k_cache), pairs, after.seq_len,
                          shape->seq_stride, shape->head_dim, block_size,
                          shape->seq_len / block_size, ss, summaries_f32,
                          static_cast<uint16_t*>(summaries_bf16), st);
  return launch_status();
}

int select_blocks(const void* q, const void* summaries, const bsa_shape* shape,
                  const bsa_select_cfg* cfg, int32_t* block_idx, float* scores_out,
                  void* workspace, size_t ws_bytes, void* hip_stream) {
  if (!q || !summaries || !block_idx || !shape_ok(shape) || !select_cfg_ok(cfg) ||
      shape->seq_len < 1)
    return BSA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(summaries) || (scores_out && !aligned16(scores_out)))
    return BSA_INVALID_ARG;
  if (!dim_supported(shape->head_dim)) return BSA_UNSUPPORTED;
  const int nb = bsa_num_blocks(shape->seq_len, cfg->block_size);
  const int ss = summary_stride(shape, cfg->block_size);
  if (ss < 0) return BSA_INVALID_ARG;
  int c0, c1, fixed;
  kept_ranges(nb, cfg->n_sink_blocks, cfg->n_local_blocks, &c0, &c1, &fixed);
  const int k = list_k(nb, cfg, c0, c1, fixed);  // adaptive: the widest list
  const int n_keep = fixed + k;
  int k_lo = k, k_hi = k;
  if (cfg->adaptive) adaptive_bounds(nb, cfg, fixed, c1 - c0, &k_lo, &k_hi);
  float* scores = scores_out;
  if (!scores) {
    if (ws_bytes < bsa_select_workspace_size(shape, cfg)) return BSA_WORKSPACE_TOO_SMALL;
    if ((c1 > c0 || cfg->adaptive) && !workspace) return BSA_INVALID_ARG;
    scores = static_cast<float*>(workspace);
  }
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  // the adaptive threshold needs the anchors' scores too: score every block
  const int s0 = cfg->adaptive ? 0 : c0, s1 = cfg->adaptive ? nb : c1;
  bsa::launch_scores(static_cast<const uint16_t*>(q), summaries, cfg->summaries_bf16 != 0,
                     shape->batch, shape->n_q_heads, shape->n_kv_heads, shape->head_dim, nb, ss,
                     s0, s1, scores, st);
  bsa::launch_topk(scores, (int64_t)shape->batch * shape->n_kv_heads, nb, c0, c1, k, n_keep,
                   block_idx, st, cfg->adaptive != 0, k_lo, k_hi, (float)cfg->anchor_margin);
  return launch_status();
}

static int decode_checks(const bsa_shape* shape, int32_t n_keep, int32_t block_size,
                         int32_t n_splits, const void* workspace, size_t ws_bytes,
                         bsa::DecodePlan* plan, int elem_bytes = 2);

int sparse_decode_step(const void* q, const void* k, const void* v, const void* summaries,
                       const bsa_shape* shape, const bsa_select_cfg* cfg, int32_t* block_idx,
                       float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                       void* hip_stream) {
  if (!q || !k || !v || !summaries || !block_idx || !out || !shape_ok(shape) ||
      !select_cfg_ok(cfg) || shape->seq_len < 1)
    return BSA_INVALID_ARG;
  if (cfg->adaptive) return BSA_UNSUPPORTED;  // the list length varies: use the two calls
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(summaries) || !aligned16(out))
    return BSA_INVALID_ARG;
  if (!dim_supported(shape->head_dim)) return BSA_UNSUPPORTED;
  const int nb = bsa_num_blocks(shape->seq_len, cfg->block_size);
  const int ss = summary_stride(shape, cfg->block_size);
  if (ss < 0) return BSA_INVALID_ARG;
  int c0, c1, fixed;
  kept_ranges(nb, cfg->n_sink_blocks, cfg->n_local_blocks, &c0, &c1, &fixed);
  const int top_k = list_k(nb, cfg, c0, c1, fixed);
  const int n_keep = fixed + top_k;
  if (ws_bytes < bsa_decode_step_workspace_size(shape, cfg)) return BSA_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned16(workspace)) return BSA_INVALID_ARG;
  const size_t sel_bytes = (bsa_select_workspace_size(shape, cfg) + 255) / 256 * 256;
  bsa::DecodePlan plan;
  const int rc = decode_checks(shape, n_keep, cfg->block_size, 0,
                               static_cast<char*>(workspace) + sel_bytes, ws_bytes - sel_bytes,
                               &plan, 2);
  if (rc != BSA_OK) return rc;
  if (scale == 0.f) scale = 1.f / sqrtf((float)shape->head_dim);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  float* scores = static_cast<float*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + sel_bytes);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
  if (c1 > c0)
    bsa::launch_scores(qb, summaries, cfg->summaries_bf16 != 0, shape->batch, shape->n_q_heads,
                       shape->n_kv_heads, shape->head_dim, nb, ss, c0, c1, scores, st);
  if (bsa::decode_select_fusable(shape->head_dim, plan.g, c1 - c0, n_keep)) {
    bsa::launch_decode_select_partials(qb, kb, vb, scores, nb, c0, c1, top_k, block_idx, n_keep,
                                       shape->batch, shape->n_q_heads, shape->n_kv_heads,
                                       shape->seq_len, shape->seq_stride, scale, plan, part, st);
  } else {  // the same steps as separate launches
    bsa::launch_topk(scores, (int64_t)shape->batch * shape->n_kv_heads, nb, c0, c1, top_k, n_keep,
                     block_idx, st, false, top_k, top_k, 0.f);
    bsa::launch_decode_partials(qb, kb, vb, block_idx, n_keep, shape->batch, shape->n_q_heads,
                                shape->n_kv_heads, shape->head_dim, shape->seq_len,
                                shape->seq_stride, scale, plan, part, st);
  }
  bsa::launch_decode_merge(shape->batch, shape->n_q_heads, shape->n_kv_heads, shape->head_dim,
                           plan, part, out, lse, st);
  return launch_status();
}

// checks shared by the decode calls (shape, list length, block size, splits,
// workspace); fills the plan.  Nothing is launched when a check fails.
// elem_bytes: bytes per cached value (2 bf16, 1 FP8); the kernels address a
// kv head's rows by 32-bit byte offsets from the head's base.
static int decode_checks(const bsa_shape* shape, int32_t n_keep, int32_t block_size,
                         int32_t n_splits, const void* workspace, size_t ws_bytes,
                         bsa::DecodePlan* plan, int elem_bytes) {
  if (!shape_ok(shape) || n_keep < 1 || n_splits < 0 || shape->seq_len < 1 || block_size < 1)
    return BSA_INVALID_ARG;
  if (n_keep > bsa_num_blocks(shape->seq_len, block_size)) return BSA_INVALID_ARG;
  const int g = shape->n_q_heads / shape->n_kv_heads;
  if (block_size != 64 || !dim_supported(shape->head_dim) || !group_supported(g))
    return BSA_UNSUPPORTED;
  if ((int64_t)shape->seq_len * shape->head_dim * elem_bytes > (int64_t(1) << 32))
    return BSA_UNSUPPORTED;
  const int64_t pairs = (int64_t)shape->batch * shape->n_kv_heads;
  *plan = bsa::plan_decode(pairs, n_keep, g, n_splits);
  if (ws_bytes < bsa::decode_workspace_bytes(pairs, shape->head_dim, *plan))
    return BSA_WORKSPACE_TOO_SMALL;
  if (!workspace || !aligned16(workspace)) return BSA_INVALID_ARG;
  return BSA_OK;
}

int sparse_decode_partials(const void* q, const void* k, const void* v, const int32_t* block_idx,
                           int32_t n_keep, const bsa_shape* shape, int32_t block_size,
                           float scale, void* workspace, size_t ws_bytes, int32_t n_splits,
                           void* hip_stream) {
  if (!q || !k || !v || !block_idx) return BSA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return BSA_INVALID_ARG;
  bsa::DecodePlan plan;
  const int rc = decode_checks(shape, n_keep, block_size, n_splits, workspace, ws_bytes, &plan);
  if (rc != BSA_OK) return rc;
  if (scale == 0.f) scale = 1.f / sqrtf((float)shape->head_dim);
  bsa::launch_decode_partials(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                              static_cast<const uint16_t*>(v), block_idx, n_keep, shape->batch,
                              shape->n_q_heads, shape->n_kv_heads, shape->head_dim,
                              shape->seq_len, shape->seq_stride, scale, plan,
                              static_cast<float*>(workspace),
                              static_cast<hipStream_t>(hip_stream));
  return launch_status();
}

int sparse_decode_merge(const bsa_shape* shape, int32_t n_keep, int32_t block_size,
                        int32_t n_splits, const void* workspace, size_t ws_bytes, float* out,
                        float* lse, void* hip_stream) {
  if (!out || !aligned16(out)) return BSA_INVALID_ARG;
  bsa::DecodePlan plan;
  const int rc = decode_checks(shape, n_keep, block_size, n_splits, workspace, ws_bytes, &plan);
  if (rc != BSA_OK) return rc;
  bsa::launch_decode_merge(shape->batch, shape->n_q_heads, shape->n_kv_heads, shape->head_dim,
                           plan, static_cast<const float*>(workspace), out, lse,
                           static_cast<hipStream_t>(hip_stream));
  return launch_status();
}

int sparse_decode_attn_split(const void* q, const void* k, const void* v,
                             const int32_t* block_idx, int32_t n_keep, const bsa_shape* shape,
                             int32_t block_size, float scale, float* out, float* lse,
                             void* workspace, size_t ws_bytes, int32_t n_splits,
                             void* hip_stream) {
  if (!q || !k || !v || !block_idx || !out) return BSA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return BSA_INVALID_ARG;
  bsa::DecodePlan plan;
  const int rc = decode_checks(shape, n_keep, block_size, n_splits, workspace, ws_bytes, &plan);
  if (rc != BSA_OK) return rc;
  if (scale == 0.f) scale = 1.f / sqrtf((float)shape->head_dim);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  bsa::launch_decode_partials(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                              static_cast<const uint16_t*>(v), block_idx, n_keep, shape->batch,
                              shape->n_q_heads, shape->n_kv_heads, shape->head_dim,
                              shape->seq_len, shape->seq_stride, scale, plan,
                              static_cast<float*>(workspace), st);
  bsa::launch_decode_merge(shape->batch, shape->n_q_heads, shape->n_kv_heads, shape->head_dim,
                           plan, static_cast<const float*>(workspace), out, lse, st);
  return launch_status();
}

int quantize_kv_fp8(const void* x, const bsa_shape* shape, int32_t block_size, void* out_fp8,
                    float* scales, void* hip_stream) {
  if (!x || !out_fp8 || !scales || !shape_ok(shape) || block_size < 1) return BSA_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out_fp8)) return BSA_INVALID_ARG;
  if (!dim_supported(shape->head_dim)) return BSA_UNSUPPORTED;
  const int ss = summary_stride(shape, block_size);
  if (ss < 0) return BSA_INVALID_ARG;
  if (shape->seq_len == 0) return BSA_OK;
  bsa::launch_quantize_fp8(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(out_fp8),
                           scales, (int64_t)shape->batch * shape->n_kv_heads, shape->seq_len,
                           shape->seq_stride, shape->head_dim, block_size, ss,
                           static_cast<hipStream_t>(hip_stream));
  return launch_status();
}

int sparse_decode_attn_fp8(const void* q, const void* k_fp8, const void* v_fp8,
                           const float* k_scales, const float* v_scales, const int32_t* block_idx,
                           int32_t n_keep, const bsa_shape* shape, int32_t block_size,
                           float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                           void* hip_stream) {
  if (!q || !k_fp8 || !v_fp8 || !k_scales || !v_scales || !block_idx || !out)
    return BSA_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_fp8) || !aligned16(v_fp8) || !aligned16(out))
    return BSA_INVALID_ARG;
  bsa::DecodePlan plan;
  const int rc = decode_checks(shape, n_keep, block_size, 0, workspace, ws_bytes, &plan, 1);
  if (rc != BSA_OK) return rc;
  const int ss = summary_stride(shape, block_size);
  if (ss < 0) return BSA_INVALID_ARG;
  if (scale == 0.f) scale = 1.f / sqrtf((float)shape->head_dim);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  bsa::launch_decode_partials_fp8(static_cast<const uint16_t*>(q),
                                  static_cast<const uint8_t*>(k_fp8),
                                  static_cast<const uint8_t*>(v_fp8), k_scales, v_scales, ss,
                                  block_idx, n_keep, shape->batch, shape->n_q_heads,
                                  shape->n_kv_heads, shape->head_dim, shape->seq_len,
                                  shape->seq_stride, scale, plan,
                                  static_cast<float*>(workspace), st);
  bsa::launch_decode_merge(shape->batch, shape->n_q_heads, shape->n_kv_heads, shape->head_dim,
                           plan, static_cast<const float*>(workspace), out, lse, st);
  return launch_status();
}

int sparse_decode_attn(const void* q, const void* k, const void* v, const int32_t* block_idx,
                       int32_t n_keep, const bsa_shape* shape, int32_t block_size, float scale,
                       float* out, float* lse, void* workspace, size_t ws_bytes,
                       void* hip_stream) {
  return sparse_decode_attn_split(q, k, v, block_idx, n_keep, shape, block_size, scale, out, lse,
                                  workspace, ws_bytes, 0, hip_stream);
}

size_t bsa_prefill_workspace_size(const bsa_shape* shape, int32_t chunk_len,
                                  const bsa_prefill_cfg* cfg) {
  if (!shape_ok(shape) || !cfg || chunk_len < 1 || cfg->m_sparse < 1 || cfg->q_tile < 1 ||
      cfg->top_k_sparse < 1 || shape->seq_len < 1)
    return SIZE_MAX;
  const int E4 = bsa_num_blocks(shape->seq_len, cfg->m_sparse);
  const int n_tiles = bsa_num_blocks(chunk_len, cfg->q_tile);
  const int ksel = cfg->top_k_sparse < E4 ? cfg->top_k_sparse : E4;
  return bsa::prefill_workspace_bytes(shape->batch, shape->n_kv_heads, shape->head_dim, n_tiles,
                                      E4, ksel, true);
}

}  // extern "C"

namespace {
// Shared checks of the prefill entry points; fills the launch description
// (pointers the caller does not pass stay null).
int prefill_setup(const void* q, int32_t chunk_len, const bsa_shape* shape,
                  const bsa_prefill_cfg* cfg, float scale, bsa::PrefillLaunch* L) {
  if (!q || !shape_ok(shape) || !cfg || chunk_len < 1 || shape->seq_len < 1) return BSA_INVALID_ARG;
  if (cfg->m_sparse < 1 || cfg->m_dense < 1 || cfg->top_k_sparse < 1 || cfg->window < 1 ||
      cfg->q_tile < 1 || (cfg->combine != BSA_COMBINE_AVERAGE && cfg->combine != BSA_COMBINE_CONCAT) ||
      (cfg->indexer != BSA_INDEXER_BF16 && cfg->indexer != BSA_INDEXER_F32))
    return BSA_INVALID_ARG;
  if ((int64_t)shape->seq_len + chunk_len > shape->seq_stride) return BSA_INVALID_ARG;
  if (!aligned16(q)) return BSA_INVALID_ARG;
  const int g = shape->n_q_heads / shape->n_kv_heads;
  const int rows = cfg->q_tile * g;
  const int E4 = bsa_num_blocks(shape->seq_len, cfg->m_sparse);
  const int ksel = cfg->top_k_sparse < E4 ? cfg->top_k_sparse : E4;
  if (shape->head_dim != 128 || (rows != 64 && rows != 128 && rows != 256) ||
      E4 > bsa::PREFILL_MAX_E4 || ksel > bsa::PREFILL_MAX_SEL)
    return BSA_UNSUPPORTED;
  // the attention addresses a pair's dense-stream rows and a tile's window rows
  // by 32-bit byte offsets from one base (256-byte rows at d = 128)
  const int64_t e_dense = bsa_num_blocks(shape->seq_len, cfg->m_dense);
  const int64_t win_rows =
      std::min<int64_t>((int64_t)cfg->window + cfg->q_tile, (int64_t)shape->seq_len + chunk_len);
  if (e_dense * 256 > (int64_t(1) << 32) || win_rows * 256 > (int64_t(1) << 32))
    return BSA_UNSUPPORTED;
  *L = bsa::PrefillLaunch{};
  L->q = static_cast<const uint16_t*>(q);
  L->B = shape->batch;
  L->C = chunk_len;
  L->Hq = shape->n_q_heads;
  L->Hkv = shape->n_kv_heads;
  L->P = shape->seq_len;
  L->stride = shape->seq_stride;
  L->E4 = E4;
  L->E128 = bsa_num_blocks(shape->seq_len, cfg->m_dense);
  L->ksel = ksel;
  L->window = cfg->window;
  L->q_tile = cfg->q_tile;
  L->n_tiles = bsa_num_blocks(chunk_len, cfg->q_tile);
  L->scale = scale == 0.f ? 1.f / sqrtf(128.f) : scale;
  L->combine = cfg->combine;
  L->indexer_f32 = cfg->indexer == BSA_INDEXER_F32 ? 1 : 0;
  return BSA_OK;
}

int prefill_set_streams(const void* k, const void* v, const void* k_cmp_sparse_bf16,
                        const void* v_cmp_sparse_bf16, const void* k_cmp_dense_bf16,
                        const void* v_cmp_dense_bf16, float* out, bsa::PrefillLaunch* L) {
  const void* ptrs[] = {k, v, k_cmp_sparse_bf16, v_cmp_sparse_bf16, k_cmp_dense_bf16,
                        v_cmp_dense_bf16, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return BSA_INVALID_ARG;
  L->k = static_cast<const uint16_t*>(k);
  L->v = static_cast<const uint16_t*>(v);
  L->k4b = static_cast<const uint16_t*>(k_cmp_sparse_bf16);
  L->v4b = static_cast<const uint16_t*>(v_cmp_sparse_bf16);
  L->k128b = static_cast<const uint16_t*>(k_cmp_dense_bf16);
  L->v128b = static_cast<const uint16_t*>(v_cmp_dense_bf16);
  L->out = out;
  return BSA_OK;
}

// the keys the selection scores against: the one cfg->indexer names must be
// given (16-byte aligned); the other is not read
int prefill_set_indexer_keys(const float* k_cmp_sparse_f32, const void* k_cmp_sparse_bf16,
                             bsa::PrefillLaunch* L) {
  const void* need = L->indexer_f32 ? static_cast<const void*>(k_cmp_sparse_f32) : k_cmp_sparse_bf16;
  if (!need || !aligned16(need)) return BSA_INVALID_ARG;
  L->k4f = k_cmp_sparse_f32;
  L->k4b = static_cast<const uint16_t*>(k_cmp_sparse_bf16);
  return BSA_OK;
}
}  // namespace

extern "C" {

int select_prefill_entries(const void* q, int32_t chunk_len, const float* k_cmp_sparse_f32,
                           const void* k_cmp_sparse_bf16, const bsa_shape* shape,
                           const bsa_prefill_cfg* cfg, int32_t* sel_out, void* workspace,
                           size_t ws_bytes, void* hip_stream) {
  bsa::PrefillLaunch L;
  int st = prefill_setup(q, chunk_len, shape, cfg, 0.f, &L);
  if (st != BSA_OK) return st;
  st = prefill_set_indexer_keys(k_cmp_sparse_f32, k_cmp_sparse_bf16, &L);
  if (st != BSA_OK) return st;
  if (!sel_out || !workspace || !aligned16(workspace)) return BSA_INVALID_ARG;
  if (ws_bytes < bsa::prefill_workspace_bytes(L.B, L.Hkv, 128, L.n_tiles, L.E4, L.ksel, false))
    return BSA_WORKSPACE_TOO_SMALL;
  L.workspace = workspace;
  if (!bsa::launch_prefill_select(L, sel_out, static_cast<hipStream_t>(hip_stream)))
    return BSA_UNSUPPORTED;
  return launch_status();
}

int sparse_prefill_attn_selected(const void* q, int32_t chunk_len, const void* k, const void* v,
                                 const void* k_cmp_sparse_bf16, const void* v_cmp_sparse_bf16,
                                 const void* k_cmp_dense_bf16, const void* v_cmp_dense_bf16,
                                 const int32_t* sel, const bsa_shape* shape,
                                 const bsa_prefill_cfg* cfg, float scale,
                                 const float* sink_logits, float* out, float* lse3,
                                 void* hip_stream) {
  bsa::PrefillLaunch L;
  int st = prefill_setup(q, chunk_len, shape, cfg, scale, &L);
  if (st != BSA_OK) return st;
  st = prefill_set_streams(k, v, k_cmp_sparse_bf16, v_cmp_sparse_bf16, k_cmp_dense_bf16,
                           v_cmp_dense_bf16, out, &L);
  if (st != BSA_OK) return st;
  if (!sel) return BSA_INVALID_ARG;
  L.lse3 = lse3;
  L.sink = sink_logits;
  if (!bsa::launch_prefill_attend(L, sel, static_cast<hipStream_t>(hip_stream)))
    return BSA_UNSUPPORTED;
  return launch_status();
}

int sparse_prefill_attn(const void* q, int32_t chunk_len, const void* k, const void* v,
                        const float* k_cmp_sparse_f32, const void* k_cmp_sparse_bf16,
                        const void* v_cmp_sparse_bf16, const void* k_cmp_dense_bf16,
                        const void* v_cmp_dense_bf16, const bsa_shape* shape,
                        const bsa_prefill_cfg* cfg, float scale, const float* sink_logits,
                        float* out, float* lse3, int32_t* sel_out, void* workspace,
                        size_t ws_bytes, void* hip_stream) {
  bsa::PrefillLaunch L;
  int st = prefill_setup(q, chunk_len, shape, cfg, scale, &L);
  if (st != BSA_OK) return st;
  st = prefill_set_streams(k, v, k_cmp_sparse_bf16, v_cmp_sparse_bf16, k_cmp_dense_bf16,
                           v_cmp_dense_bf16, out, &L);
  if (st != BSA_OK) return st;
  st = prefill_set_indexer_keys(k_cmp_sparse_f32, k_cmp_sparse_bf16, &L);
  if (st != BSA_OK) return st;
  if (!workspace || !aligned16(workspace)) return BSA_INVALID_ARG;
  if (ws_bytes < bsa::prefill_workspace_bytes(L.B, L.Hkv, 128, L.n_tiles, L.E4, L.ksel,
                                              sel_out == nullptr))
    return BSA_WORKSPACE_TOO_SMALL;
  L.lse3 = lse3;
  L.sink = sink_logits;
  L.workspace = workspace;
  int32_t* sel = sel_out;
  if (!sel) {  // after the pooled queries and the scores
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    sel = reinterpret_cast<int32_t*>(
        static_cast<char*>(workspace) + al((size_t)L.B * L.n_tiles * L.Hkv * 128 * 4) +
        al((size_t)L.B * L.Hkv * L.n_tiles * (size_t)((L.E4 + 3) & ~3) * 4));
  }
  hipStream_t hs = static_cast<hipStream_t>(hip_stream);
  if (!bsa::launch_prefill_select(L, sel, hs) || !bsa::launch_prefill_attend(L, sel, hs))
    return BSA_UNSUPPORTED;
  return launch_status();
}

}  // extern "C"
