/* bsa.h -- block-summary sparse attention on MI355X (gfx950): the C ABI.
 *
 * The method (sources are web pages; sections as printed on them):
 *  - Keys are grouped into fixed blocks of 64 consecutive tokens, the unit of
 *    scoring and retention; the first block (attention sink) and the most
 *    recent ~128 tokens (2 blocks) are always kept, and the middle blocks are
 *    kept by importance, 10-20 % of the cache in total.  hotdry.top post
 *    "claude-opus-long-context-kv-cache-sparse-attention", sections
 *    "稀疏注意力与 KV Cache 压缩的工程实现" and the parameter table under
 *    "可落地的配置参数与监控要点".
 *  - Every block is scored, the top-k are kept, and exact scaled-dot-product
 *    attention softmax(q K^T / sqrt(d)) V runs over the kept tokens only.
 *    "CSA + HCA 混合注意力机制", §2.1 and §4.4 (块稀疏模式图解).
 *  - Chunked-prefill variant: m consecutive tokens pooled into one compressed
 *    entry with top-k selection (§4.1-4.2, m = 4), a heavily compressed
 *    stream attended densely (§5.1-5.2, m' = 128), and a sliding window of
 *    raw tokens (§4.3).  Mean pooling is the parameter-free pooling (§4.1).
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE memory owned by the caller, row-major,
 *    16-byte aligned.  bf16 tensors are passed as `const void*`.
 *  - The library never allocates device memory and keeps no state between
 *    calls except cached device properties; calls are thread-safe.
 *  - Every call only enqueues work on `hip_stream` (a hipStream_t; NULL is
 *    the default stream) and does not synchronise.  Outputs are valid once
 *    the stream has completed the work.
 *  - All argument checks run before any launch: a call that returns an
 *    error has launched nothing and written nothing.
 *  - Query head h reads kv head h / (n_q_heads / n_kv_heads).
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define BSA_OK 0
#define BSA_INVALID_ARG (-1)       /* NULL pointer, bad shape, misalignment, n_keep mismatch */
#define BSA_UNSUPPORTED (-2)       /* head_dim not in {64, 128}, unsupported block size or group,
                                      or a size beyond a documented limit */
#define BSA_WORKSPACE_TOO_SMALL (-3)
#define BSA_HIP_ERROR (-4)         /* a launch failed (hipGetLastError after launch) */

typedef struct {
  int32_t batch;       /* B */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t seq_len;     /* N: valid tokens in the cache (prefill: prior tokens P) */
  int32_t seq_stride;  /* cache capacity in tokens, >= seq_len (prefill: >= P + C) */
  int32_t summary_stride; /* blocks between (b, kv head) rows of a block-summary buffer
                             (build/update_block_summaries, select_blocks); 0 means
                             ceil(seq_len / block_size).  A fixed stride (e.g.
                             ceil(seq_stride / block_size)) lets a decode loop keep
                             one buffer while blocks open.  Prefill streams are dense. */
} bsa_shape;

typedef struct {
  int32_t block_size;      /* tokens per block; the decode kernels support 64 */
  int32_t n_sink_blocks;   /* always-kept leading blocks (1 on the page's table) */
  int32_t n_local_blocks;  /* always-kept trailing blocks (2 on the page's table) */
  int32_t top_k;           /* middle blocks kept by score; < 0: derive from keep_ratio */
  double keep_ratio;       /* used when top_k < 0: total kept = floor(r * nb + 0.5), evaluated
                              in double on this value; adaptive: the smallest kept fraction */
  int32_t adaptive;        /* 1: anchor-adaptive k per (b, kv head), see select_blocks */
  double keep_ratio_max;   /* adaptive: the largest kept fraction (rounded as keep_ratio) */
  double anchor_margin;    /* adaptive: tau = a_max + anchor_margin * (a_max - a_min); the
                              kernels form tau in fp32 from (float)anchor_margin */
  int32_t summaries_bf16;  /* 0: the summaries select_blocks / sparse_decode_step read are
                              fp32; 1: bf16 (build_block_summaries' out_bf16: the rounding,
                              ties to even, of the fp32 means), half the bytes to score */
} bsa_select_cfg;

typedef struct {
  int32_t m_sparse;      /* tokens per entry of the selected stream (4) */
  int32_t top_k_sparse;  /* entries kept per (query tile, kv head) (2048) */
  int32_t m_dense;       /* tokens per entry of the dense stream (128) */
  int32_t window;        /* raw tokens attended up to and including the query (128) */
  int32_t q_tile;        /* consecutive queries sharing one selection (64) */
  int32_t combine;       /* BSA_COMBINE_AVERAGE or BSA_COMBINE_CONCAT */
  int32_t indexer;       /* BSA_INDEXER_BF16 (0) or BSA_INDEXER_F32: the keys the branch-A
                            selection scores against */
} bsa_prefill_cfg;

/* how sparse_prefill_attn joins its three branches */
#define BSA_COMBINE_AVERAGE 0 /* (o_A + o_B + o_C) / 3, each branch its own softmax */
#define BSA_COMBINE_CONCAT 1  /* one softmax over the concatenated logits of all three
                                 ("CSA + HCA 混合注意力机制" §4.3) */

/* which pooled keys the branch-A selection scores against ("CSA + HCA 混合注意力机制"
 * §4.2: the indexer scores the compressed entries, its QK product at low precision,
 * its recall measured against a BF16 indexer) */
#define BSA_INDEXER_BF16 0 /* the bf16 compressed keys k_cmp_sparse_bf16, the same entries
                              branch A attends; the pooled query stays fp32 (split exactly
                              into three bf16 terms on the bf16 matrix cores) */
#define BSA_INDEXER_F32 1  /* the fp32 means k_cmp_sparse_f32 (fp32 matrix cores) */

/* ceil(n / m): blocks (or compressed entries) covering n tokens; -1 if m <= 0 or n < 0 */
int32_t bsa_num_blocks(int32_t n, int32_t m);

/* kept blocks per (batch, kv head) for nb blocks: |sink U local| + k, where
 * the candidates are the blocks that are neither sink nor local and
 * k = top_k (or floor(keep_ratio*nb + 0.5) - n_sink - n_local when top_k < 0),
 * clamped to [0, #candidates].  With nb <= sink + local every block is kept.
 * Adaptive selection: the widest list, sink + local + k_hi (see select_blocks).
 * Returns -1 on an invalid cfg. */
int32_t bsa_num_kept(int32_t nb, const bsa_select_cfg* cfg);

/* workspace bytes needed by select_blocks / sparse_decode_attn /
 * sparse_prefill_attn for these arguments (0 if none is needed; SIZE_MAX on
 * invalid arguments).  n_splits = 0 selects the library's own split plan. */
size_t bsa_select_workspace_size(const bsa_shape* shape, const bsa_select_cfg* cfg);
size_t bsa_decode_step_workspace_size(const bsa_shape* shape, const bsa_select_cfg* cfg);
size_t bsa_decode_workspace_size(const bsa_shape* shape, int32_t n_keep, int32_t block_size,
                                 int32_t n_splits);
size_t bsa_prefill_workspace_size(const bsa_shape* shape, int32_t chunk_len,
                                  const bsa_prefill_cfg* cfg);

/* human-readable text of a status code (static storage) */
const char* bsa_status_string(int status);

/* build_block_summaries -- mean of each block of `block_size` consecutive
 * tokens (the block-level importance unit of the hotdry.top post, section
 * 稀疏注意力与 KV Cache 压缩的工程实现; mean pooling per "CSA + HCA
 * 混合注意力机制" §4.1; also the compressed streams of §4.1 and §5.1).
 *   x         bf16 [B][n_kv_heads][seq_stride][d]
 *   out_f32   fp32 [B][n_kv_heads][S][d] or NULL    (S = summary_stride, or nb =
 *             ceil(seq_len / block_size) when that is 0)
 *   out_bf16  bf16 [B][n_kv_heads][S][d] or NULL    (the fp32 mean rounded to nearest even)
 * A partial last block is averaged over its valid tokens.  Tokens past
 * seq_len are never read.  Sums are fp32.  At least one output is required.
 * Any block_size >= 1 is supported. */
int build_block_summaries(const void* x, const bsa_shape* shape, int32_t block_size,
                          float* out_f32, void* out_bf16, void* hip_stream);

/* update_block_summaries -- the per-token part of the decode loop (the block
 * summary bookkeeping of the hotdry.top post, 稀疏注意力与 KV Cache 压缩的工程实现,
 * on a growing cache): recomputes the summaries of the blocks holding tokens
 * [first_token, seq_len) -- the partial last block and any blocks opened
 * since -- from their tokens, with the same arithmetic and order as
 * build_block_summaries, so the result is bit-identical to a rebuild.
 * Other blocks are not touched.  Layout as build_block_summaries (rows
 * shape->summary_stride blocks apart when non-zero).  0 <= first_token <= seq_len. */
int update_block_summaries(const void* x, const bsa_shape* shape, int32_t block_size,
                           int32_t first_token, float* out_f32, void* out_bf16,
                           void* hip_stream);

/* append_kv -- writes n_new tokens' K and V rows into the caches at positions
 * [seq_len, seq_len + n_new) of every (b, kv head), and, when a summaries
 * buffer is given, refreshes the summaries of the blocks those tokens land in
 * (the growing partial block, or blocks they open) in the same launch, with
 * results bit-identical to update_block_summaries / a rebuild.
 *   k_new, v_new      bf16 [B][Hkv][n_new][d]
 *   k_cache, v_cache  bf16 [B][Hkv][seq_stride][d]
 *   summaries_f32/_bf16  [B][Hkv][S][d] or NULL (both NULL: no refresh, block_size unused);
 *                     S = summary_stride, or ceil((seq_len + n_new) / block_size) when 0
 * Requires seq_len + n_new <= seq_stride; seq_len in `shape` is the count
 * before the append. */
int append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              const bsa_shape* shape, int32_t n_new, int32_t block_size, float* summaries_f32,
              void* summaries_bf16, void* hip_stream);

/* select_blocks -- per (batch, kv head): pooled query qbar = sum of the
 * group's query heads (fp32), block scores s_j = qbar . summary_j for the
 * candidate blocks, and the kept list = sink blocks U top-k candidates (by
 * descending score, lower index first on equal scores) U local blocks,
 * ascending.  hotdry.top post, 稀疏注意力与 KV Cache 压缩的工程实现;
 * "CSA + HCA 混合注意力机制" §4.4 steps 1-3.
 *   q          bf16 [B][Hq][d]
 *   summaries  fp32 [B][Hkv][S][d] from build_block_summaries, or its bf16 output when
 *              cfg->summaries_bf16 is 1 (S = summary_stride, or
 *              nb = ceil(seq_len / block_size) when that is 0)
 *   block_idx  int32 [B][Hkv][n_keep] output, n_keep = bsa_num_kept(nb, cfg)
 *   scores_out fp32 [B][Hkv][nb] or NULL: candidate scores (other entries are not written;
 *              adaptive: every block's score)
 *   workspace  bsa_select_workspace_size() bytes of device memory (may be NULL if 0)
 * Anchor-adaptive mode (cfg->adaptive = 1; hotdry.top post, the anchor-point
 * Top-P selection and 锚点动态选择): the sink and local blocks are anchors;
 * tau = a_max + anchor_margin * (a_max - a_min) over their scores (fp32); k per
 * (b, kv head) = #(candidates scoring above tau), clamped so the kept total lies
 * in [keep_ratio * nb, keep_ratio_max * nb] (each rounded as floor(x + 0.5));
 * the list holds sink + top-k + local ascending and is padded with -1 to
 * n_keep.  sparse_decode_attn accepts such padded lists.
 * Requires seq_len >= 1. */
int select_blocks(const void* q, const void* summaries, const bsa_shape* shape,
                  const bsa_select_cfg* cfg, int32_t* block_idx, float* scores_out,
                  void* workspace, size_t ws_bytes, void* hip_stream);

/* sparse_decode_step -- select_blocks followed by sparse_decode_attn, as one call:
 * block scores (the hotdry.top post's block-level evaluation; "CSA + HCA 混合注意力机制"
 * §4.4 steps 1-3), then, for d = 128 and up to 4,096 candidate blocks per (b, kv head),
 * one attention launch whose workgroups each select their pair's kept blocks from the
 * scores before attending (§2.1, §4.4 step 4), then the merge; other shapes run the
 * same steps as separate launches.  block_idx and out/lse are those of the two calls
 * (the same list, the same outputs bit for bit).
 *   q, k, v, out, lse, scale  as for sparse_decode_attn
 *   summaries   fp32 or bf16 (cfg->summaries_bf16) as for select_blocks
 *   cfg         as for select_blocks; adaptive selection is BSA_UNSUPPORTED here
 *   block_idx   int32 [B][Hkv][bsa_num_kept(nb, cfg)], written
 *   workspace   bsa_decode_step_workspace_size(shape, cfg) bytes, 16-byte aligned
 *               (block scores, then the split partials); contents on entry irrelevant */
int sparse_decode_step(const void* q, const void* k, const void* v, const void* summaries,
                       const bsa_shape* shape, const bsa_select_cfg* cfg, int32_t* block_idx,
                       float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                       void* hip_stream);

/* sparse_decode_step_noalloc -- sparse_decode_step for callers that cannot allocate
 * device memory: code under HIP stream capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The workspace is a static array inside the library, one copy per
 * GPU of BSA_NOALLOC_SCRATCH_BYTES, held until the process ends; no call allocates.
 * Arguments, outputs (bit-identical to sparse_decode_step's) and errors as
 * sparse_decode_step without the workspace; BSA_UNSUPPORTED when
 * bsa_decode_step_workspace_size(shape, cfg) exceeds BSA_NOALLOC_SCRATCH_BYTES.
 * hip_stream must belong to the current device.  Every call on one GPU uses the same
 * array: calls that overlap in time on one GPU (other streams, other host threads)
 * race and must be serialised by the caller. */
#define BSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int sparse_decode_step_noalloc(const void* q, const void* k, const void* v,
                               const void* summaries, const bsa_shape* shape,
                               const bsa_select_cfg* cfg, int32_t* block_idx, float scale,
                               float* out, float* lse, void* hip_stream);

/* sparse_decode_attn -- exact softmax(q K^T * scale) V for every query head
 * over the tokens of its kv head's kept blocks ("CSA + HCA 混合注意力机制"
 * §2.1 and §4.4 step 4; the decode step of §2.3 reads the cache after the
 * new token's K/V were appended, so no mask is applied).
 *   q          bf16 [B][Hq][d]
 *   k, v       bf16 [B][Hkv][seq_stride][d]
 *   block_idx  int32 [B][Hkv][n_keep], strictly ascending block indices < nb, each
 *              list optionally ended by a run of -1 (absent entries, as written by an
 *              adaptive select_blocks) and holding at least one block.  Not checked
 *              on the device: any other entry outside [0, nb) is the caller's error;
 *              the kernels clamp it to a valid block, so every read stays inside the
 *              cache (and the scales), but the result is then unspecified
 *   scale      0 selects 1/sqrt(d)
 *   out        fp32 [B][Hq][d]
 *   lse        fp32 [B][Hq] natural-log log-sum-exp of the scaled logits, or NULL
 *   workspace  bsa_decode_workspace_size(shape, n_keep, block_size, 0) bytes, 16-byte
 *              aligned: split partials (o, m, l); contents on entry are irrelevant.
 *              Calls that overlap in time must not share a workspace.
 * block_size must be 64; n_keep >= 1; Hq/Hkv in {1, 2, 4, 8, 16}.  A partial
 * last block contributes only its tokens below seq_len.  seq_len * d * 2 must not
 * exceed 2^32 (a kv head's rows are addressed by 32-bit byte offsets; 16,777,216
 * tokens at d = 128), else BSA_UNSUPPORTED; the same holds for
 * sparse_decode_attn_split and sparse_decode_partials, and for
 * sparse_decode_attn_fp8 with seq_len * d. */
int sparse_decode_attn(const void* q, const void* k, const void* v, const int32_t* block_idx,
                       int32_t n_keep, const bsa_shape* shape, int32_t block_size, float scale,
                       float* out, float* lse, void* workspace, size_t ws_bytes,
                       void* hip_stream);

/* quantize_kv_fp8 -- an FP8 copy of a K or V cache for sparse_decode_attn_fp8
 * (the FP8 KV cache of the aicoding.csdn.net page, 二.2 KV缓存分层存储, (3)
 * FP8量化与无损压缩; the pages fix neither the format nor the scale
 * granularity: this library uses OCP E4M3 with one fp32 scale per (b, kv
 * head, block)).  Per block:
 * amax = max |x| over its valid tokens; scale = amax / 448 and
 * inv = 448 / amax in fp32 (correctly rounded); each value is stored as the
 * E4M3 code nearest (ties to even) to clamp(x * inv, -448, 448).  A block of
 * zeros gets scale 0.  The dequantized value is scale * E4M3(code).
 *   x        bf16 [B][Hkv][seq_stride][d]
 *   out_fp8  uint8 [B][Hkv][seq_stride][d] (rows past seq_len are not written)
 *   scales   fp32 [B][Hkv][S], S = summary_stride or ceil(seq_len / block_size) */
int quantize_kv_fp8(const void* x, const bsa_shape* shape, int32_t block_size, void* out_fp8,
                    float* scales, void* hip_stream);

/* sparse_decode_attn_fp8 -- sparse_decode_attn over an FP8 cache written by
 * quantize_kv_fp8: the exact softmax attention of the dequantized keys and
 * values (E4M3 converts exactly to bf16; the block scales multiply the
 * logits and the weights).  k_scales / v_scales as quantize_kv_fp8's scales.
 * Workspace, lists (incl. -1 padding), requirements and errors as
 * sparse_decode_attn. */
int sparse_decode_attn_fp8(const void* q, const void* k_fp8, const void* v_fp8,
                           const float* k_scales, const float* v_scales, const int32_t* block_idx,
                           int32_t n_keep, const bsa_shape* shape, int32_t block_size,
                           float scale, float* out, float* lse, void* workspace, size_t ws_bytes,
                           void* hip_stream);

/* sparse_decode_attn_split -- sparse_decode_attn with an explicit number of
 * kept-block splits per (batch, kv head) (>= 1; 0 = the library's plan).
 * The result equals sparse_decode_attn's up to fp32 rounding of the merge.
 * Workspace: bsa_decode_workspace_size(shape, n_keep, block_size, n_splits). */
int sparse_decode_attn_split(const void* q, const void* k, const void* v,
                             const int32_t* block_idx, int32_t n_keep, const bsa_shape* shape,
                             int32_t block_size, float scale, float* out, float* lse,
                             void* workspace, size_t ws_bytes, int32_t n_splits,
                             void* hip_stream);

/* The two steps of sparse_decode_attn_split as calls of their own (same
 * kernels, same arguments; calling them in order on one stream with one
 * workspace gives sparse_decode_attn_split's result bit for bit).
 *
 * sparse_decode_partials -- the kept tokens of each (batch, kv head) are cut
 * into runs of kept blocks (splits); per split and query head it writes the
 * unnormalised partial softmax state of "CSA + HCA 混合注意力机制" §2.1 /
 * §4.4 step 4 restricted to the split: m = max of the base-2 scaled logits,
 * l = sum 2^(z - m), o = sum 2^(z - m) V.  Into the workspace (16-byte
 * aligned, bsa_decode_workspace_size(shape, n_keep, block_size, n_splits)
 * bytes): fp32 (m, l) [B*Hkv][splits][g][2], then fp32 o [B*Hkv][splits][g][d].
 * Arguments, lists, requirements and errors as sparse_decode_attn_split. */
int sparse_decode_partials(const void* q, const void* k, const void* v, const int32_t* block_idx,
                           int32_t n_keep, const bsa_shape* shape, int32_t block_size,
                           float scale, void* workspace, size_t ws_bytes, int32_t n_splits,
                           void* hip_stream);

/* sparse_decode_merge -- the exact log-sum-exp merge of the partials that
 * sparse_decode_partials wrote into `workspace` with the same shape, n_keep,
 * block_size and n_splits: M = max_s m_s, L = sum_s 2^(m_s - M) l_s,
 * out = sum_s 2^(m_s - M) o_s / L (fp32 [B][Hq][d]), lse = (M + log2 L) ln 2
 * (fp32 [B][Hq], or NULL).  Errors as sparse_decode_attn_split. */
int sparse_decode_merge(const bsa_shape* shape, int32_t n_keep, int32_t block_size,
                        int32_t n_splits, const void* workspace, size_t ws_bytes, float* out,
                        float* lse, void* hip_stream);

/* sparse_prefill_attn -- chunked prefill of C new queries at positions
 * P + i (P = shape->seq_len prior tokens), three branches averaged:
 *   A ("CSA + HCA 混合注意力机制" §4.1-4.2, §4.4): per (tile of q_tile
 *     consecutive queries, kv head) the pooled query (sum over the tile's
 *     queries and the group's heads, fp32) scores every m_sparse entry against
 *     the keys cfg->indexer names (by default the bf16 compressed keys); the
 *     top_k_sparse entries (descending, lower index first) are attended with
 *     the bf16 streams;
 *   B (§5.1-5.2): all m_dense entries, attended densely;
 *   C (§4.3): raw tokens [P + i - window + 1, P + i] of k, v.
 * The compressed streams cover the P prior tokens only; the chunk's own K/V
 * are already appended at [P, P + C).
 *   q                    bf16 [B][C][Hq][d]
 *   k, v                 bf16 [B][Hkv][seq_stride][d], seq_stride >= P + C
 *   k_cmp_sparse_f32     fp32 [B][Hkv][E_s][d]   (E_s = ceil(P / m_sparse); from build_block_summaries),
 *                        read only with BSA_INDEXER_F32 (may be NULL otherwise)
 *   k/v_cmp_sparse_bf16  bf16 [B][Hkv][E_s][d]
 *   k/v_cmp_dense_bf16   bf16 [B][Hkv][E_d][d]   (E_d = ceil(P / m_dense))
 *   sink_logits          fp32 [Hq] or NULL: one learnable sink logit per query head
 *                        (natural-log units, "CSA + HCA 混合注意力机制" §5.4): an extra
 *                        logit with a zero value vector in each branch's softmax
 *                        (average) or in the single concatenated softmax (concat)
 *   out                  fp32 [B][C][Hq][d]: the branches joined per cfg->combine
 *   lse3                 fp32 [3][B][C][Hq] per-branch log-sum-exp, or NULL
 *   sel_out              int32 [B][ceil(C / q_tile)][Hkv][min(top_k_sparse, E_s)] ascending, or NULL
 *   workspace            bsa_prefill_workspace_size() bytes, 16-byte aligned
 * Values: P V runs on the fp16 matrix cores (fp16 weights, V converted to fp16), so every
 * value attended -- both value streams and the window rows of v -- must lie within fp16's
 * range, |v| <= 65504; larger values give infinite or NaN outputs.  The conversion is
 * exact for bf16 values of magnitude 2^-14 and above (smaller ones keep an absolute error
 * below 2^-25), and the output error, from the fp16 weights, scales with the values'
 * magnitude (about 2e-4 for N(0,1) values).
 * Requires P >= 1, head_dim 128, q_tile * Hq/Hkv in {64, 128, 256},
 * E_s <= 131072, min(top_k_sparse, E_s) <= 4096, E_d <= 16,777,216 and
 * min(window + q_tile, P + C) <= 16,777,216 (a pair's dense-stream rows and a tile's
 * window rows are addressed by 32-bit byte offsets) and, for the selection,
 * ceil(C / q_tile) <= 64 (else BSA_UNSUPPORTED).
 * Equals select_prefill_entries followed by sparse_prefill_attn_selected. */
int sparse_prefill_attn(const void* q, int32_t chunk_len, const void* k, const void* v,
                        const float* k_cmp_sparse_f32, const void* k_cmp_sparse_bf16,
                        const void* v_cmp_sparse_bf16, const void* k_cmp_dense_bf16,
                        const void* v_cmp_dense_bf16, const bsa_shape* shape,
                        const bsa_prefill_cfg* cfg, float scale, const float* sink_logits,
                        float* out, float* lse3, int32_t* sel_out, void* workspace,
                        size_t ws_bytes, void* hip_stream);

/* select_prefill_entries -- the selection step of sparse_prefill_attn alone
 * (the indexer role of "CSA + HCA 混合注意力机制" §4.2 with the pooled tile
 * query of §4.4): per (tile, kv head) the pooled query scores every m_sparse
 * entry against the keys cfg->indexer names and the top_k_sparse entries are
 * written, ascending (descending score, lower index first on equal scores).
 *   q                  bf16 [B][C][Hq][d]
 *   k_cmp_sparse_f32   fp32 [B][Hkv][E_s][d]: read with BSA_INDEXER_F32, else may be NULL
 *   k_cmp_sparse_bf16  bf16 [B][Hkv][E_s][d]: read with BSA_INDEXER_BF16, else may be NULL
 *   sel_out            int32 [B][ceil(C / q_tile)][Hkv][min(top_k_sparse, E_s)]
 *   workspace          bsa_prefill_workspace_size() bytes, 16-byte aligned
 * Same requirements as sparse_prefill_attn. */
int select_prefill_entries(const void* q, int32_t chunk_len, const float* k_cmp_sparse_f32,
                           const void* k_cmp_sparse_bf16, const bsa_shape* shape,
                           const bsa_prefill_cfg* cfg, int32_t* sel_out, void* workspace,
                           size_t ws_bytes, void* hip_stream);

/* sparse_prefill_attn_selected -- the three attention branches and their
 * average (§4.3, §5.2 and the average of sparse_prefill_attn) over a given
 * branch-A selection `sel` (layout of select_prefill_entries' sel_out; each
 * list ascending).  Entry indices outside [0, E_s) are clamped into it.
 * Needs no workspace.  Same requirements as sparse_prefill_attn. */
int sparse_prefill_attn_selected(const void* q, int32_t chunk_len, const void* k, const void* v,
                                 const void* k_cmp_sparse_bf16, const void* v_cmp_sparse_bf16,
                                 const void* k_cmp_dense_bf16, const void* v_cmp_dense_bf16,
                                 const int32_t* sel, const bsa_shape* shape,
                                 const bsa_prefill_cfg* cfg, float scale,
                                 const float* sink_logits, float* out, float* lse3,
                                 void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
