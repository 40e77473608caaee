/*
 * dfv.h -- C ABI of the MI355X (gfx950) DFlash2 verification-attention library.
 *
 * What the library computes (restated from three pull-request pages of a vLLM
 * fork; cited by PR number and section):
 *   [#556] "[Perf] Add opt-in DFlash2 schedules and numerical audits"
 *   [#587] "[Perf] Reduce DFlash2 long-context verification decay"
 *   [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK reuse"
 *
 * q draft-verification query tokens (q8 in the pages; 1..8 here), causal among
 * themselves and placed at the last q positions of the context, with six FP16
 * query heads sharing one KV head of dimension 256, attend over a paged KV cache
 * held in OCP E4M3 with per-tensor FP32 scales ([#589] Test Plan; [#556] Test
 * Plan).  The context is cut into logical splits (80 in the pages: [#587]
 * Implementation, [#589] Purpose); every split keeps an FP32 online-softmax
 * state -- running max, compensated sum, FP32 numerator -- and a combine kernel
 * merges the splits into the FP16 output ([#589] Test Result).  The full FP32
 * per-split workspace is an output in its own right ([#589] Test Plan).
 *
 * Definitions used throughout:
 *   L_b       context length of sequence b, including its q query tokens.
 *   p_i       = L_b - q + i, position of query token i; it sees keys 0..p_i.
 *   row r     = i * 6 + h for query token i and head h (6q rows per sequence).
 *   S         split size in tokens: desc.split_tokens, or when that is 0 the
 *             per-sequence rule S = 32 * ceil(ceil(L_b / NS) / 32), which gives
 *             the pages' 3296-token split at the 261888-token capacity boundary
 *             ([#589] Test Plan, [#587] Purpose).  Split j covers keys
 *             [j*S, min((j+1)*S, p_i + 1)) of row (b, i, h).
 *   c         = softmax_scale * k_scale; score s_t = c * <Q_row, K_t>, where K_t
 *             and V_t are the E4M3-decoded cache rows of token t.
 *   state     of split j: m = max_t s_t (natural-log units of the scaled
 *             score), l = sum_t exp(s_t - m), o[d] = v_scale * sum_t
 *             exp(s_t - m) * V_t[d].  An empty split is (-inf, 0, 0).
 *   output    = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j, M = max_j m_j,
 *             rounded to FP16 (round to nearest even).
 *
 * Memory layouts (all row-major, all device memory owned by the caller):
 *   q            FP16   [B][q][6][256]
 *   k_cache      uint8  [num_blocks][16][1][256]   E4M3 codes, 16-token pages
 *   v_cache      uint8  [num_blocks][16][1][256]
 *   block_table  int32  [B][max_blocks_per_seq]    token t of sequence b lives in
 *                                                  page block_table[b][t/16], slot t%16
 *   context_lens int32  [B]
 *   k_scale      float32[1], v_scale float32[1]    device scalars (per layer)
 *   ws_max       float32[B][q][6][NS]
 *   ws_sum       float32[B][q][6][NS]
 *   ws_num       float32[B][q][6][NS][256]
 *   out          FP16   [B][q][6][256]
 *
 * Conventions:
 *   - Every call is asynchronous and stream-ordered on `stream` (a hipStream_t;
 *     NULL is the default stream).  No call synchronizes the host.
 *   - The library allocates no memory and keeps no state between calls except
 *     what the caller hands in (the scratch buffer of the split stage).
 *   - Every argument the host can check is checked before any launch; on error
 *     nothing is launched and nothing is written.  A launch failure returns
 *     DFV_ERR_LAUNCH.  No C++ exception crosses this boundary.
 *   - Device-resident values cannot be checked without a synchronization.  The
 *     caller guarantees q <= context_lens[b] <= max_context_len, block ids
 *     within the caches for every page a context touches, and scales > 0.
 *     Kernels clamp context_lens[b] into [q, max_context_len], so a bad length
 *     cannot index past a block-table row.
 *   - Results are deterministic: the same inputs on the same device give
 *     byte-identical outputs and workspaces.
 */
#ifndef DFV_H_
#define DFV_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DFV_API __attribute__((visibility("default")))
#else
#define DFV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFV_OK = 0,
  DFV_ERR_NULL = -1,        /* a required pointer is NULL                         */
  DFV_ERR_UNSUPPORTED = -2, /* shape outside the admitted set (caller keeps its own
                               operator, as the pages' shape-guarded admission does:
                               [#556] Purpose, [#587] Implementation)              */
  DFV_ERR_ALIGN = -3,       /* a pointer is not aligned as documented              */
  DFV_ERR_ARG = -4,         /* an inconsistent size or count                       */
  DFV_ERR_LAUNCH = -5,      /* the HIP runtime rejected a launch                   */
  DFV_ERR_SCRATCH = -7      /* scratch buffer smaller than dfv_attn_scratch_bytes  */
} dfv_status;

/* Shape descriptor.  Admitted set: num_q_heads = 6, num_kv_heads = 1,
 * head_dim = 256, block_size = 16, 1 <= num_q <= 8, 1 <= num_splits <= 256,
 * batch >= 1, batch * num_splits <= 2^20, split_tokens = 0 or a positive
 * multiple of 32 with num_splits * split_tokens >= max_context_len,
 * num_q <= max_context_len <= min(16 * max_blocks_per_seq, 2^22) (2^22 =
 * 4194304 tokens, sixteen times the pages' 262144-token capacity, keeps every
 * key index of the kernels inside 32-bit arithmetic), softmax_scale > 0 and
 * finite. */
typedef struct {
  int32_t batch;              /* B                                                   */
  int32_t num_q;              /* q, verification tokens per sequence                 */
  int32_t num_q_heads;        /* 6                                                   */
  int32_t num_kv_heads;       /* 1                                                   */
  int32_t head_dim;           /* 256                                                 */
  int32_t block_size;         /* 16 tokens per page                                  */
  int32_t max_blocks_per_seq; /* block-table row stride (entries)                    */
  int32_t num_splits;         /* NS, logical splits (80 in the pages)                */
  int32_t split_tokens;       /* 0 = per-sequence rule; else fixed S, multiple of 32 */
  int32_t max_context_len;    /* host-known bound on every context_lens[b]           */
  float softmax_scale;        /* 1/sqrt(256) in the pages' configuration             */
} dfv_attn_desc;

/* Human-readable name of a status code (static string, never NULL). */
DFV_API const char* dfv_status_string(int status);

/* Validate a descriptor without touching a device.  Returns DFV_OK or the
 * status any entry point would return for it. */
DFV_API dfv_status dfv_attn_check(const dfv_attn_desc* desc);

/* Bytes of caller-provided scratch that dfv_attn_split and dfv_attn need for
 * `desc`, written to *bytes.  To fill the GPU every logical split is cut into
 * C = max(1, min(4, 256 / (batch * num_splits))) key chunks processed by
 * separate workgroups; with C > 1 their FP32 states (B*q*6*NS*C of them,
 * 258 floats each) are staged in the scratch buffer and merged, in chunk
 * order, into the workspace by a second kernel.  With C = 1 the size is 0 and
 * `scratch` may be NULL.  The contents need no initialisation and are
 * meaningless between calls.  Calls that may overlap in time must not share a
 * scratch buffer.  Returns the descriptor's status. */
DFV_API dfv_status dfv_attn_scratch_bytes(const dfv_attn_desc* desc, size_t* bytes);

/* Every byte the split stage writes for `desc`, from one call: the workspace
 * (ws_max and ws_sum, B*q*6*NS floats each; ws_num, B*q*6*NS*256 floats)
 * plus the scratch that dfv_attn_scratch_bytes reports.  The workspace is an
 * output whose layout the pages fix ([#589] Test Plan: the full FP32
 * numerator/max/sum workspace is compared), the scratch is internal; they
 * stay separate arguments so the workspace keeps exactly that layout and a
 * caller can reuse one scratch buffer across layers.  Returns 0 when the
 * descriptor is not admitted (shape-guarded admission: [#556] Purpose). */
DFV_API size_t dfv_attn_workspace_bytes(const dfv_attn_desc* desc);

/* Split stage: per-split FP32 states of every row ([#587] Implementation:
 * 80 logical splits, 32-key online updates, compensated FP32 sums, probability
 * residual products, FP32 state; [#589] Test Plan: full numerator/max/sum
 * workspace).  Reads q, the caches through block_table, context_lens and the
 * two scales; writes ws_max, ws_sum, ws_num (every split of every row,
 * including empty ones).  scratch_bytes must be at least what
 * dfv_attn_scratch_bytes reports (scratch may be NULL when that is 0).
 * Launches the split kernel and, with C > 1 key chunks, the chunk merge.
 * Alignment: q, k_cache, v_cache, ws_num 16 bytes; others 4 bytes. */
DFV_API dfv_status dfv_attn_split(const dfv_attn_desc* desc, const void* q,
                          const uint8_t* k_cache, const uint8_t* v_cache,
                          const int32_t* block_table, const int32_t* context_lens,
                          const float* k_scale, const float* v_scale,
                          float* ws_max, float* ws_sum, float* ws_num,
                          void* scratch, size_t scratch_bytes, void* stream);

/* Number of key chunks C >= 1 each logical split is cut into for `desc`
 * (C = max(1, min(4, 256 / (batch * num_splits)))), written to *chunks.
 * Returns the descriptor's status. */
DFV_API dfv_status dfv_attn_chunks(const dfv_attn_desc* desc, int32_t* chunks);

/* The split stage's first kernel on its own: the FP32 state of every
 * (row, split j, key chunk c), the same state definition as the workspace
 * applied to the chunk's keys.  With T = ceil(L_b / 32) key tiles, split j
 * holds tiles [a_j, b_j) = [min(j*S/32, T), min((j+1)*S/32, T)); with
 * n_j = b_j - a_j, chunk c holds tiles [a_j + floor(c*n_j/C), a_j +
 * floor((c+1)*n_j/C)), i.e. keys 32x that, cut at the row's causal bound p_i.
 * Layout: chunk_max, chunk_sum float32[B][q][6][NS][C], chunk_num
 * float32[B][q][6][NS][C][256] (the workspace layout when C = 1, so the
 * workspace buffers may be passed).  dfv_attn_split is this kernel followed,
 * when C > 1, by a merge of the C chunk states of each split in chunk order.
 * Alignment: q, k_cache, v_cache, chunk_num 16 bytes; others 4 bytes. */
DFV_API dfv_status dfv_attn_split_chunks(const dfv_attn_desc* desc, const void* q,
                                 const uint8_t* k_cache, const uint8_t* v_cache,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 const float* k_scale, const float* v_scale,
                                 float* chunk_max, float* chunk_sum, float* chunk_num,
                                 void* stream);

/* The split stage's second kernel on its own: merges the C chunk states of
 * every (row, split) written by dfv_attn_split_chunks, in chunk order, into
 * the workspace (ws_max, ws_sum, ws_num; the same values dfv_attn_split
 * writes) and, when out is not NULL, forms the FP16 output from exactly the
 * values written, as dfv_attn does ([#589] Test Result: one combine kernel
 * follows each attention kernel).  dfv_attn_split_chunks followed by this
 * call gives the bytes of dfv_attn.  With C = 1 the chunk states are copied
 * into the workspace, or, when chunk_num is ws_num (and then chunk_max is
 * ws_max and chunk_sum is ws_sum, else DFV_ERR_ARG), only read.  The chunk
 * buffers must not overlap the workspace otherwise.
 * Alignment: chunk_num, ws_num and out 16 bytes; others 4 bytes. */
DFV_API dfv_status dfv_attn_combine_chunks(const dfv_attn_desc* desc, const float* chunk_max,
                                   const float* chunk_sum, const float* chunk_num,
                                   float* ws_max, float* ws_sum, float* ws_num, void* out,
                                   void* stream);

/* Combine stage: merges the NS split states of every row into the FP16 output
 * ([#589] Test Result: one combine kernel follows each q8 attention kernel).
 * Reads only the workspace, so it can run on a saved workspace.
 * Alignment: ws_num and out 16 bytes; others 4 bytes. */
DFV_API dfv_status dfv_attn_combine(const dfv_attn_desc* desc, const float* ws_max,
                            const float* ws_sum, const float* ws_num, void* out,
                            void* stream);

/* Both stages on one stream: the results (workspace and FP16 out) are
 * byte-identical to dfv_attn_split followed by dfv_attn_combine; with C > 1
 * the chunk merge and the combine run as one kernel. */
DFV_API dfv_status dfv_attn(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                    const uint8_t* v_cache, const int32_t* block_table,
                    const int32_t* context_lens, const float* k_scale, const float* v_scale,
                    float* ws_max, float* ws_sum, float* ws_num, void* scratch,
                    size_t scratch_bytes, void* out, void* stream);

/* dfv_attn for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * and results as dfv_attn without the scratch pair.  The key-chunk states go
 * to a static device array of 16 MiB inside the library (each GPU holds its
 * own copy until the process ends), which covers every admitted descriptor
 * (at most 12,681,216 bytes); a descriptor needing more would return
 * DFV_ERR_SCRATCH.  The call allocates nothing; on its first use on a device
 * it looks up that device's array address (DFV_ERR_LAUNCH if the runtime
 * refuses).  Every call on one GPU shares that GPU's array, so calls that may
 * overlap in time on one GPU (other streams, other threads) race: serialize
 * them.  The array needs no initialisation between calls. */
DFV_API dfv_status dfv_attn_noalloc(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                            const uint8_t* v_cache, const int32_t* block_table,
                            const int32_t* context_lens, const float* k_scale, const float* v_scale,
                            float* ws_max, float* ws_sum, float* ws_num, void* out, void* stream);

/* QK stage on its own ([#589] Purpose: the QK producer the pages time by
 * itself, without softmax, PV or the split merge; [#589] Test Plan: checked
 * score by score and guard tile by guard tile before timing).  Computes
 *   s[b][r][t] = c * <Q[b, i, h, :], K_t>,   r = 6i + h,
 * in FP32 for whole 32-key tiles, stored tile-major:
 *   scores float32[B][tiles_per_seq][6q][32],  s[b][r][t] at [b][t/32][r][t%32].
 * Tile u of sequence b is written when it starts inside the context (u <
 * ceil(L_b / 32)); inside it, -inf where row r must not look (t > p_i, which
 * covers t >= L_b).  Tiles u >= ceil(L_b / 32) are guard tiles: never written,
 * they keep the caller's contents.  tiles_per_seq >= ceil(max_context_len / 32).
 * The descriptor is validated as for the other calls; its split fields are not
 * used.  v_cache, v_scale and the workspace play no part.
 * Alignment: q, k_cache, scores 16 bytes; block_table, context_lens, k_scale
 * 4 bytes. */
DFV_API dfv_status dfv_qk_scores(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                                 const int32_t* block_table, const int32_t* context_lens,
                                 const float* k_scale, float* scores, int64_t tiles_per_seq,
                                 void* stream);

/* Paged E4M3 KV append: writes the keys and values of num_tokens new tokens
 * (the q verification tokens of each sequence) into the caches, the step that
 * precedes the attention.  The pages keep the KV cache in E4M3 with per-tensor
 * scales ([#589] Test Plan; [#556] Test Plan: E4M3 target KV) without stating
 * the write; here every element is x / scale in FP32 (correctly rounded),
 * saturated to +-448, rounded to the nearest E4M3 code (ties to even; NaN
 * stays NaN) and stored at cache[slot / 16][slot % 16][0][d].
 *   k_new, v_new   FP16  [num_tokens][1][256]
 *   slot_mapping   int64 [num_tokens]; a slot outside [0, num_blocks * 16) is
 *                  padding and writes nothing (device values are not checked
 *                  on the host)
 *   k_scale, v_scale  device FP32 scalars
 *   k_cache, v_cache  uint8 [num_blocks][16][1][256]
 * Tokens with equal slots race (the last writer is unspecified).  num_tokens =
 * 0 launches nothing.  Alignment: k_new, v_new, k_cache, v_cache 16 bytes;
 * slot_mapping 8 bytes; scales 4 bytes. */
DFV_API dfv_status dfv_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                 int32_t num_tokens, const float* k_scale, const float* v_scale,
                                 uint8_t* k_cache, uint8_t* v_cache, int64_t num_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFV_H_ */
