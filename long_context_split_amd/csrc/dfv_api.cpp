// C ABI of the gfx950 DFlash2 verification-attention library (see include/dfv.h).
//
// Host-side admission mirrors the pages' shape-guarded operator selection: only
// the admitted shapes are launched, anything else is refused before any device
// work so the caller keeps its own operator ([#556] "[Perf] Add opt-in DFlash2
// schedules and numerical audits", Purpose; [#587] "[Perf] Reduce DFlash2
// long-context verification decay", Implementation).
#include "dfv.h"

#include <math.h>

#include "dfv_common.h"
#include "dfv_append.h"
#include "dfv_qk.h"

namespace {

using dfv::kHeadDim;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

dfv_status check_desc(const dfv_attn_desc* d) {
  if (!d) return DFV_ERR_NULL;
  if (d->num_q_heads != dfv::kQHeads || d->num_kv_heads != 1 || d->head_dim != kHeadDim ||
      d->block_size != dfv::kPage)
    return DFV_ERR_UNSUPPORTED;
  if (d->num_q < 1 || d->num_q > dfv::kMaxQ) return DFV_ERR_UNSUPPORTED;
  if (d->num_splits < 1 || d->num_splits > dfv::kMaxSplits) return DFV_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->max_blocks_per_seq < 1) return DFV_ERR_ARG;
  if ((long long)d->batch * d->num_splits > (1LL << 20)) return DFV_ERR_ARG;
  if (d->max_context_len < d->num_q || d->max_context_len > dfv::kMaxContext) return DFV_ERR_ARG;
  if ((long long)d->max_context_len > 16LL * d->max_blocks_per_seq) return DFV_ERR_ARG;
  if (d->split_tokens < 0 || d->split_tokens % dfv::kTile != 0) return DFV_ERR_ARG;
  if (d->split_tokens > 0 && (long long)d->split_tokens * d->num_splits < d->max_context_len)
    return DFV_ERR_ARG;
  if (!(d->softmax_scale > 0.0f) || !isfinite(d->softmax_scale)) return DFV_ERR_ARG;
  return DFV_OK;
}

// Scratch the split kernel needs: the key-chunk states when a split is cut into
// several chunks (zero otherwise).
size_t scratch_need(const dfv_attn_desc* d) {
  return dfv::scratch_bytes(d->batch, d->num_q, d->num_splits);
}

dfv_status check_split_ptrs(const void* q, const uint8_t* kc, const uint8_t* vc, const int32_t* bt,
                            const int32_t* cl, const float* ks, const float* vs, const float* wm,
                            const float* wl, const float* wn, const void* scratch) {
  if (!q || !kc || !vc || !bt || !cl || !ks || !vs || !wm || !wl || !wn) return DFV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(wn, 16) || !aligned(bt, 4) ||
      !aligned(cl, 4) || !aligned(ks, 4) || !aligned(vs, 4) || !aligned(wm, 4) || !aligned(wl, 4) ||
      !aligned(scratch, 256))
    return DFV_ERR_ALIGN;
  return DFV_OK;
}

dfv_status check_combine_ptrs(const float* wm, const float* wl, const float* wn, const void* out) {
  if (!wm || !wl || !wn || !out) return DFV_ERR_NULL;
  if (!aligned(wn, 16) || !aligned(out, 16) || !aligned(wm, 4) || !aligned(wl, 4)) return DFV_ERR_ALIGN;
  return DFV_OK;
}

// Where the chunk states of the split kernel live inside the scratch buffer.
struct ChunkStates {
  int chunks;
  float* num;
  float* max;
  float* sum;
};

ChunkStates chunk_states(const dfv_attn_desc* d, void* scratch) {
  ChunkStates c;
  c.chunks = dfv::split_chunks(d->batch, d->num_splits);
  if (c.chunks == 1) scratch = nullptr;   // one chunk: the split kernel writes the workspace itself
  const size_t n = dfv::scratch_floats(d->batch * d->num_q * dfv::kQHeads, d->num_splits, c.chunks);
  c.num = (float*)scratch;
  c.max = c.num ? c.num + n * kHeadDim : nullptr;
  c.sum = c.max ? c.max + n : nullptr;
  return c;
}

dfv_status launch_split_checked(const dfv_attn_desc* d, const void* q, const uint8_t* kc,
                                const uint8_t* vc, const int32_t* bt, const int32_t* cl,
                                const float* ks, const float* vs, float* wm, float* wl, float* wn,
                                const ChunkStates& cs, hipStream_t stream) {
  dfv::SplitArgs a;
  a.q = (const _Float16*)q;
  a.k_cache = kc;
  a.v_cache = vc;
  a.block_table = bt;
  a.context_lens = cl;
  a.k_scale = ks;
  a.v_scale = vs;
  a.chunks = cs.chunks;
  a.st_max = cs.chunks > 1 ? cs.max : wm;
  a.st_sum = cs.chunks > 1 ? cs.sum : wl;
  a.st_num = cs.chunks > 1 ? cs.num : wn;   // with one chunk the states are the workspace
  a.batch = d->batch;
  a.num_q = d->num_q;
  a.max_blocks = d->max_blocks_per_seq;
  a.num_splits = d->num_splits;
  a.split_tokens = d->split_tokens;
  a.max_context_len = d->max_context_len;
  a.softmax_scale = d->softmax_scale;
  return dfv::launch_split(a, stream) == hipSuccess ? DFV_OK : DFV_ERR_LAUNCH;
}

// Merge of chunk states into the workspace (chunks > 1, or one chunk held in
// buffers other than the workspace: then a copy), and/or the combine into
// `out` (out != NULL).  With the workspace as the only states and out = NULL
// there is nothing to do.
dfv_status launch_combine_checked(const dfv_attn_desc* d, const ChunkStates& cs, float* wm, float* wl,
                                  float* wn, void* out, hipStream_t stream) {
  // With one chunk the states are the workspace unless the caller named other buffers.
  const bool own = cs.chunks > 1 || (cs.num && cs.num != wn);
  if (!own && !out) return DFV_OK;
  dfv::CombineArgs a;
  a.chunks = cs.chunks;
  a.src_max = own ? cs.max : wm;
  a.src_sum = own ? cs.sum : wl;
  a.src_num = own ? cs.num : wn;
  a.ws_max = wm;
  a.ws_sum = wl;
  a.ws_num = wn;
  a.write_ws = own;
  a.out = (_Float16*)out;
  a.rows = d->batch * d->num_q * dfv::kQHeads;
  a.num_splits = d->num_splits;
  return dfv::launch_combine(a, stream) == hipSuccess ? DFV_OK : DFV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char* dfv_status_string(int status) {
  switch (status) {
    case DFV_OK: return "DFV_OK";
    case DFV_ERR_NULL: return "DFV_ERR_NULL: required pointer is NULL";
    case DFV_ERR_UNSUPPORTED: return "DFV_ERR_UNSUPPORTED: shape outside the admitted set";
    case DFV_ERR_ALIGN: return "DFV_ERR_ALIGN: pointer misaligned";
    case DFV_ERR_ARG: return "DFV_ERR_ARG: inconsistent size or count";
    case DFV_ERR_LAUNCH: return "DFV_ERR_LAUNCH: kernel launch failed";
    case DFV_ERR_SCRATCH: return "DFV_ERR_SCRATCH: scratch buffer too small";
    default: return "unknown dfv status";
  }
}

dfv_status dfv_attn_check(const dfv_attn_desc* desc) { return check_desc(desc); }

dfv_status dfv_attn_scratch_bytes(const dfv_attn_desc* desc, size_t* bytes) {
  if (!bytes) return DFV_ERR_NULL;
  *bytes = 0;
  const dfv_status s = check_desc(desc);
  if (s == DFV_OK) *bytes = scratch_need(desc);
  return s;
}

size_t dfv_attn_workspace_bytes(const dfv_attn_desc* desc) {
  if (check_desc(desc) != DFV_OK) return 0;
  const size_t states = (size_t)desc->batch * desc->num_q * dfv::kQHeads * desc->num_splits;
  return states * (2 + kHeadDim) * sizeof(float) + scratch_need(desc);
}

dfv_status dfv_attn_split(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                          const uint8_t* v_cache, const int32_t* block_table,
                          const int32_t* context_lens, const float* k_scale, const float* v_scale,
                          float* ws_max, float* ws_sum, float* ws_num, void* scratch,
                          size_t scratch_bytes, void* stream) {
  dfv_status s = check_desc(desc);
  if (s != DFV_OK) return s;
  s = check_split_ptrs(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, ws_max,
                       ws_sum, ws_num, scratch);
  if (s != DFV_OK) return s;
  if (scratch_bytes < scratch_need(desc) || (scratch_need(desc) && !scratch)) return DFV_ERR_SCRATCH;
  const ChunkStates cs = chunk_states(desc, scratch);
  s = launch_split_checked(desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                           ws_max, ws_sum, ws_num, cs, (hipStream_t)stream);
  if (s != DFV_OK) return s;
  return launch_combine_checked(desc, cs, ws_max, ws_sum, ws_num, nullptr, (hipStream_t)stream);
}

dfv_status dfv_attn_chunks(const dfv_attn_desc* desc, int32_t* chunks) {
  if (!chunks) return DFV_ERR_NULL;
  *chunks = 0;
  const dfv_status s = check_desc(desc);
  if (s == DFV_OK) *chunks = dfv::split_chunks(desc->batch, desc->num_splits);
  return s;
}

dfv_status dfv_attn_split_chunks(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                                 const uint8_t* v_cache, const int32_t* block_table,
                                 const int32_t* context_lens, const float* k_scale,
                                 const float* v_scale, float* chunk_max, float* chunk_sum,
                                 float* chunk_num, void* stream) {
  dfv_status s = check_desc(desc);
  if (s != DFV_OK) return s;
  s = check_split_ptrs(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, chunk_max,
                       chunk_sum, chunk_num, nullptr);
  if (s != DFV_OK) return s;
  ChunkStates cs{dfv::split_chunks(desc->batch, desc->num_splits), chunk_num, chunk_max, chunk_sum};
  return launch_split_checked(desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                              chunk_max, chunk_sum, chunk_num, cs, (hipStream_t)stream);
}

dfv_status dfv_attn_combine_chunks(const dfv_attn_desc* desc, const float* chunk_max,
                                   const float* chunk_sum, const float* chunk_num, float* ws_max,
                                   float* ws_sum, float* ws_num, void* out, void* stream) {
  dfv_status s = check_desc(desc);
  if (s != DFV_OK) return s;
  if (!chunk_max || !chunk_sum || !chunk_num || !ws_max || !ws_sum || !ws_num) return DFV_ERR_NULL;
  if (!aligned(chunk_num, 16) || !aligned(ws_num, 16) || !aligned(chunk_max, 4) || !aligned(chunk_sum, 4) ||
      !aligned(ws_max, 4) || !aligned(ws_sum, 4) || !aligned(out, 16))
    return DFV_ERR_ALIGN;
  ChunkStates cs{dfv::split_chunks(desc->batch, desc->num_splits), (float*)chunk_num, (float*)chunk_max,
                 (float*)chunk_sum};
  // One chunk per split: the chunk states are split states; they are copied into
  // the workspace unless they already are the workspace.
  if (cs.chunks == 1 && cs.num == ws_num && (cs.max != ws_max || cs.sum != ws_sum)) return DFV_ERR_ARG;
  return launch_combine_checked(desc, cs, ws_max, ws_sum, ws_num, out, (hipStream_t)stream);
}

dfv_status dfv_attn_combine(const dfv_attn_desc* desc, const float* ws_max, const float* ws_sum,
                            const float* ws_num, void* out, void* stream) {
  dfv_status s = check_desc(desc);
  if (s != DFV_OK) return s;
  s = check_combine_ptrs(ws_max, ws_sum, ws_num, out);
  if (s != DFV_OK) return s;
  ChunkStates cs{1, (float*)ws_num, (float*)ws_max, (float*)ws_sum};
  // With one chunk whose states are the workspace itself, the workspace is only read.
  return launch_combine_checked(desc, cs, (float*)ws_max, (float*)ws_sum, (float*)ws_num, out,
                                (hipStream_t)stream);
}

dfv_status dfv_attn(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                    const uint8_t* v_cache, const int32_t* block_table, const int32_t* context_lens,
                    const float* k_scale, const float* v_scale, float* ws_max, float* ws_sum,
                    float* ws_num, void* scratch, size_t scratch_bytes, void* out, void* stream) {
  dfv_status s = check_desc(desc);
  if (s != DFV_OK) return s;
  s = check_split_ptrs(q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale, ws_max,
                       ws_sum, ws_num, scratch);
  if (s != DFV_OK) return s;
  s = check_combine_ptrs(ws_max, ws_sum, ws_num, out);
  if (s != DFV_OK) return s;
  if (scratch_bytes < scratch_need(desc) || (scratch_need(desc) && !scratch)) return DFV_ERR_SCRATCH;
  const ChunkStates cs = chunk_states(desc, scratch);
  s = launch_split_checked(desc, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
                           ws_max, ws_sum, ws_num, cs, (hipStream_t)stream);
  if (s != DFV_OK) return s;
  return launch_combine_checked(desc, cs, ws_max, ws_sum, ws_num, out, (hipStream_t)stream);
}

dfv_status dfv_qk_scores(const dfv_attn_desc* desc, const void* q, const uint8_t* k_cache,
                         const int32_t* block_table, const int32_t* context_lens, const float* k_scale,
                         float* scores, int64_t tiles_per_seq, void* stream) {
  dfv_status s = check_desc(desc);
  if (s != DFV_OK) return s;
  if (!q || !k_cache || !block_table || !context_lens || !k_scale || !scores) return DFV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(scores, 16) || !aligned(block_table, 4) ||
      !aligned(context_lens, 4) || !aligned(k_scale, 4))
    return DFV_ERR_ALIGN;
  const long long tiles = (desc->max_context_len + dfv::kTile - 1) / dfv::kTile;
  if (tiles_per_seq < tiles) return DFV_ERR_ARG;
  dfv::QkArgs a;
  a.q = (const _Float16*)q;
  a.k_cache = k_cache;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k_scale = k_scale;
  a.scores = scores;
  a.tiles_per_seq = tiles_per_seq;
  a.batch = desc->batch;
  a.num_q = desc->num_q;
  a.max_blocks = desc->max_blocks_per_seq;
  a.max_context_len = desc->max_context_len;
  a.softmax_scale = desc->softmax_scale;
  return dfv::launch_qk(a, (hipStream_t)stream) == hipSuccess ? DFV_OK : DFV_ERR_LAUNCH;
}

dfv_status dfv_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                         int32_t num_tokens, const float* k_scale, const float* v_scale,
                         uint8_t* k_cache, uint8_t* v_cache, int64_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_blocks < 1 || num_blocks > (1LL << 40)) return DFV_ERR_ARG;
  if (num_tokens > (1 << 28)) return DFV_ERR_ARG;
  if (!k_new || !v_new || !slot_mapping || !k_scale || !v_scale || !k_cache || !v_cache)
    return DFV_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return DFV_ERR_ALIGN;
  dfv::AppendArgs a;
  a.k_new = (const _Float16*)k_new;
  a.v_new = (const _Float16*)v_new;
  a.slot_mapping = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_slots = num_blocks * dfv::kPage;
  a.num_tokens = num_tokens;
  return dfv::launch_kv_append(a, (hipStream_t)stream) == hipSuccess ? DFV_OK : DFV_ERR_LAUNCH;
}

}  // extern "C"
