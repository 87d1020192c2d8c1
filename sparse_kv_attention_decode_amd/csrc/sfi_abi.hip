// C ABI shell: argument validation, workspace sizing and launch of the SFI kernels.
// Every check runs on the host before anything is enqueued; see include/sfi.h.
#include "sfi_internal.h"

#include <math.h>
#include <stdint.h>

namespace {

using sfi::SplitPlan;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const sfi_shape* s) {
  if (!s) return SFI_E_ARG;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->head_dim < 1 ||
      s->page_size < 1 || s->max_pages_per_seq < 1)
    return SFI_E_ARG;
  if (s->num_q_heads % s->num_kv_heads != 0) return SFI_E_ARG;
  if (s->num_q_heads / s->num_kv_heads > sfi::kMaxGroup) return SFI_E_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return SFI_E_UNSUPPORTED;
  if (s->page_size != 16) return SFI_E_UNSUPPORTED;
  if (s->dtype != SFI_BF16 && s->dtype != SFI_F32) return SFI_E_UNSUPPORTED;
  return SFI_OK;
}

int check_params(const sfi_select_params* p) {
  if (!p) return SFI_E_ARG;
  if (p->n_sink < 0 || p->n_recent < 0 || p->top_k < 1 || p->nms_radius < 0) return SFI_E_ARG;
  // Written so that NaN fails every comparison.
  if (!(p->lambda >= 0.f && p->lambda <= 1.f)) return SFI_E_ARG;
  if (!(p->alpha_soft >= 0.f && p->alpha_soft <= 1.f)) return SFI_E_ARG;
  if (!(p->alpha_cross >= 0.f && p->alpha_cross <= 1.f)) return SFI_E_ARG;
  if (!(p->lambda_clip < 0.f || p->lambda_clip <= 1.f)) return SFI_E_ARG;  // NaN fails too
  if (p->nms_greedy != 0 && p->nms_greedy != 1) return SFI_E_ARG;
  if ((int64_t)p->n_sink + p->top_k > (1 << 28)) return SFI_E_CAPACITY;
  return SFI_OK;
}

int check_rows(const sfi_shape* s, int32_t n_seqs, int32_t max_seq_len) {
  if (n_seqs < 0 || n_seqs > s->batch) return SFI_E_ARG;
  if (max_seq_len < 1) return SFI_E_ARG;
  if ((int64_t)max_seq_len > (int64_t)s->max_pages_per_seq * 16) return SFI_E_CAPACITY;
  return SFI_OK;
}

int32_t packed_cap_of(const sfi_select_params* p) {
  return (int32_t)((((int64_t)p->n_sink + p->top_k) + 15) / 16 * 16);
}

int finish(hipError_t e) { return e == hipSuccess ? SFI_OK : SFI_E_HIP; }

}  // namespace

extern "C" {

int sfi_abi_version(void) { return SFI_ABI_VERSION; }

const char* sfi_status_str(int code) {
  switch (code) {
    case SFI_OK: return "ok";
    case SFI_E_ARG: return "invalid argument";
    case SFI_E_UNSUPPORTED: return "unsupported shape or dtype";
    case SFI_E_ALIGN: return "misaligned pointer or stride";
    case SFI_E_WORKSPACE: return "workspace missing or too small";
    case SFI_E_CAPACITY: return "length exceeds buffer or block-table capacity";
    case SFI_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int32_t sfi_packed_cap(const sfi_select_params* params) {
  if (check_params(params) != SFI_OK) return 0;
  return packed_cap_of(params);
}

size_t sfi_slow_attn_ws(const sfi_shape* shape, int32_t n_seqs, int32_t max_seq_len) {
  if (check_shape(shape) != SFI_OK || check_rows(shape, n_seqs, max_seq_len) != SFI_OK) return 0;
  const SplitPlan sp = sfi::plan_slow(*shape, n_seqs, max_seq_len);
  return sfi::partial_bytes(*shape, n_seqs, sp.nsplit);
}

size_t sfi_fast_attn_ws(const sfi_shape* shape, int32_t n_seqs, int32_t packed_cap,
                        int32_t max_recent) {
  if (check_shape(shape) != SFI_OK || n_seqs < 0 || n_seqs > shape->batch) return 0;
  if (packed_cap < 0 || packed_cap % 16 != 0 || max_recent < 0) return 0;
  const SplitPlan sp = sfi::plan_fast(*shape, n_seqs, packed_cap, max_recent);
  return sfi::partial_bytes(*shape, n_seqs, sp.nsplit);
}

size_t sfi_select_ws(const sfi_shape* shape, const sfi_select_params* params, int32_t n_seqs,
                     int32_t max_seq_len) {
  if (check_shape(shape) != SFI_OK || check_params(params) != SFI_OK ||
      check_rows(shape, n_seqs, max_seq_len) != SFI_OK || max_seq_len > sfi::kSelectMaxLen)
    return 0;
  return sfi::select_layout(*shape, n_seqs, max_seq_len, params->nms_greedy != 0).total;
}

int sfi_key_norms(const sfi_shape* shape, const void* k_cache, const int32_t* block_table,
                  const int32_t* seq_lens, const int32_t* seq_ids, int32_t n_seqs,
                  int32_t pos_begin, int32_t pos_end, float* key_norm, int64_t norm_stride,
                  void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!k_cache || !block_table || !seq_lens || !seq_ids || !key_norm) return SFI_E_ARG;
  if (n_seqs < 0 || n_seqs > shape->batch) return SFI_E_ARG;
  if (pos_begin < 0 || pos_end < pos_begin) return SFI_E_ARG;
  if ((int64_t)pos_end > (int64_t)shape->max_pages_per_seq * 16) return SFI_E_CAPACITY;
  if (norm_stride < pos_end) return SFI_E_CAPACITY;
  if (!aligned16(k_cache)) return SFI_E_ALIGN;
  if (n_seqs == 0 || pos_end == pos_begin) return SFI_OK;
  return finish(sfi::launch_key_norms(*shape, k_cache, block_table, seq_lens, seq_ids, n_seqs,
                                      pos_begin, pos_end, key_norm, norm_stride,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The model's shape with every query head repeated `window` times: the row layout of a
// windowed slow step.  Returns SFI_E_ARG for window < 1 and SFI_E_UNSUPPORTED when the
// repeated group exceeds the kernels' group limit.
int window_shape(const sfi_shape* shape, int32_t window, sfi_shape* out) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (window < 1) return SFI_E_ARG;
  if ((int64_t)(shape->num_q_heads / shape->num_kv_heads) * window > sfi::kMaxGroup)
    return SFI_E_UNSUPPORTED;
  *out = *shape;
  out->num_q_heads = shape->num_q_heads * window;
  return SFI_OK;
}

// Checks of a slow call of `shape` (already widened by the window) and its launch
// parameters in *p; the output is written for window slot 0 only.
int prep_slow(const sfi_shape* shape, int32_t window, const float* q, const void* k_cache,
              const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
              const int32_t* seq_ids, int32_t n_seqs, int32_t max_seq_len, float* out,
              float* logits, int64_t logits_stride, float* lse, uint32_t* status, void* ws,
              size_t ws_bytes, sfi::AttnParams* pp) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !seq_ids || !out || !lse)
    return SFI_E_ARG;
  if ((rc = check_rows(shape, n_seqs, max_seq_len))) return rc;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return SFI_E_ALIGN;
  if (logits) {
    if (!aligned16(logits) || logits_stride % 4 != 0) return SFI_E_ALIGN;
    if (logits_stride < max_seq_len) return SFI_E_CAPACITY;
  }
  const size_t need = sfi_slow_attn_ws(shape, n_seqs, max_seq_len);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SFI_E_WORKSPACE;
  sfi::AttnParams& p = *pp;
  p = {};
  p.n_seqs = n_seqs;
  if (n_seqs == 0) return SFI_OK;
  const SplitPlan sp = sfi::plan_slow(*shape, n_seqs, max_seq_len);
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.seq_ids = seq_ids;
  p.logits = logits;
  p.logits_stride = logits_stride;
  p.status = status;
  const size_t units = (size_t)n_seqs * shape->num_kv_heads * sp.nsplit *
                       (shape->num_q_heads / shape->num_kv_heads);
  const size_t ml = ((units * sizeof(float) + 255) / 256) * 256;
  p.part_m = reinterpret_cast<float*>(ws);
  p.part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ml);
  p.part_o = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 2 * ml);
  p.max_pages = shape->max_pages_per_seq;
  p.max_len = max_seq_len;
  p.n_seqs = n_seqs;
  p.Hq = shape->num_q_heads;
  p.Hkv = shape->num_kv_heads;
  p.G = p.Hq / p.Hkv;
  p.tps = sp.tps;
  p.tps_b = sp.tps;
  p.nsplit = sp.nsplit;
  p.nsplit_a = 0;
  p.fast = 0;
  p.win = window;
  p.scale = 1.0f / sqrtf((float)shape->head_dim);
  return SFI_OK;
}

int slow_attn(const sfi_shape* shape, int32_t window, const float* q, const void* k_cache,
              const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
              const int32_t* seq_ids, int32_t n_seqs, int32_t max_seq_len, float* out,
              float* logits, int64_t logits_stride, float* lse, uint32_t* status, void* ws,
              size_t ws_bytes, void* stream) {
  sfi::AttnParams p;
  const int rc = prep_slow(shape, window, q, k_cache, v_cache, block_table, seq_lens, seq_ids,
                           n_seqs, max_seq_len, out, logits, logits_stride, lse, status, ws,
                           ws_bytes, &p);
  if (rc || n_seqs == 0) return rc;
  return finish(sfi::launch_attention(p, shape->head_dim, shape->dtype, out, lse,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int sfi_slow_attn(const sfi_shape* shape, const float* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* seq_ids, int32_t n_seqs, int32_t max_seq_len, float* out,
                  float* logits, int64_t logits_stride, float* lse, uint32_t* status, void* ws,
                  size_t ws_bytes, void* stream) {
  return slow_attn(shape, 1, q, k_cache, v_cache, block_table, seq_lens, seq_ids, n_seqs,
                   max_seq_len, out, logits, logits_stride, lse, status, ws, ws_bytes, stream);
}

size_t sfi_slow_attn_window_ws(const sfi_shape* shape, int32_t window, int32_t n_seqs,
                               int32_t max_seq_len) {
  sfi_shape sw;
  if (window_shape(shape, window, &sw) != SFI_OK) return 0;
  return sfi_slow_attn_ws(&sw, n_seqs, max_seq_len);
}

int sfi_slow_attn_window(const sfi_shape* shape, int32_t window, const float* q_win,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* seq_ids, int32_t n_seqs,
                         int32_t max_seq_len, float* out, float* logits, int64_t logits_stride,
                         float* lse, uint32_t* status, void* ws, size_t ws_bytes,
                         void* stream) {
  sfi_shape sw;
  int rc = window_shape(shape, window, &sw);
  if (rc) return rc;
  return slow_attn(&sw, window, q_win, k_cache, v_cache, block_table, seq_lens, seq_ids, n_seqs,
                   max_seq_len, out, logits, logits_stride, lse, status, ws, ws_bytes, stream);
}

int sfi_select(const sfi_shape* shape, const sfi_select_params* params, const float* logits,
               int64_t logits_stride, const float* lse, const float* key_norm,
               int64_t norm_stride, const int32_t* seq_lens, const int32_t* seq_ids,
               int32_t n_seqs, int32_t max_seq_len, int32_t* sel_idx, float* dbg_scores,
               void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if (!logits || !lse || !key_norm || !seq_lens || !seq_ids || !sel_idx) return SFI_E_ARG;
  if ((rc = check_rows(shape, n_seqs, max_seq_len))) return rc;
  if (logits_stride < max_seq_len || norm_stride < max_seq_len) return SFI_E_CAPACITY;
  if (logits_stride % 4 != 0 || norm_stride % 4 != 0) return SFI_E_ALIGN;
  if (!aligned16(logits) || !aligned16(key_norm) || (dbg_scores && !aligned16(dbg_scores)))
    return SFI_E_ALIGN;
  if (params->nms_radius > 1024 || max_seq_len > sfi::kSelectMaxLen) return SFI_E_UNSUPPORTED;
  if (sfi::score_tile(shape->num_kv_heads, shape->num_q_heads, params->nms_radius) == 0)
    return SFI_E_UNSUPPORTED;
  const size_t need = sfi_select_ws(shape, params, n_seqs, max_seq_len);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SFI_E_WORKSPACE;
  if (n_seqs == 0) return SFI_OK;
  return finish(sfi::launch_select(*shape, *params, logits, logits_stride, lse, key_norm,
                                   norm_stride, seq_lens, seq_ids, n_seqs, max_seq_len, sel_idx,
                                   dbg_scores, ws, reinterpret_cast<hipStream_t>(stream)));
}

size_t sfi_select_window_ws(const sfi_shape* shape, const sfi_select_params* params,
                            int32_t window, int32_t n_seqs, int32_t max_seq_len) {
  sfi_shape sw;
  if (window_shape(shape, window, &sw) != SFI_OK) return 0;
  return sfi_select_ws(&sw, params, n_seqs, max_seq_len);
}

int sfi_select_window(const sfi_shape* shape, const sfi_select_params* params, int32_t window,
                      const float* logits, int64_t logits_stride, const float* lse,
                      const float* key_norm, int64_t norm_stride, const int32_t* seq_lens,
                      const int32_t* seq_ids, int32_t n_seqs, int32_t max_seq_len,
                      int32_t* sel_idx, float* dbg_scores, void* ws, size_t ws_bytes,
                      void* stream) {
  // The evidence of KV head g is the mean over its G * window rows: the Selector of the
  // widened shape computes exactly that.
  sfi_shape sw;
  int rc = window_shape(shape, window, &sw);
  if (rc) return rc;
  return sfi_select(&sw, params, logits, logits_stride, lse, key_norm, norm_stride, seq_lens,
                    seq_ids, n_seqs, max_seq_len, sel_idx, dbg_scores, ws, ws_bytes, stream);
}

size_t sfi_pack_update_ws(const sfi_shape* shape, const sfi_select_params* params,
                          int32_t n_seqs) {
  if (check_shape(shape) != SFI_OK || check_params(params) != SFI_OK) return 0;
  if (n_seqs < 0 || n_seqs > shape->batch) return 0;
  return sfi::pack_update_ws(*shape, *params, n_seqs);
}

int sfi_pack_update(const sfi_shape* shape, const sfi_select_params* params,
                    const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* sel_idx, const int32_t* seq_ids, int32_t n_seqs,
                    void* packed_k, void* packed_v, int32_t* packed_pos, int32_t* packed_len,
                    int32_t packed_cap, int32_t* slot_map, int64_t map_stride, uint32_t* status,
                    void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if (!k_cache || !v_cache || !block_table || !sel_idx || !seq_ids || !packed_k || !packed_v ||
      !packed_pos || !packed_len || !slot_map)
    return SFI_E_ARG;
  if (n_seqs < 0 || n_seqs > shape->batch) return SFI_E_ARG;
  if (packed_cap != packed_cap_of(params)) return SFI_E_CAPACITY;
  if (map_stride < params->n_sink || map_stride < 1) return SFI_E_CAPACITY;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(packed_k) || !aligned16(packed_v))
    return SFI_E_ALIGN;
  const size_t need = sfi_pack_update_ws(shape, params, n_seqs);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SFI_E_WORKSPACE;
  if (n_seqs == 0) return SFI_OK;
  return finish(sfi::launch_pack_update(*shape, *params, k_cache, v_cache, block_table, sel_idx,
                                        seq_ids, n_seqs, packed_k, packed_v, packed_pos,
                                        packed_len, packed_cap, slot_map, map_stride, status,
                                        ws, reinterpret_cast<hipStream_t>(stream)));
}

int sfi_pack(const sfi_shape* shape, const sfi_select_params* params, const void* k_cache,
             const void* v_cache, const int32_t* block_table, const int32_t* sel_idx,
             const int32_t* seq_ids, int32_t n_seqs, void* packed_k, void* packed_v,
             int32_t* packed_pos, int32_t* packed_len, int32_t packed_cap, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if (!k_cache || !v_cache || !block_table || !sel_idx || !seq_ids || !packed_k || !packed_v ||
      !packed_pos || !packed_len)
    return SFI_E_ARG;
  if (n_seqs < 0 || n_seqs > shape->batch) return SFI_E_ARG;
  if (packed_cap != packed_cap_of(params)) return SFI_E_CAPACITY;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(packed_k) || !aligned16(packed_v))
    return SFI_E_ALIGN;
  if (n_seqs == 0) return SFI_OK;
  return finish(sfi::launch_pack(*shape, *params, k_cache, v_cache, block_table, sel_idx,
                                 seq_ids, n_seqs, packed_k, packed_v, packed_pos, packed_len,
                                 packed_cap, reinterpret_cast<hipStream_t>(stream)));
}

int sfi_step_control(const sfi_shape* shape, const sfi_select_params* params,
                     int32_t refresh_budget, int32_t sliding_recent, const int32_t* token_ids,
                     const int32_t* boundary_tokens, int32_t n_boundary,
                     const int32_t* state_in, int32_t* state_out, int32_t* slow_ids,
                     int32_t* fast_ids, int32_t* counts, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if (refresh_budget < 0 || n_boundary < 0) return SFI_E_ARG;
  if (sliding_recent != 0 && sliding_recent != 1) return SFI_E_ARG;
  if (n_boundary > sfi::kMaxBoundaryTokens) return SFI_E_UNSUPPORTED;
  if (!token_ids || (n_boundary > 0 && !boundary_tokens) || !state_in || !state_out ||
      !slow_ids || !fast_ids || !counts)
    return SFI_E_ARG;
  return finish(sfi::launch_step_control(shape->batch, token_ids, boundary_tokens, n_boundary,
                                         refresh_budget, sliding_recent, params->n_sink,
                                         params->n_recent,
                                         state_in, state_out, slow_ids, fast_ids, counts,
                                         reinterpret_cast<hipStream_t>(stream)));
}

int sfi_kv_append(const sfi_shape* shape, const void* k_new, const void* v_new, void* k_cache,
                  void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* seq_ids, int32_t n_seqs, float* key_norm, int64_t norm_stride,
                  void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !seq_lens || !seq_ids)
    return SFI_E_ARG;
  if (n_seqs < 0 || n_seqs > shape->batch) return SFI_E_ARG;
  if (key_norm && norm_stride < 1) return SFI_E_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return SFI_E_ALIGN;
  if (n_seqs == 0) return SFI_OK;
  return finish(sfi::launch_kv_append(*shape, k_new, v_new, k_cache, v_cache, block_table,
                                      seq_lens, seq_ids, n_seqs, key_norm, norm_stride,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of a fast call and its launch parameters in *p.
int prep_fast(const sfi_shape* shape, const float* q, const void* packed_k, const void* packed_v,
              const int32_t* packed_len, int32_t packed_cap, const void* k_cache,
              const void* v_cache, const int32_t* block_table, const int32_t* recent_start,
              const int32_t* seq_lens, const int32_t* seq_ids, int32_t n_seqs,
              int32_t max_recent, float* out, uint32_t* status, void* ws, size_t ws_bytes,
              sfi::AttnParams* pp) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !packed_k || !packed_v || !packed_len || !k_cache || !v_cache || !block_table ||
      !recent_start || !seq_lens || !seq_ids || !out)
    return SFI_E_ARG;
  if (n_seqs < 0 || n_seqs > shape->batch) return SFI_E_ARG;
  if (packed_cap < 16 || packed_cap % 16 != 0) return SFI_E_CAPACITY;
  if (max_recent < 0) return SFI_E_ARG;
  if ((int64_t)max_recent > (int64_t)shape->max_pages_per_seq * 16) return SFI_E_CAPACITY;
  if (!aligned16(q) || !aligned16(packed_k) || !aligned16(packed_v) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out))
    return SFI_E_ALIGN;
  const size_t need = sfi_fast_attn_ws(shape, n_seqs, packed_cap, max_recent);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SFI_E_WORKSPACE;
  sfi::AttnParams& p = *pp;
  p = {};
  p.n_seqs = n_seqs;
  if (n_seqs == 0) return SFI_OK;
  const SplitPlan sp = sfi::plan_fast(*shape, n_seqs, packed_cap, max_recent);
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.seq_ids = seq_ids;
  p.packed_k = packed_k;
  p.packed_v = packed_v;
  p.packed_len = packed_len;
  p.recent_start = recent_start;
  p.logits = nullptr;
  p.status = status;
  const size_t units = (size_t)n_seqs * shape->num_kv_heads * sp.nsplit *
                       (shape->num_q_heads / shape->num_kv_heads);
  const size_t ml = ((units * sizeof(float) + 255) / 256) * 256;
  p.part_m = reinterpret_cast<float*>(ws);
  p.part_l = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ml);
  p.part_o = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + 2 * ml);
  p.max_pages = shape->max_pages_per_seq;
  p.max_len = shape->max_pages_per_seq * 16;
  p.packed_cap = packed_cap;
  p.Hq = shape->num_q_heads;
  p.Hkv = shape->num_kv_heads;
  p.G = p.Hq / p.Hkv;
  p.tps = sp.tps;
  p.tps_b = sp.tps_b;
  p.nsplit = sp.nsplit;
  p.nsplit_a = sp.nsplit_a;
  p.fast = 1;
  p.win = 1;
  p.scale = 1.0f / sqrtf((float)shape->head_dim);
  return SFI_OK;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

extern "C" {

int sfi_fast_attn(const sfi_shape* shape, const float* q, const void* packed_k,
                  const void* packed_v, const int32_t* packed_len, int32_t packed_cap,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* recent_start, const int32_t* seq_lens, const int32_t* seq_ids,
                  int32_t n_seqs, int32_t max_recent, float* out, float* lse, uint32_t* status,
                  void* ws, size_t ws_bytes, void* stream) {
  sfi::AttnParams p;
  const int rc = prep_fast(shape, q, packed_k, packed_v, packed_len, packed_cap, k_cache,
                           v_cache, block_table, recent_start, seq_lens, seq_ids, n_seqs,
                           max_recent, out, status, ws, ws_bytes, &p);
  if (rc || n_seqs == 0) return rc;
  return finish(sfi::launch_attention(p, shape->head_dim, shape->dtype, out, lse,
                                      reinterpret_cast<hipStream_t>(stream)));
}

size_t sfi_decode_attn_ws(const sfi_shape* shape, int32_t window, int32_t n_seqs,
                          int32_t packed_cap, int32_t max_recent, int32_t max_seq_len) {
  const size_t f = sfi_fast_attn_ws(shape, n_seqs, packed_cap, max_recent);
  const size_t sl = sfi_slow_attn_window_ws(shape, window, n_seqs, max_seq_len);
  if (f == 0 || sl == 0) return 0;
  return round256(f) + sl;
}

int sfi_decode_attn(const sfi_shape* shape, int32_t window, const float* q,
                    const float* q_win, const void* packed_k, const void* packed_v,
                    const int32_t* packed_len, int32_t packed_cap, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* recent_start, const int32_t* seq_lens,
                    const int32_t* fast_ids, const int32_t* slow_ids, int32_t n_seqs,
                    int32_t max_recent, int32_t max_seq_len, float* out, float* logits,
                    int64_t logits_stride, float* lse, uint32_t* status, void* ws,
                    size_t ws_bytes, void* stream) {
  sfi_shape sw;
  int rc = window_shape(shape, window, &sw);
  if (rc) return rc;
  const size_t need = sfi_decode_attn_ws(shape, window, n_seqs, packed_cap, max_recent,
                                         max_seq_len);
  // (need == 0: an invalid argument, which the checks below name)
  if (need != 0 && (!ws || ws_bytes < need)) return SFI_E_WORKSPACE;
  const size_t wf = round256(sfi_fast_attn_ws(shape, n_seqs, packed_cap, max_recent));
  char* w8 = reinterpret_cast<char*>(ws);
  sfi::AttnParams pf, ps;
  if ((rc = prep_fast(shape, q, packed_k, packed_v, packed_len, packed_cap, k_cache, v_cache,
                      block_table, recent_start, seq_lens, fast_ids, n_seqs, max_recent, out,
                      status, ws, wf, &pf)))
    return rc;
  if ((rc = prep_slow(&sw, window, q_win, k_cache, v_cache, block_table, seq_lens, slow_ids,
                      n_seqs, max_seq_len, out, logits, logits_stride, lse, status, w8 + wf,
                      ws_bytes - wf, &ps)))
    return rc;
  if (n_seqs == 0) return SFI_OK;
  return finish(sfi::launch_attention_pair(pf, ps, shape->head_dim, shape->dtype, out, lse,
                                           reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
