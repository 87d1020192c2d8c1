// Host-side interfaces between the C ABI shell and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sfi.h"

namespace sfi {

constexpr int kMaxGroup = 16;  // query heads per KV head supported by the kernels

// Work decomposition of one attention call: every (listed row, KV head) pair is cut into
// `nsplit` splits of `tps` 16-row tiles; each split is one wavefront.  For a fast call the
// first `nsplit_a` splits cover the packed segment and the rest the recent segment.
struct SplitPlan {
  int tps = 0;
  int tps_b = 0;  // fast calls: tiles per split of the paged (recent) segment
  int nsplit = 0;
  int nsplit_a = 0;
};

SplitPlan plan_slow(const sfi_shape& s, int n_seqs, int max_seq_len);
SplitPlan plan_fast(const sfi_shape& s, int n_seqs, int packed_cap, int max_recent);
// Bytes of the per-split partial results (m, l, o) of one attention call.
size_t partial_bytes(const sfi_shape& s, int n_seqs, int nsplit);

struct AttnParams {
  const float* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  const void* packed_k;        // fast only
  const void* packed_v;        // fast only
  const int32_t* packed_len;   // fast only
  const int32_t* recent_start; // fast only
  float* logits;               // slow only, may be null
  uint32_t* status;            // device contract flags (sfi_device_status), may be null
  int64_t logits_stride;
  float* part_m;
  float* part_l;
  float* part_o;
  int max_pages;
  int max_len;                 // row lengths are clamped to this (slow: max_seq_len; fast:
                               // the page table's span), so no index leaves the buffers
  int packed_cap;
  int n_seqs, Hq, Hkv, G;
  int tps, nsplit, nsplit_a;
  int tps_b;                   // fast only: tiles per split of the paged (recent) segment
  int fast;
  int win;                     // query-window slots per head (1: no window)
  float scale;
};

hipError_t launch_attention(const AttnParams& p, int head_dim, int dtype, float* out,
                            float* lse, hipStream_t stream);
// A fast call (pf, no lse) and a slow call (ps) in one partial and one merge launch; both
// write `out`, for the rows of their own lists.
hipError_t launch_attention_pair(const AttnParams& pf, const AttnParams& ps, int head_dim,
                                 int dtype, float* out, float* lse_slow, hipStream_t stream);

hipError_t launch_key_norms(const sfi_shape& s, const void* k_cache,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* seq_ids, int n_seqs, int pos_begin, int pos_end,
                            float* key_norm, int64_t norm_stride, hipStream_t stream);

struct SelectLayout {
  int nchunk = 0;        // prior-normaliser chunks per (row, KV head)
  int64_t kstride = 0;   // key slots per (row, KV head)
  int nslice = 0;        // top-K slices of 4096 candidates per (row, KV head)
  size_t zpart_off = 0, hpart_off = 0, taken_off = 0, ready_off = 0, keys_off = 0, hist_off = 0, state_off = 0, above_off = 0,
         sloff_off = 0, ckey_off = 0, cidx_off = 0, total = 0;
};
// Longest KV length the Selector takes: 1024 top-K slices of 4096 candidates.
constexpr int kSelectMaxLen = 1 << 22;
SelectLayout select_layout(const sfi_shape& s, int n_seqs, int max_seq_len, bool greedy);
// LDS of one scoring block: s for every KV head over `tile` positions plus a halo of
// nms_radius on each side, the prior normalisers and the lse of every query head.
size_t score_lds_bytes(int num_kv_heads, int num_q_heads, int nms_radius, int tile);
constexpr size_t kScoreLdsLimit = 64 * 1024;
// Scoring tile: 256 - 2 nms_radius positions (one position per thread with the halo)
// when the radius is at most 96, else 64; 0 if its LDS does not fit.
int score_tile(int num_kv_heads, int num_q_heads, int nms_radius);

hipError_t launch_select(const sfi_shape& s, const sfi_select_params& prm,
                         const float* logits, int64_t logits_stride, const float* lse,
                         const float* key_norm, int64_t norm_stride, const int32_t* seq_lens,
                         const int32_t* seq_ids, int n_seqs, int max_seq_len,
                         int32_t* sel_idx, float* dbg_scores, void* ws, hipStream_t stream);

hipError_t launch_step_control(int batch, const int32_t* tokens, const int32_t* boundary,
                               int n_boundary, int budget, int sliding, int n_sink, int n_recent,
                               const int32_t* state_in, int32_t* state_out, int32_t* slow_ids,
                               int32_t* fast_ids, int32_t* counts, hipStream_t stream);
// Longest boundary-token table sfi_step_control takes.
constexpr int kMaxBoundaryTokens = 1024;

hipError_t launch_kv_append(const sfi_shape& s, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* seq_ids, int n_seqs,
                            float* key_norm, int64_t norm_stride, hipStream_t stream);

// Workspace of the incremental pack and its launch (both kernels).
size_t pack_update_ws(const sfi_shape& s, const sfi_select_params& prm, int n_seqs);
hipError_t launch_pack_update(const sfi_shape& s, const sfi_select_params& prm,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* sel_idx,
                              const int32_t* seq_ids, int n_seqs, void* packed_k, void* packed_v,
                              int32_t* packed_pos, int32_t* packed_len, int packed_cap,
                              int32_t* slot_map, int64_t map_stride, uint32_t* status, void* ws,
                              hipStream_t stream);

hipError_t launch_pack(const sfi_shape& s, const sfi_select_params& prm, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* sel_idx,
                       const int32_t* seq_ids, int n_seqs, void* packed_k, void* packed_v,
                       int32_t* packed_pos, int32_t* packed_len, int packed_cap,
                       hipStream_t stream);

}  // namespace sfi
