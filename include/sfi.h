/*
 * sfi.h -- C ABI of the Slow-Fast Inference (SFI) decode path on MI355X (gfx950).
 *
 * The method (pages: "Slow-Fast Inference: Training-Free Inference Acceleration via
 * Within-Sentence Support Stability", cited by summary language and section):
 *   - slow steps run dense attention over the whole history and hand their attention
 *     evidence to the Selector (es "2. Metodología", zh "2.1 慢快推理框架");
 *   - the Selector fuses that evidence f with a cached-statistics prior r as
 *     s = (1-λ) f + λ r, refines the log-scores with soft-NMS and cross-head exclusivity
 *     and takes a Top-K per head (zh "2.2 训练无感的 Selector", nl "De Selector");
 *   - sink and selected rows are packed into a contiguous buffer; fast steps attend to
 *     that buffer plus the recent window read from the paged cache (zh "2.3 系统级优化",
 *     nl "Systeemontwerp en Kernel-optimalisatie").
 *
 * Conventions shared by every entry point
 *   Memory     Every pointer argument except `shape`/`params` is DEVICE memory owned by
 *              the caller.  The library never allocates, frees or retains memory and
 *              keeps no mutable global state; it is safe to call from several threads on
 *              different streams.  The one exception is sfi_fast_attn_noalloc, whose
 *              scratch is a device array inside the library (see there).
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *              work and never synchronise; buffers must stay alive until the stream has
 *              passed the work.
 *   Batch rows `seq_ids[0..n_seqs)` (device, int32) lists the batch rows b a call serves,
 *              so one decode step can send slow and fast sequences to different calls.
 *              Per-row tensors are indexed by b.  n_seqs == 0 is a no-op returning SFI_OK.
 *              A negative entry marks an unused slot: every call skips it and writes
 *              nothing for it, so the -1-padded lists of sfi_step_control can be passed
 *              whole (n_seqs = batch) without the host reading the counts.
 *   Errors     Host-side checks run before anything is enqueued and return a negative
 *              code with nothing enqueued.  After enqueueing, a launch failure reported
 *              by hipGetLastError is returned as SFI_E_HIP.  Device-side contracts (seq
 *              lengths within bounds, valid pages, indices in range) are trusted, with
 *              one safeguard: the attention calls clamp seq_lens to max_seq_len (slow)
 *              or to the page table's span (fast), packed_len to [0, packed_cap] and
 *              recent_start to [0, N], so such a value cannot index past their buffers
 *              (the results for that row are then unspecified).
 *   Layouts    (all row-major, innermost last)
 *     q            f32  [batch, Hq, D]
 *     k_cache      elt  [num_pages, Hkv, 16, D]   page p holds 16 consecutive positions
 *     v_cache      elt  [num_pages, Hkv, 16, D]
 *     block_table  i32  [batch, max_pages_per_seq]  position j of row b lives in physical
 *                       page block_table[b][j / 16], slot j % 16
 *     seq_lens     i32  [batch]   KV length N_b; position N_b-1 is the current token
 *     out          f32  [batch, Hq, D]
 *     lse          f32  [batch, Hq]   natural-log partition function of the logits
 *     logits       f32  [batch, Hq, logits_stride]  z = q·k / sqrt(D)
 *     key_norm     f32  [batch, Hkv, norm_stride]   ||k||_2 of every stored key row
 *     sel_idx      i32  [batch, Hkv, top_k]   ascending positions, then -1 padding
 *     packed_k/v   elt  [batch, Hkv, packed_cap, D]   packed_cap = round_up(n_sink+top_k, 16)
 *     packed_pos   i32  [batch, Hkv, packed_cap]
 *     packed_len   i32  [batch, Hkv]
 *     recent_start i32  [batch]
 *   Query head h reads KV head h / G, G = Hq / Hkv.  "elt" is bf16 or f32 per
 *   sfi_shape.dtype.  q, K/V, packed and out pointers must be 16-byte aligned;
 *   logits/key_norm strides must be multiples of 4 elements.
 */
#ifndef SFI_H
#define SFI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFI_ABI_VERSION 8

enum sfi_status {
  SFI_OK = 0,
  SFI_E_ARG = -1,          /* NULL pointer, non-positive dims, Hq % Hkv != 0, bad params  */
  SFI_E_UNSUPPORTED = -2,  /* D not in {64,128}, dtype, G > 16, page_size != 16          */
  SFI_E_ALIGN = -3,        /* a pointer or stride breaks the alignment rules above       */
  SFI_E_WORKSPACE = -4,    /* workspace NULL or smaller than the matching *_ws() query   */
  SFI_E_CAPACITY = -5,     /* a length exceeds what the buffers or block table can hold  */
  SFI_E_HIP = -6           /* a kernel launch failed                                     */
};

enum sfi_dtype { SFI_BF16 = 0, SFI_F32 = 1 };

/* Device-side contract violations.  The attention calls and sfi_pack_update take a
 * `status` pointer (device memory, uint32, may be NULL): a kernel that finds a contract of
 * its call broken ORs the matching bit into *status and carries on with the documented
 * safeguard, so the host can see afterwards that the results of those rows are
 * unspecified.  The library never clears *status; a caller that wants fresh flags zeroes
 * it first.  The checks cost a few scalar loads per (row, KV head). */
enum sfi_device_status {
  SFI_DEV_SEQ_LEN = 1u,     /* a row length outside [0, the call's bound]: clamped          */
  SFI_DEV_PACKED_LEN = 2u,  /* packed_len outside [0, packed_cap]: clamped                  */
  SFI_DEV_RECENT = 4u,      /* recent_start outside [0, N], or a recent segment longer than
                               max_recent: clamped / truncated                             */
  SFI_DEV_PACK_SLOT = 8u    /* the incremental pack placed a row outside the buffer (state
                               not maintained by these calls): that row was not written    */
};

typedef struct {
  int32_t batch;              /* rows of block_table / seq_lens                           */
  int32_t num_q_heads;        /* Hq                                                       */
  int32_t num_kv_heads;       /* Hkv, Hq % Hkv == 0 and G = Hq / Hkv <= 16               */
  int32_t head_dim;           /* D in {64, 128}                                           */
  int32_t page_size;          /* must be 16                                               */
  int32_t max_pages_per_seq;  /* columns of block_table                                   */
  int32_t dtype;              /* enum sfi_dtype: element type of every K/V buffer         */
} sfi_shape;

typedef struct {
  int32_t n_sink;       /* sink rows [0, n_sink) always in the fast memory (>= 0)         */
  int32_t n_recent;     /* recent window W: candidates are [n_sink, N - W) (>= 0)         */
  int32_t top_k;        /* K selected positions per KV head (>= 1)                        */
  int32_t nms_radius;   /* soft-NMS radius R (>= 0)                                       */
  float lambda;         /* fusion weight of the prior, in [0, 1]                          */
  float alpha_soft;     /* soft-NMS penalty: a dominated score is scaled by 1 - alpha     */
  float alpha_cross;    /* exclusivity penalty: a non-owner score is scaled by 1 - alpha  */
  float lambda_clip;    /* < 0: the fusion weight is `lambda`.  In [0, 1]: it adapts per
                           (row, KV head) to the evidence, lambda_g = min(lambda_clip,
                           H(f_g) / ln N) with H the entropy of f_g, and `lambda` is unused */
  int32_t nms_greedy;   /* 0: one-pass soft-NMS (dominance on the unrefined score).  1: greedy
                           soft-NMS: per head, the candidate with the largest current score
                           (lower position on ties) is taken and keeps that score; every
                           untaken candidate within nms_radius is scaled by 1 - alpha_soft;
                           repeated until all are taken; Top-K of the taken scores */
} sfi_select_params;

/* ABI version (SFI_ABI_VERSION) and a static description of a status code. */
int sfi_abi_version(void);
const char* sfi_status_str(int code);

/* Workspace sizes in bytes for the calls below (pure host functions, 0 if the arguments
 * are invalid).  The workspace needs no initialisation and holds nothing between calls. */
size_t sfi_slow_attn_ws(const sfi_shape* shape, int32_t n_seqs, int32_t max_seq_len);
size_t sfi_fast_attn_ws(const sfi_shape* shape, int32_t n_seqs, int32_t packed_cap,
                        int32_t max_recent);
size_t sfi_select_ws(const sfi_shape* shape, const sfi_select_params* params,
                     int32_t n_seqs, int32_t max_seq_len);

/* The same for the query-window calls (sfi_slow_attn_window, sfi_select_window). */
size_t sfi_slow_attn_window_ws(const sfi_shape* shape, int32_t window, int32_t n_seqs,
                               int32_t max_seq_len);
size_t sfi_select_window_ws(const sfi_shape* shape, const sfi_select_params* params,
                            int32_t window, int32_t n_seqs, int32_t max_seq_len);

/* The same for sfi_decode_attn: the fast call's workspace rounded up to 256 bytes plus the
 * windowed slow call's. */
size_t sfi_decode_attn_ws(const sfi_shape* shape, int32_t window, int32_t n_seqs,
                          int32_t packed_cap, int32_t max_recent, int32_t max_seq_len);

/* Round-up of n_sink + top_k to a multiple of 16: rows per (b, KV head) of the packed
 * buffers. */
int32_t sfi_packed_cap(const sfi_select_params* params);

/*
 * sfi_key_norms -- cached key statistic ||k_{b,g,j}||_2 for positions [pos_begin, pos_end)
 * of every KV head of the listed rows (the Selector's prior is built from statistics kept
 * with the cache, key norms among them: zh "2.2 训练无感的 Selector").  Run at prefill / append time.
 * key_norm[b][g][j] is written for j in [pos_begin, min(pos_end, N_b)).
 */
int sfi_key_norms(const sfi_shape* shape, const void* k_cache, const int32_t* block_table,
                  const int32_t* seq_lens, const int32_t* seq_ids, int32_t n_seqs,
                  int32_t pos_begin, int32_t pos_end, float* key_norm, int64_t norm_stride,
                  void* stream);

/*
 * sfi_slow_attn -- dense decode attention of a slow step over all N_b positions of each
 * listed row (es "2. Metodología": dense attention over the whole accessible history).
 * Writes out[b] and lse[b]; when `logits` is not NULL also z[b][h][j] for j < N_b, the
 * evidence the Selector reads.  With logits == NULL this is the Full-KV dense step.
 * max_seq_len >= every listed N_b sizes the split of the work (<= max_pages_per_seq*16).
 * ws: sfi_slow_attn_ws(shape, n_seqs, max_seq_len) bytes.
 */
int sfi_slow_attn(const sfi_shape* shape, const float* q, const void* k_cache,
                  const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* seq_ids, int32_t n_seqs, int32_t max_seq_len, float* out,
                  float* logits, int64_t logits_stride, float* lse, uint32_t* status, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * sfi_slow_attn_window -- a slow step whose evidence comes from a window of `window`
 * queries per head instead of the current query alone (the pages describe the evidence as
 * the attention observed in the slow step's window: es "2. Metodología",
 * zh "2.2 训练无感的 Selector").  Slot 0 is the current query; the other slots are earlier decode queries
 * chosen by the caller.  Every slot attends to all N_b positions (no causal mask between
 * the slots).  The window's queries of KV head g are extra rows of its group, so K and V
 * are read once for all of them.
 *   q_win   f32 [batch, Hkv, window, G, D]   slot k of query head g*G + i at [b][g][k][i]
 *   out     f32 [batch, Hq, D]               slot 0 only: the step's attention output
 *   lse     f32 [batch, Hkv, window, G]      every slot
 *   logits  f32 [batch, Hkv, window, G, logits_stride]  every slot (or NULL)
 * Requires window >= 1 (SFI_E_ARG) and G * window <= 16 (SFI_E_UNSUPPORTED); window 1 is
 * sfi_slow_attn.  ws: sfi_slow_attn_window_ws(shape, window, n_seqs, max_seq_len) bytes.
 */
int sfi_slow_attn_window(const sfi_shape* shape, int32_t window, const float* q_win,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, const int32_t* seq_ids, int32_t n_seqs,
                         int32_t max_seq_len, float* out, float* logits, int64_t logits_stride,
                         float* lse, uint32_t* status, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * sfi_select -- the training-free Selector of a slow step (zh "2.2 训练无感的 Selector",
 * fr "2.B", nl "De Selector"), per listed row b and KV head g, at N = N_b:
 *   f(g,j)  = mean over the G query heads of g of exp(z(h,j) - lse(h))
 *   r(g,j)  = phi_key * phi_pos / sum_{j'<N} phi_key * phi_pos,
 *             phi_key = 1 / max(key_norm, 1e-6), phi_pos = 1 + ln(1 + (N - 1 - j))
 *   s       = (1 - lambda) f + lambda r                       (the closed-form fusion)
 *             with lambda_clip >= 0: lambda_g = min(lambda_clip, H(f_g) / ln N) per (b, g),
 *             H(f) = -sum_j f_j ln f_j (0 ln 0 = 0); lambda_g = 0 when N = 1 (the ablation
 *             of the pages names the fusion knob lambda_clip, zh "4. 实验结果")
 *   on candidates C = [n_sink, N - n_recent):
 *   s'      = s * (1-alpha_soft)^dom * (1-alpha_cross)^exc   (log-score refinement)
 *             (with nms_greedy = 1 the soft-NMS factor is the greedy one described at
 *             sfi_select_params instead of (1-alpha_soft)^dom)
 *             dom: a candidate within nms_radius in the same head has a strictly larger s
 *             exc: g is not the owner of j (the head with the largest s at j, lowest g
 *                  on ties)
 *   sel_idx = the min(top_k, |C|) candidates with the largest s' (ties to the lower
 *             position), ascending, then -1 up to top_k.
 * logits/lse come from sfi_slow_attn of the same step.  When dbg_scores is not NULL it
 * receives s as f32 [batch, Hkv, logits_stride] for j < N_b.
 * max_seq_len <= 4194304 (SFI_E_UNSUPPORTED beyond).
 * ws: sfi_select_ws(shape, params, n_seqs, max_seq_len) bytes.
 */
int sfi_select(const sfi_shape* shape, const sfi_select_params* params, const float* logits,
               int64_t logits_stride, const float* lse, const float* key_norm,
               int64_t norm_stride, const int32_t* seq_lens, const int32_t* seq_ids,
               int32_t n_seqs, int32_t max_seq_len, int32_t* sel_idx, float* dbg_scores,
               void* ws, size_t ws_bytes, void* stream);

/*
 * sfi_select_window -- sfi_select on the logits and lse of sfi_slow_attn_window: the
 * evidence f(g,j) is the mean of exp(z - lse) over the G * window rows of KV head g (every
 * query of the window weighs the same); prior, fusion, refinement and Top-K are those of
 * sfi_select.  Same limits as sfi_slow_attn_window.
 * ws: sfi_select_window_ws(shape, params, window, n_seqs, max_seq_len) bytes.
 */
int sfi_select_window(const sfi_shape* shape, const sfi_select_params* params, int32_t window,
                      const float* logits, int64_t logits_stride, const float* lse,
                      const float* key_norm, int64_t norm_stride, const int32_t* seq_lens,
                      const int32_t* seq_ids, int32_t n_seqs, int32_t max_seq_len,
                      int32_t* sel_idx, float* dbg_scores, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * sfi_pack -- gather the sink rows [0, n_sink) and the selected rows sel_idx[b][g][*]
 * (ascending, -1 padded) from the paged cache into the contiguous buffers
 * (zh "2.3 系统级优化": sink and selected rows side by side for sequential reads).  Row i of packed_k/v[b][g]
 * is a byte copy of the cache row at packed_pos[b][g][i]; rows past packed_len[b][g] are
 * zero with packed_pos -1.  sel_idx must hold its valid entries first (as sfi_select
 * writes it).  packed_cap must equal sfi_packed_cap(params).
 */
int sfi_pack(const sfi_shape* shape, const sfi_select_params* params, const void* k_cache,
             const void* v_cache, const int32_t* block_table, const int32_t* sel_idx,
             const int32_t* seq_ids, int32_t n_seqs, void* packed_k, void* packed_v,
             int32_t* packed_pos, int32_t* packed_len, int32_t packed_cap, void* stream);

/*
 * sfi_pack_update -- sfi_pack for a buffer that already holds the previous selection: rows
 * whose position stays selected keep their slot and are not copied again; newly selected
 * rows are copied into the slots of dropped ones, then past the old end (K_eff grows with
 * N).  The slow steps of one sentence select nearly the same support (the pages' within-
 * sentence stability, nl "Kernobservatie", zh "1. 问题背景"), so an update copies a few
 * rows where a full pack copies all of them.
 * After the call rows [0, packed_len[b][g]) of packed_k/v hold exactly the sink rows and the
 * selected rows, each a byte copy of the cache row at packed_pos; the ORDER of the selected
 * rows is unspecified (fast attention does not depend on it).  When a buffer is empty
 * (packed_len 0) or the selection is smaller than what it holds, it is rebuilt in
 * sfi_pack's order.
 *   slot_map  i32 [batch, Hkv, map_stride]: the slot of each position, or -1.  The caller
 *             fills it with -1, packed_pos with -1 and packed_len with 0 once; afterwards
 *             only these calls may change slot_map, packed_pos and the packed rows.  Setting
 *             packed_len[b][g] to 0 empties a buffer (a new sequence): the next call
 *             rebuilds it.  map_stride >= every N_b (device contract) and >= n_sink.
 * ws: sfi_pack_update_ws(shape, params, n_seqs) bytes (no initialisation).
 */
size_t sfi_pack_update_ws(const sfi_shape* shape, const sfi_select_params* params,
                          int32_t n_seqs);
int sfi_pack_update(const sfi_shape* shape, const sfi_select_params* params,
                    const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* sel_idx, const int32_t* seq_ids, int32_t n_seqs,
                    void* packed_k, void* packed_v, int32_t* packed_pos, int32_t* packed_len,
                    int32_t packed_cap, int32_t* slot_map, int64_t map_stride, uint32_t* status,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * sfi_fast_attn -- two-segment attention of a fast step (zh "2.3 系统级优化"): segment A is
 * rows [0, packed_len[b][g]) of the packed buffers, read contiguously; segment B is
 * positions [recent_start[b], N_b) read from the paged cache.  The two partial results
 * are merged by log-sum-exp into out[b] (and lse[b] if not NULL).
 * max_recent >= every listed N_b - recent_start[b] sizes the split of segment B.
 * ws: sfi_fast_attn_ws(shape, n_seqs, packed_cap, max_recent) bytes.
 */
int sfi_fast_attn(const sfi_shape* shape, const float* q, const void* packed_k,
                  const void* packed_v, const int32_t* packed_len, int32_t packed_cap,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* recent_start, const int32_t* seq_lens,
                  const int32_t* seq_ids, int32_t n_seqs, int32_t max_recent, float* out,
                  float* lse, uint32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * sfi_fast_attn_noalloc -- sfi_fast_attn for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as sfi_fast_attn, without the workspace: the split
 * partials go to a device array inside the library, SFI_NOALLOC_SCRATCH_BYTES per GPU,
 * which each GPU holds from the library's load until the process ends.  A call whose
 * workspace, sfi_fast_attn_ws(shape, n_seqs, packed_cap, max_recent), exceeds it returns
 * SFI_E_WORKSPACE with nothing enqueued.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller.  The array
 * needs no initialisation; what a call leaves there is never read by a later call.  The
 * calling thread's current device must be the device of `stream` (SFI_E_ARG otherwise).
 */
#define SFI_NOALLOC_SCRATCH_BYTES (8u << 20)
int sfi_fast_attn_noalloc(const sfi_shape* shape, const float* q, const void* packed_k,
                          const void* packed_v, const int32_t* packed_len, int32_t packed_cap,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          const int32_t* recent_start, const int32_t* seq_lens,
                          const int32_t* seq_ids, int32_t n_seqs, int32_t max_recent,
                          float* out, float* lse, uint32_t* status, void* stream);

/*
 * sfi_decode_attn -- the attention of a whole decode step in one partial launch and one
 * merge launch: the rows listed in fast_ids get sfi_fast_attn (lse not written), the rows
 * listed in slow_ids get sfi_slow_attn_window, with the same arguments those calls take.
 * Both lists hold n_seqs slots (-1 = unused) and must not share a row.  The results are
 * bit-identical to the two separate calls with the same lists and n_seqs.  For steps
 * decided on the device (sfi_step_control), where the host does not know which list is
 * empty, this saves the launches of the empty call.
 * ws: sfi_decode_attn_ws(shape, window, n_seqs, packed_cap, max_recent, max_seq_len) bytes.
 */
int sfi_decode_attn(const sfi_shape* shape, int32_t window, const float* q,
                    const float* q_win, const void* packed_k, const void* packed_v,
                    const int32_t* packed_len, int32_t packed_cap, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* recent_start, const int32_t* seq_lens,
                    const int32_t* fast_ids, const int32_t* slow_ids, int32_t n_seqs,
                    int32_t max_recent, int32_t max_seq_len, float* out, float* logits,
                    int64_t logits_stride, float* lse, uint32_t* status, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * sfi_step_control -- the slow/fast decision of one decode step for every row of the batch,
 * on the device (es "2. Metodología", zh "2.1 慢快推理框架": a slow step follows a semantic-
 * boundary token such as sentence punctuation or a line break, or a spent refresh budget).
 * The state is i32 [3, batch]: rows seq_lens, since_slow, recent_start.  For each row b,
 * from state_in to state_out:
 *   seq_lens        = seq_lens + 1            (the token decoded now joins the history)
 *   slow            = since_slow < 0          (no slow step yet)
 *                     || token_ids[b] is one of boundary_tokens[0..n_boundary)
 *                     || since_slow >= refresh_budget
 *   since_slow      = slow ? 0 : since_slow + 1
 *   recent_start    = (slow || sliding_recent) ? max(n_sink, seq_lens - n_recent)
 *                                              : recent_start
 *                     (frozen at the slow step, or with sliding_recent = 1 the newest
 *                     n_recent positions at every step)
 * slow_ids / fast_ids [batch] receive the slow and the fast rows in ascending order, each
 * padded with -1; counts [2] = {slow rows, fast rows}.  n_sink and n_recent come from
 * params.  Initial state: seq_lens = stored length before the first step, since_slow = -1.
 * state_out may be state_in.  The calls of the step read seq_lens and recent_start from
 * state_out (rows 0 and 2) and the lists; work of the previous step still running on
 * another stream reads the previous buffers, so a caller that overlaps steps alternates
 * two state buffers and two pairs of lists.
 * Requires refresh_budget >= 0, sliding_recent in {0, 1} and 0 <= n_boundary <= 1024
 * (SFI_E_UNSUPPORTED beyond).
 * One workgroup; rows are independent.
 */
int sfi_step_control(const sfi_shape* shape, const sfi_select_params* params,
                     int32_t refresh_budget, int32_t sliding_recent, const int32_t* token_ids,
                     const int32_t* boundary_tokens, int32_t n_boundary,
                     const int32_t* state_in, int32_t* state_out, int32_t* slow_ids,
                     int32_t* fast_ids, int32_t* counts, void* stream);

/*
 * sfi_kv_append -- store the K and V rows of the token decoded now at position
 * seq_lens[b] - 1 of each listed row (after sfi_step_control has counted it), and its key
 * norm ||k||_2 into key_norm[b][g][seq_lens[b] - 1] when key_norm is not NULL (the cache
 * statistic the Selector's prior reads, zh "2.2 训练无感的 Selector"; the same bits
 * sfi_key_norms stores).
 *   k_new, v_new  elt [batch, Hkv, D]   16-byte aligned
 * The page of the position must already be in block_table (device contract).
 */
int sfi_kv_append(const sfi_shape* shape, const void* k_new, const void* v_new, void* k_cache,
                  void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                  const int32_t* seq_ids, int32_t n_seqs, float* key_norm, int64_t norm_stride,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SFI_H */
