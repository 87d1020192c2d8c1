// On-device step control: the slow/fast decision of a decode step and the append of the
// new token's K/V rows, so that a decode step needs no schedule from the host.
//
// The pages trigger a slow step when the model emits a semantic-boundary token (sentence
// punctuation, a line or paragraph break) or when a refresh budget of fast steps is spent
// (es "2. Metodología", zh "2.1 慢快推理框架", fr "2.A Le Paradigme Lente-Rapide").
// The Selector's prior is built from statistics kept with the cache, key norms among them
// (zh "2.2 训练无感的 Selector"), so the append also stores the new key's norm.
#include "sfi_device.h"
#include "sfi_internal.h"

namespace sfi {

namespace {

constexpr int kCtrlThreads = 256;

struct CtrlArgs {
  const int32_t* tokens;     // [batch] token each row decodes this step
  const int32_t* boundary;   // [n_boundary] boundary token ids
  const int32_t* state_in;   // [3][batch]: seq_lens, since_slow, recent_start
  int32_t* state_out;        // [3][batch], may be state_in
  int32_t* slow_ids;         // [batch] out
  int32_t* fast_ids;         // [batch] out
  int32_t* counts;           // [2] out
  int batch, n_boundary, budget, sliding, n_sink, n_recent;
};

// One block.  Thread t decides row c0 + t of each chunk of 256 rows; the two row lists are
// compacted with block prefix sums, so both come out in ascending row order, and the
// unused tail of each list is filled with -1.
__global__ __launch_bounds__(kCtrlThreads) void k_step_control(CtrlArgs a) {
  __shared__ uint32_t wsum[kCtrlThreads / 64 + 1];
  uint32_t n_slow = 0, n_fast = 0;
  for (int c0 = 0; c0 < a.batch; c0 += kCtrlThreads) {
    const int b = c0 + (int)threadIdx.x;
    const bool live = b < a.batch;
    bool slow = false;
    if (live) {
      const int B = a.batch;
      const int N = a.state_in[b] + 1;  // the decoded token is appended this step
      const int since = a.state_in[B + b];
      const int rs = a.state_in[2 * B + b];
      const int tok = a.tokens[b];
      bool boundary = false;
      for (int k = 0; k < a.n_boundary; ++k) boundary |= a.boundary[k] == tok;
      slow = since < 0 || boundary || since >= a.budget;
      a.state_out[b] = N;
      a.state_out[B + b] = slow ? 0 : since + 1;
      // The recent segment's left edge is frozen at the slow step, or slides every step.
      a.state_out[2 * B + b] = (slow || a.sliding) ? max(a.n_sink, N - a.n_recent) : rs;
    }
    uint32_t tot_s, tot_f;
    const uint32_t ps = block_exscan<kCtrlThreads>(live && slow ? 1u : 0u, wsum, &tot_s);
    const uint32_t pf = block_exscan<kCtrlThreads>(live && !slow ? 1u : 0u, wsum, &tot_f);
    if (live) {
      if (slow)
        a.slow_ids[n_slow + ps] = b;
      else
        a.fast_ids[n_fast + pf] = b;
    }
    n_slow += tot_s;
    n_fast += tot_f;
  }
  for (int k = (int)n_slow + (int)threadIdx.x; k < a.batch; k += kCtrlThreads) a.slow_ids[k] = -1;
  for (int k = (int)n_fast + (int)threadIdx.x; k < a.batch; k += kCtrlThreads) a.fast_ids[k] = -1;
  if (threadIdx.x == 0) {
    a.counts[0] = (int32_t)n_slow;
    a.counts[1] = (int32_t)n_fast;
  }
}

template <typename T>
struct AppendArgs {
  const T* k_new;            // [batch, Hkv, D]
  const T* v_new;
  T* kc;
  T* vc;
  const int32_t* bt;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  float* key_norm;
  int64_t norm_stride;
  int n_seqs, Hkv, max_pages;
};

// LPR = D * sizeof(T) / 16 lanes per (row, KV head): each lane moves 16 bytes of K and of V
// and adds the squares of its K bytes; the lanes' sums are then reduced exactly as the
// key-norm kernel reduces a stored row, so the stored norm is the same bits.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_kv_append(AppendArgs<T> a) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPR = D / EPL;
  constexpr int PPB = 256 / LPR;  // (row, KV head) pairs per block
  const int pair = blockIdx.x * PPB + (int)threadIdx.x / LPR;
  const int part = (int)threadIdx.x % LPR;
  const bool in = pair < a.n_seqs * a.Hkv;
  const int g = pair % a.Hkv;
  const int b = in ? a.seq_ids[pair / a.Hkv] : -1;
  const bool ok = b >= 0;  // the same for every lane of the pair
  float ss = 0.f;
  int pos = 0;
  if (ok) {
    pos = a.seq_lens[b] - 1;
    const int page = a.bt[(size_t)b * a.max_pages + pos / kPage];
    const size_t src = ((size_t)b * a.Hkv + g) * D + part * EPL;
    const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(a.k_new + src);
    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(a.v_new + src);
    const size_t dst = (((size_t)page * a.Hkv + g) * kPage + pos % kPage) * D + part * EPL;
    *reinterpret_cast<u32x4_t*>(a.kc + dst) = kv;
    *reinterpret_cast<u32x4_t*>(a.vc + dst) = vv;
    ss = sumsq16<T>(kv);
  }
  ss = wave_sum_xor(ss, LPR);
  if (ok && part == 0 && a.key_norm)
    a.key_norm[((size_t)b * a.Hkv + g) * a.norm_stride + pos] = sqrtf(ss);
}

template <typename T, int D>
hipError_t append_t(const sfi_shape& s, const void* k_new, const void* v_new, void* k_cache,
                    void* v_cache, const int32_t* bt, const int32_t* seq_lens,
                    const int32_t* seq_ids, int n_seqs, float* key_norm, int64_t norm_stride,
                    hipStream_t st) {
  constexpr int LPR = D * (int)sizeof(T) / 16;
  constexpr int PPB = 256 / LPR;
  AppendArgs<T> a;
  a.k_new = reinterpret_cast<const T*>(k_new);
  a.v_new = reinterpret_cast<const T*>(v_new);
  a.kc = reinterpret_cast<T*>(k_cache);
  a.vc = reinterpret_cast<T*>(v_cache);
  a.bt = bt;
  a.seq_lens = seq_lens;
  a.seq_ids = seq_ids;
  a.key_norm = key_norm;
  a.norm_stride = norm_stride;
  a.n_seqs = n_seqs;
  a.Hkv = s.num_kv_heads;
  a.max_pages = s.max_pages_per_seq;
  const int pairs = n_seqs * s.num_kv_heads;
  hipLaunchKernelGGL((k_kv_append<T, D>), dim3((pairs + PPB - 1) / PPB), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_control(int batch, const int32_t* tokens, const int32_t* boundary,
                               int n_boundary, int budget, int sliding, int n_sink, int n_recent,
                               const int32_t* state_in, int32_t* state_out, int32_t* slow_ids,
                               int32_t* fast_ids, int32_t* counts, hipStream_t stream) {
  CtrlArgs a;
  a.tokens = tokens;
  a.boundary = boundary;
  a.state_in = state_in;
  a.state_out = state_out;
  a.slow_ids = slow_ids;
  a.fast_ids = fast_ids;
  a.counts = counts;
  a.batch = batch;
  a.n_boundary = n_boundary;
  a.budget = budget;
  a.sliding = sliding;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  hipLaunchKernelGGL(k_step_control, dim3(1), dim3(kCtrlThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const sfi_shape& s, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* seq_ids, int n_seqs,
                            float* key_norm, int64_t norm_stride, hipStream_t stream) {
  if (s.dtype == SFI_BF16)
    return s.head_dim == 64
               ? append_t<uint16_t, 64>(s, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                        seq_ids, n_seqs, key_norm, norm_stride, stream)
               : append_t<uint16_t, 128>(s, k_new, v_new, k_cache, v_cache, block_table,
                                         seq_lens, seq_ids, n_seqs, key_norm, norm_stride,
                                         stream);
  return s.head_dim == 64
             ? append_t<float, 64>(s, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                   seq_ids, n_seqs, key_norm, norm_stride, stream)
             : append_t<float, 128>(s, k_new, v_new, k_cache, v_cache, block_table, seq_lens,
                                    seq_ids, n_seqs, key_norm, norm_stride, stream);
}

}  // namespace sfi
