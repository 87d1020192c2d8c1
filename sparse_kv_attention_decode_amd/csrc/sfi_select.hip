// The SFI Selector on the device (zh "2.2 训练无感的 Selector", fr "2.B Le Sélecteur",
// nl "De Selector"), plus the cached key-norm statistic it reads.
//
// Per listed row b and KV head g at KV length N:
//   evidence  f(g,j) = (1/G) sum_h exp(z(h,j) - lse(h))           (slow-step softmax)
//   prior     r(g,j) = phi_key * phi_pos / Z_g,  phi_key = 1/max(||k||, 1e-6),
//             phi_pos = 1 + ln(1 + (N-1-j)),  Z_g = sum over [0, N)
//   fusion    s = (1 - lambda) f + lambda r                        (closed form)
//   refine    on candidates C = [n_sink, N - W):
//             s' = s * (1-alpha_soft)^dom * (1-alpha_cross)^exc, where dom = a candidate
//             within R in the same head has strictly larger s, exc = g is not the head
//             with the largest s at j (lowest head on ties).  Scaling s is the same as
//             adding ln(1-alpha) to the log-score; comparing s is the same as comparing
//             ln s.
//   top-K     the min(K, |C|) largest s' per (b, g), ties to the lower position,
//             written ascending and padded with -1.
//
// Kernels:
//   k_sel_zsum   Z_g partial sums over chunks of 4096 positions.
//   k_sel_score  one block per 256-position tile with an R-position halo, all KV heads at
//                once (NMS couples neighbours, exclusivity couples heads): s into LDS,
//                then the refined score s' as an order-preserving uint32 key (s' >= 0, so
//                its IEEE bits already order like the value).
//   k_sel_topk   one 1024-thread block per (b, g): radix select of the K-th largest key,
//                8 bits per pass with an LDS histogram, then an ordered compaction that
//                takes every key above the threshold and the lowest-position ties.
#include "sfi_device.h"
#include "sfi_internal.h"

#include <math.h>

namespace sfi {

namespace {

constexpr int kZChunk = 4096;
constexpr int kTopkThreads = 1024;

template <int BLOCK>
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int tid = threadIdx.x;
  v = wave_sum_xor(v, kWave);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float t = 0.f;
  if (tid < kWave) {
    t = tid < BLOCK / kWave ? red[tid] : 0.f;
    t = wave_sum_xor(t, kWave);
  }
  __syncthreads();
  if (tid == 0) red[0] = t;
  __syncthreads();
  const float out = red[0];
  __syncthreads();
  return out;
}

// ---------------------------------------------------------------------------- key norms
// Lanes per row: 16-byte loads, LPR = D * esize / 16 lanes cover one row.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_key_norms(const T* __restrict__ kc,
                                                   const int32_t* __restrict__ bt,
                                                   const int32_t* __restrict__ seq_lens,
                                                   const int32_t* __restrict__ seq_ids,
                                                   int Hkv, int max_pages, int pos_begin,
                                                   int pos_end, int rows_per_block,
                                                   float* __restrict__ out, int64_t stride) {
  constexpr int EPL = 16 / sizeof(T);  // elements per lane
  constexpr int LPR = D / EPL;         // lanes per row
  const int nblk_pos = (pos_end - pos_begin + rows_per_block - 1) / rows_per_block;
  const int ig = blockIdx.x / nblk_pos;
  const int pb = blockIdx.x % nblk_pos;
  const int g = ig % Hkv, i = ig / Hkv;
  const int b = seq_ids[i];
  const int N = seq_lens[b];
  const int j = pos_begin + pb * rows_per_block + (int)threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float ss = 0.f;
  const bool ok = j < pos_end && j < N;
  if (ok) {
    const int page = bt[(size_t)b * max_pages + j / kPage];
    const T* row = kc + (((size_t)page * Hkv + g) * kPage + (j % kPage)) * D + part * EPL;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(row);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = u2f(v[w] << 16), c = u2f(v[w] & 0xffff0000u);
        ss = fmaf(a, a, ss);
        ss = fmaf(c, c, ss);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = u2f(v[w]);
        ss = fmaf(a, a, ss);
      }
    }
  }
  ss = wave_sum_xor(ss, LPR);
  if (ok && part == 0) out[((size_t)b * Hkv + g) * stride + j] = sqrtf(ss);
}

template <typename T, int D>
void launch_norms_t(const sfi_shape& s, const void* kc, const int32_t* bt, const int32_t* sl,
                    const int32_t* ids, int n, int pb, int pe, float* out, int64_t stride,
                    hipStream_t st) {
  constexpr int LPR = D / (16 / sizeof(T));
  const int rpb = 256 / LPR;
  const int nblk_pos = (pe - pb + rpb - 1) / rpb;
  hipLaunchKernelGGL((k_key_norms<T, D>), dim3(n * s.num_kv_heads * nblk_pos), dim3(256), 0, st,
                     reinterpret_cast<const T*>(kc), bt, sl, ids, s.num_kv_heads,
                     s.max_pages_per_seq, pb, pe, rpb, out, stride);
}

// ------------------------------------------------------------------------- prior norm Z
__global__ __launch_bounds__(256) void k_sel_zsum(const float* __restrict__ key_norm,
                                                  int64_t norm_stride,
                                                  const int32_t* __restrict__ seq_lens,
                                                  const int32_t* __restrict__ seq_ids, int Hkv,
                                                  int nchunk, float* __restrict__ zpart) {
  __shared__ float red[8];
  const int chunk = blockIdx.x % nchunk;
  const int ig = blockIdx.x / nchunk;
  const int g = ig % Hkv, i = ig / Hkv;
  const int b = seq_ids[i];
  const int N = seq_lens[b];
  const float* a = key_norm + ((size_t)b * Hkv + g) * norm_stride;
  float acc = 0.f;
  const int j0 = chunk * kZChunk;
  const int j1 = min(j0 + kZChunk, N);
  for (int j = j0 + (int)threadIdx.x; j < j1; j += 256) {
    const float phi_key = 1.f / fmaxf(a[j], 1e-6f);
    const float phi_pos = 1.f + logf(1.f + (float)(N - 1 - j));
    acc += phi_key * phi_pos;
  }
  acc = block_sum<256>(acc, red);
  if (threadIdx.x == 0) zpart[blockIdx.x] = acc;
}

// ------------------------------------------------------------------------ fused scoring
struct ScoreArgs {
  const float* logits;
  int64_t logits_stride;
  const float* lse;
  const float* key_norm;
  int64_t norm_stride;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  const float* zpart;
  uint32_t* keys;
  int64_t kstride;
  float* dbg;
  int Hq, Hkv, G, nchunk, ntile;
  int n_sink, n_recent, R;
  float lam, a_soft, a_cross;
};

__global__ __launch_bounds__(256) void k_sel_score(ScoreArgs a) {
  extern __shared__ float lds[];
  const int W = kScoreTile + 2 * a.R;
  float* s_t = lds;                         // [Hkv][W]
  float* zs = lds + a.Hkv * W;              // [Hkv]
  float* lses = zs + a.Hkv;                 // [Hq]
  const int tid = threadIdx.x;
  const int i = blockIdx.x / a.ntile;
  const int tile = blockIdx.x % a.ntile;
  const int b = a.seq_ids[i];
  const int N = a.seq_lens[b];
  const int t0 = tile * kScoreTile;
  if (t0 >= N) return;  // block-uniform
  const int lo = a.n_sink;
  const int hi = max(lo, N - a.n_recent);

  for (int g = tid; g < a.Hkv; g += 256) {
    const float* zp = a.zpart + ((size_t)i * a.Hkv + g) * a.nchunk;
    float z = 0.f;
    for (int c = 0; c < a.nchunk; ++c) z += zp[c];
    zs[g] = z;
  }
  for (int h = tid; h < a.Hq; h += 256) lses[h] = a.lse[(size_t)b * a.Hq + h];
  __syncthreads();

  const float invG = 1.f / (float)a.G;
  for (int idx = tid; idx < W; idx += 256) {
    const int j = t0 - a.R + idx;
    const bool in = j >= 0 && j < N;
    const float phi_pos = in ? 1.f + logf(1.f + (float)(N - 1 - j)) : 0.f;
    for (int g = 0; g < a.Hkv; ++g) {
      float s = -1.f;
      if (in) {
        float f = 0.f;
        for (int hh = 0; hh < a.G; ++hh) {
          const int h = g * a.G + hh;
          f += expf(a.logits[((size_t)b * a.Hq + h) * a.logits_stride + j] - lses[h]);
        }
        f *= invG;
        const float nrm = a.key_norm[((size_t)b * a.Hkv + g) * a.norm_stride + j];
        const float r = (1.f / fmaxf(nrm, 1e-6f)) * phi_pos / zs[g];
        s = (1.f - a.lam) * f + a.lam * r;
        if (a.dbg && idx >= a.R && idx < a.R + kScoreTile)
          a.dbg[((size_t)b * a.Hkv + g) * a.logits_stride + j] = s;
      }
      s_t[g * W + idx] = s;
    }
  }
  __syncthreads();

  const int j = t0 + tid;
  if (j < lo || j >= hi) return;
  const int c = a.R + tid;
  int own = 0;
  float best = s_t[c];
  for (int g = 1; g < a.Hkv; ++g) {
    const float v = s_t[g * W + c];
    if (v > best) {
      best = v;
      own = g;
    }
  }
  const float ws = 1.f - a.a_soft, wc = 1.f - a.a_cross;
  const int dlo = max(lo, j - a.R) - j;    // <= 0
  const int dhi = min(hi - 1, j + a.R) - j;  // >= 0
  for (int g = 0; g < a.Hkv; ++g) {
    const float* row = s_t + g * W + c;
    const float sj = row[0];
    bool dom = false;
    for (int d = dlo; d <= dhi; ++d) dom |= (d != 0) && (row[d] > sj);
    float sp = sj;
    if (dom) sp *= ws;
    if (a.Hkv > 1 && g != own) sp *= wc;
    a.keys[((size_t)i * a.Hkv + g) * a.kstride + (j - lo)] = f2u(sp) & 0x7fffffffu;
  }
}

// ------------------------------------------------------------------------------- top-K
__device__ __forceinline__ void hist_add(uint32_t* hist, int bin, bool active) {
  // Aggregate lanes that share the first active lane's bin into one LDS atomic; the rest
  // add one by one.  Skewed key distributions put most lanes into a few bins.
  uint64_t act = __builtin_amdgcn_ballot_w64(active);
  for (int rep = 0; rep < 2 && act; ++rep) {
    const int leader = __builtin_ctzll(act);
    const int lb = __shfl(bin, leader);
    const uint64_t same = __builtin_amdgcn_ballot_w64(active && bin == lb);
    if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[lb], (uint32_t)__builtin_popcountll(same));
    if (active && bin == lb) active = false;
    act &= ~same;
  }
  if (active) atomicAdd(&hist[bin], 1u);
}

// Exclusive prefix of v over the block (1024 threads); returns the block total in *tot.
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* wsum, uint32_t* tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  if (tid < 64) {
    uint32_t w = tid < kTopkThreads / 64 ? wsum[tid] : 0u;
    uint32_t s = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(s, o);
      if (tid >= o) s += y;
    }
    if (tid < kTopkThreads / 64) wsum[tid] = s - w;  // exclusive
    if (tid == kTopkThreads / 64 - 1) wsum[16] = s;
  }
  __syncthreads();
  const uint32_t res = wsum[wv] + x - v;
  *tot = wsum[16];
  __syncthreads();
  return res;
}

struct TopkArgs {
  const uint32_t* keys;
  int64_t kstride;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  int32_t* sel;
  int Hkv, K, n_sink, n_recent;
};

__global__ __launch_bounds__(kTopkThreads) void k_sel_topk(TopkArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[17];
  __shared__ uint32_t bc[4];
  const int tid = threadIdx.x;
  const int ig = blockIdx.x;
  const int g = ig % a.Hkv, i = ig / a.Hkv;
  const int b = a.seq_ids[i];
  const int N = a.seq_lens[b];
  const int lo = a.n_sink;
  const int hi = max(lo, N - a.n_recent);
  const int nC = hi - lo;
  const int keff = min(a.K, nC);
  int32_t* out = a.sel + ((size_t)b * a.Hkv + g) * a.K;
  const uint32_t* keys = a.keys + (size_t)ig * a.kstride;
  for (int k = keff + tid; k < a.K; k += kTopkThreads) out[k] = -1;
  if (keff == 0) return;

  uint32_t thr = 0, need_eq;
  if (keff == nC) {
    need_eq = 0xffffffffu;  // every candidate is taken: threshold 0 with unlimited ties
  } else {
    uint32_t prefix = 0, pmask = 0, krem = (uint32_t)keff;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int k = tid; k < 256; k += kTopkThreads) hist[k] = 0;
      __syncthreads();
      for (int base = 0; base < nC; base += kTopkThreads) {
        const int c = base + tid;
        const uint32_t key = c < nC ? keys[c] : 0u;
        const bool act = c < nC && (key & pmask) == prefix;
        hist_add(hist, (key >> shift) & 255u, act);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l owns bins 4l .. 4l+3; suffix sums from the top bin down
        uint32_t h4[4], s = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h4[q] = hist[4 * tid + q];
          s += h4[q];
        }
        // inclusive suffix scan over lanes (sum of lanes >= tid)
        uint32_t suf = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_down(suf, o);
          if (tid + o < 64) suf += y;
        }
        uint32_t above = suf - s;  // keys in bins of higher lanes
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (above < krem && above + h4[q] >= krem) {
            bc[0] = 4 * tid + q;
            bc[1] = above;
          }
          above += h4[q];
        }
      }
      __syncthreads();
      const uint32_t d = bc[0];
      krem -= bc[1];
      prefix |= d << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    need_eq = krem;
  }

  // Ordered compaction: keys > thr, plus the first need_eq keys == thr by position.
  uint32_t taken = 0, eq_seen = 0;
  for (int base = 0; base < nC && taken < (uint32_t)keff; base += 4 * kTopkThreads) {
    const int c0 = base + 4 * tid;
    uint32_t kv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) kv[q] = (c0 + q < nC) ? keys[c0 + q] : 0u;
    uint32_t neq = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) neq += (c0 + q < nC && kv[q] == thr) ? 1u : 0u;
    uint32_t eq_tot;
    uint32_t eq_before = eq_seen + block_exscan(neq, wsum, &eq_tot);
    bool take[4];
    uint32_t nsel = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool valid = c0 + q < nC;
      const bool gt = valid && kv[q] > thr;
      const bool eq = valid && kv[q] == thr;
      take[q] = gt || (eq && eq_before < need_eq);
      if (eq) ++eq_before;
      nsel += take[q] ? 1u : 0u;
    }
    uint32_t sel_tot;
    uint32_t at = taken + block_exscan(nsel, wsum, &sel_tot);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (take[q] && at < (uint32_t)keff) out[at++] = lo + c0 + q;
    taken += sel_tot;
    eq_seen += eq_tot;
  }
}

}  // namespace

hipError_t launch_key_norms(const sfi_shape& s, const void* kc, const int32_t* bt,
                            const int32_t* sl, const int32_t* ids, int n, int pb, int pe,
                            float* out, int64_t stride, hipStream_t st) {
  if (s.dtype == SFI_BF16) {
    if (s.head_dim == 64) launch_norms_t<uint16_t, 64>(s, kc, bt, sl, ids, n, pb, pe, out, stride, st);
    else launch_norms_t<uint16_t, 128>(s, kc, bt, sl, ids, n, pb, pe, out, stride, st);
  } else {
    if (s.head_dim == 64) launch_norms_t<float, 64>(s, kc, bt, sl, ids, n, pb, pe, out, stride, st);
    else launch_norms_t<float, 128>(s, kc, bt, sl, ids, n, pb, pe, out, stride, st);
  }
  return hipGetLastError();
}

SelectLayout select_layout(const sfi_shape& s, int n_seqs, int max_seq_len) {
  SelectLayout L;
  L.nchunk = (max_seq_len + kZChunk - 1) / kZChunk;
  L.kstride = ((int64_t)max_seq_len + 63) / 64 * 64;
  const size_t units = (size_t)n_seqs * s.num_kv_heads;
  L.zpart_off = 0;
  const size_t zbytes = ((units * L.nchunk * sizeof(float) + 255) / 256) * 256;
  L.keys_off = zbytes;
  L.total = zbytes + units * (size_t)L.kstride * sizeof(uint32_t);
  return L;
}

size_t score_lds_bytes(int num_kv_heads, int num_q_heads, int nms_radius) {
  return sizeof(float) * ((size_t)num_kv_heads * (kScoreTile + 2 * (size_t)nms_radius) +
                          num_kv_heads + num_q_heads);
}

hipError_t launch_select(const sfi_shape& s, const sfi_select_params& prm, const float* logits,
                         int64_t logits_stride, const float* lse, const float* key_norm,
                         int64_t norm_stride, const int32_t* seq_lens, const int32_t* seq_ids,
                         int n_seqs, int max_seq_len, int32_t* sel_idx, float* dbg, void* ws,
                         hipStream_t st) {
  const SelectLayout L = select_layout(s, n_seqs, max_seq_len);
  char* w = reinterpret_cast<char*>(ws);
  float* zpart = reinterpret_cast<float*>(w + L.zpart_off);
  uint32_t* keys = reinterpret_cast<uint32_t*>(w + L.keys_off);
  const int Hkv = s.num_kv_heads, Hq = s.num_q_heads;
  hipLaunchKernelGGL(k_sel_zsum, dim3(n_seqs * Hkv * L.nchunk), dim3(256), 0, st, key_norm,
                     norm_stride, seq_lens, seq_ids, Hkv, L.nchunk, zpart);
  ScoreArgs a;
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.lse = lse;
  a.key_norm = key_norm;
  a.norm_stride = norm_stride;
  a.seq_lens = seq_lens;
  a.seq_ids = seq_ids;
  a.zpart = zpart;
  a.keys = keys;
  a.kstride = L.kstride;
  a.dbg = dbg;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.nchunk = L.nchunk;
  a.ntile = (max_seq_len + kScoreTile - 1) / kScoreTile;
  a.n_sink = prm.n_sink;
  a.n_recent = prm.n_recent;
  a.R = prm.nms_radius;
  a.lam = prm.lambda;
  a.a_soft = prm.alpha_soft;
  a.a_cross = prm.alpha_cross;
  const size_t lds = score_lds_bytes(Hkv, Hq, prm.nms_radius);
  hipLaunchKernelGGL(k_sel_score, dim3(n_seqs * a.ntile), dim3(256), lds, st, a);
  TopkArgs t;
  t.keys = keys;
  t.kstride = L.kstride;
  t.seq_lens = seq_lens;
  t.seq_ids = seq_ids;
  t.sel = sel_idx;
  t.Hkv = Hkv;
  t.K = prm.top_k;
  t.n_sink = prm.n_sink;
  t.n_recent = prm.n_recent;
  hipLaunchKernelGGL(k_sel_topk, dim3(n_seqs * Hkv), dim3(kTopkThreads), 0, st, t);
  return hipGetLastError();
}

}  // namespace sfi
