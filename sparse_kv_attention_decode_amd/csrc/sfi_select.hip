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
//   k_sel_score  one block per 1024-position tile (256 when LDS is short) with an
//                R-position halo, all KV heads at once (NMS couples neighbours,
//                exclusivity couples heads): s into LDS, then the refined score s' as an
//                order-preserving uint32 key (s' >= 0, so its IEEE bits already order
//                like the value).
//   k_sel_topk   one 1024-thread block per (b, g): radix select of the K-th largest key
//                (an 11-bit histogram pass over global memory, then LDS-resident passes
//                over the boundary bin), then one ordered pass that writes every key
//                above the threshold and the lowest-position ties.
#include "sfi_device.h"
#include "sfi_internal.h"

#include <math.h>

namespace sfi {

namespace {

constexpr int kZChunk = 4096;
constexpr int kCandCapBytes = 48 * 1024;

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
// Z_g partial sums: one block per (row, KV head, chunk of 4096 positions); each thread
// covers 16 positions with four float4 loads issued before any arithmetic.
__device__ __forceinline__ float prior_weight(float norm, int N, int j) {
  return (1.f / fmaxf(norm, 1e-6f)) * (1.f + logf(1.f + (float)(N - 1 - j)));
}

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
  const int j0 = chunk * kZChunk + 4 * (int)threadIdx.x;
  float4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = j0 + 1024 * k;
    v[k] = (j + 3 < N) ? *reinterpret_cast<const float4*>(a + j) : make_float4(1.f, 1.f, 1.f, 1.f);
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = j0 + 1024 * k;
    if (j + 3 < N) {
      acc += prior_weight(v[k].x, N, j) + prior_weight(v[k].y, N, j + 1) +
             prior_weight(v[k].z, N, j + 2) + prior_weight(v[k].w, N, j + 3);
    } else {
      for (int q = 0; q < 4; ++q)
        if (j + q < N) acc += prior_weight(a[j + q], N, j + q);
    }
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

// Fused score s(g, j) of one position for every KV head, written to LDS row idx.
template <int GT>
__device__ __forceinline__ void score_scalar(const ScoreArgs& a, const float* zs,
                                             const float* lses, float* s_t, int W, int b,
                                             int N, int j, int idx, bool dbg) {
  const int G = GT > 0 ? GT : a.G;
  const bool in = j >= 0 && j < N;
  const float phi_pos = in ? 1.f + logf(1.f + (float)(N - 1 - j)) : 0.f;
  for (int g = 0; g < a.Hkv; ++g) {
    float s = -1.f;
    if (in) {
      float f = 0.f;
      for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        f += expf(a.logits[((size_t)b * a.Hq + h) * a.logits_stride + j] - lses[h]);
      }
      f *= 1.f / (float)G;
      const float nrm = a.key_norm[((size_t)b * a.Hkv + g) * a.norm_stride + j];
      const float r = (1.f / fmaxf(nrm, 1e-6f)) * phi_pos / zs[g];
      s = (1.f - a.lam) * f + a.lam * r;
      if (dbg) a.dbg[((size_t)b * a.Hkv + g) * a.logits_stride + j] = s;
    }
    s_t[g * W + idx] = s;
  }
}

// One block per (row, tile of TILE positions): every KV head of the tile plus an R-wide
// halo on each side (soft-NMS reads neighbours, exclusivity reads all heads of a
// position), then the refined keys of the tile's candidates.
template <int GT, int PPT>
__global__ __launch_bounds__(256) void k_sel_score(ScoreArgs a) {
  constexpr int TILE = 256 * PPT;
  constexpr int GU = GT > 0 ? GT : kMaxG;  // unroll bound; runtime G when GT == 0
  const int G = GT > 0 ? GT : a.G;
  extern __shared__ float lds[];
  const int W = TILE + 2 * a.R;
  float* s_t = lds;                         // [Hkv][W]
  float* zs = lds + a.Hkv * W;              // [Hkv]
  float* lses = zs + a.Hkv;                 // [Hq]
  const int tid = threadIdx.x;
  const int i = blockIdx.x / a.ntile;
  const int tile = blockIdx.x % a.ntile;
  const int b = a.seq_ids[i];
  const int N = a.seq_lens[b];
  const int t0 = tile * TILE;
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

  // Main positions: thread tid owns j = t0 + PPT*tid .. +PPT-1.
  const int jm = t0 + PPT * tid;
  if (PPT == 4 && jm + 3 < N) {
    float phi[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) phi[q] = 1.f + logf(1.f + (float)(N - 1 - (jm + q)));
    for (int g = 0; g < a.Hkv; ++g) {
      float4 zv[GU];
#pragma unroll
      for (int hh = 0; hh < GU; ++hh)
        if (hh < G)
          zv[hh] = *reinterpret_cast<const float4*>(
              a.logits + ((size_t)b * a.Hq + g * G + hh) * a.logits_stride + jm);
      const float4 nv = *reinterpret_cast<const float4*>(
          a.key_norm + ((size_t)b * a.Hkv + g) * a.norm_stride + jm);
      float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hh = 0; hh < GU; ++hh) {
        if (hh >= G) break;
        const float l = lses[g * G + hh];
        f[0] += expf(zv[hh].x - l);
        f[1] += expf(zv[hh].y - l);
        f[2] += expf(zv[hh].z - l);
        f[3] += expf(zv[hh].w - l);
      }
      const float nr[4] = {nv.x, nv.y, nv.z, nv.w};
      float s[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float r = (1.f / fmaxf(nr[q], 1e-6f)) * phi[q] / zs[g];
        s[q] = (1.f - a.lam) * (f[q] * (1.f / (float)G)) + a.lam * r;
        s_t[g * W + a.R + PPT * tid + q] = s[q];
      }
      if (a.dbg)
        *reinterpret_cast<float4*>(a.dbg + ((size_t)b * a.Hkv + g) * a.logits_stride + jm) =
            make_float4(s[0], s[1], s[2], s[3]);
    }
  } else {
#pragma unroll
    for (int q = 0; q < PPT; ++q)
      score_scalar<GT>(a, zs, lses, s_t, W, b, N, jm + q, a.R + PPT * tid + q, a.dbg != nullptr);
  }
  // Halo: R positions left of the tile and R right of it.
  for (int k = tid; k < 2 * a.R; k += 256) {
    const int left = k < a.R;
    const int j = left ? t0 - a.R + k : t0 + TILE + (k - a.R);
    const int idx = left ? k : a.R + TILE + (k - a.R);
    score_scalar<GT>(a, zs, lses, s_t, W, b, N, j, idx, false);
  }
  __syncthreads();

  const float ws = 1.f - a.a_soft, wc = 1.f - a.a_cross;
#pragma unroll
  for (int q = 0; q < PPT; ++q) {
    const int j = jm + q;
    if (j < lo || j >= hi) continue;
    const int c = a.R + PPT * tid + q;
    int own = 0;
    float best = s_t[c];
    for (int g = 1; g < a.Hkv; ++g) {
      const float v = s_t[g * W + c];
      if (v > best) {
        best = v;
        own = g;
      }
    }
    const int dlo = max(lo, j - a.R) - j;      // <= 0
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
}

// ------------------------------------------------------------------------------- top-K
// Radix selection of the K_eff-th largest refined key per (row, KV head), one 1024-thread
// block each:
//   1. 11-bit histogram passes over the keys in global memory, each restricted to the
//      digits fixed so far, until the bin holding the K_eff-th key has at most kCandCap
//      keys (usually after one pass);
//   2. that bin's keys and candidate indices are compacted into LDS;
//   3. the remaining bits are resolved with LDS-resident histogram passes, giving the
//      exact threshold T and the number of keys equal to T still to take; the last of
//      those ties (lowest positions first) is found by the same selection on the
//      complemented candidate index;
//   4. one ordered pass writes every candidate above T and the ties up to that index,
//      ascending, with a block-wide prefix sum per chunk.
constexpr int kTopkThreads = 1024;
constexpr int kHistBins = 2048;
constexpr int kCandCap = kCandCapBytes / 8;  // key + index per candidate

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

// Bin of hist[0..2048) holding the krem-th largest counted element: thread t owns bins
// 2047-2t and 2046-2t.  Writes (bin, count above the bin) to res[0..1].  All threads call.
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t krem, uint32_t* wsum,
                                         uint32_t* res) {
  const int t = threadIdx.x;
  const uint32_t hh = hist[kHistBins - 1 - 2 * t], hl = hist[kHistBins - 2 - 2 * t];
  uint32_t tot;
  const uint32_t above = block_exscan(hh + hl, wsum, &tot);
  if (above < krem && above + hh >= krem) {
    res[0] = kHistBins - 1 - 2 * t;
    res[1] = above;
  } else if (above + hh < krem && above + hh + hl >= krem) {
    res[0] = kHistBins - 2 - 2 * t;
    res[1] = above + hh;
  }
  __syncthreads();
}

struct TopkArgs {
  const uint32_t* keys;
  int64_t kstride;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  int32_t* sel;
  int Hkv, K, n_sink, n_recent;
};

// Load keys[c .. c+8) (c a multiple of 8) into kv; entries past n read as 0 and are
// marked invalid by the caller's bounds check.
__device__ __forceinline__ void load8(const uint32_t* keys, int c, int n, uint32_t kv[8]) {
  if (c + 8 <= n) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(keys + c);
    const u32x4_t y = *reinterpret_cast<const u32x4_t*>(keys + c + 4);
    kv[0] = x[0]; kv[1] = x[1]; kv[2] = x[2]; kv[3] = x[3];
    kv[4] = y[0]; kv[5] = y[1]; kv[6] = y[2]; kv[7] = y[3];
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) kv[q] = (c + q < n) ? keys[c + q] : 0u;
  }
}

__global__ __launch_bounds__(kTopkThreads) void k_sel_topk(TopkArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t ckey[kCandCap];
  __shared__ uint32_t cidx[kCandCap];
  __shared__ uint32_t wsum[17];
  __shared__ uint32_t res[4];
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
  if (keff == nC) {  // every candidate is taken
    for (int k = tid; k < nC; k += kTopkThreads) out[k] = lo + k;
    return;
  }
  constexpr int STEP = 8 * kTopkThreads;

  // 1. global histogram passes
  uint32_t prefix = 0, krem = (uint32_t)keff, cnt = 0;
  int done = 0;  // resolved top bits
  while (true) {
    const int nb = min(11, 32 - done);
    const int sh = 32 - done - nb;
    for (int k = tid; k < kHistBins; k += kTopkThreads) hist[k] = 0;
    __syncthreads();
    for (int base = 0; base < nC; base += STEP) {
      const int c = base + 8 * tid;
      uint32_t kv[8];
      load8(keys, c, nC, kv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool match = c + q < nC && (done == 0 || (kv[q] >> (32 - done)) == prefix);
        hist_add(hist, (kv[q] >> sh) & ((1u << nb) - 1u), match);
      }
    }
    __syncthreads();
    find_bin(hist, krem, wsum, res);
    const uint32_t d = res[0];
    krem -= res[1];
    cnt = hist[d];
    prefix = (prefix << nb) | d;
    done += nb;
    __syncthreads();
    if (cnt <= (uint32_t)kCandCap || done == 32) break;
  }

  uint32_t T, need_eq, c_last = 0xffffffffu;
  bool by_index = false;
  if (done == 32) {
    T = prefix;
    need_eq = krem;
  } else {
    // 2. compact the boundary bin into LDS (unordered)
    if (tid == 0) res[2] = 0;
    __syncthreads();
    for (int base = 0; base < nC; base += STEP) {
      const int c = base + 8 * tid;
      uint32_t kv[8];
      load8(keys, c, nC, kv);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool match = c + q < nC && (kv[q] >> (32 - done)) == prefix;
        const uint64_t m = __builtin_amdgcn_ballot_w64(match);
        const int lane = tid & 63;
        uint32_t slot0 = 0;
        if (m && lane == __builtin_ctzll(m)) slot0 = atomicAdd(&res[2], (uint32_t)__builtin_popcountll(m));
        slot0 = __shfl(slot0, m ? __builtin_ctzll(m) : 0);
        if (match) {
          const uint32_t slot = slot0 + __builtin_popcountll(m & ((1ull << lane) - 1ull));
          ckey[slot] = kv[q];
          cidx[slot] = (uint32_t)(c + q);
        }
      }
    }
    __syncthreads();
    const int n = (int)res[2];
    // 3. LDS passes over the remaining bits
    while (done < 32) {
      const int nb = min(11, 32 - done);
      const int sh = 32 - done - nb;
      for (int k = tid; k < kHistBins; k += kTopkThreads) hist[k] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += kTopkThreads) {
        const int e = base + tid;
        const uint32_t key = e < n ? ckey[e] : 0u;
        const bool match = e < n && (key >> (32 - done)) == prefix;
        hist_add(hist, (key >> sh) & ((1u << nb) - 1u), match);
      }
      __syncthreads();
      find_bin(hist, krem, wsum, res);
      krem -= res[1];
      prefix = (prefix << nb) | res[0];
      done += nb;
      __syncthreads();
    }
    T = prefix;
    need_eq = krem;
    // ties at T: the need_eq-th smallest candidate index is the last one taken
    {
      uint32_t uprefix = 0, urem = need_eq;
      int udone = 0;
      while (udone < 32) {
        const int nb = min(11, 32 - udone);
        const int sh = 32 - udone - nb;
        for (int k = tid; k < kHistBins; k += kTopkThreads) hist[k] = 0;
        __syncthreads();
        for (int base = 0; base < n; base += kTopkThreads) {
          const int e = base + tid;
          const bool tie = e < n && ckey[e] == T;
          const uint32_t u = tie ? ~cidx[e] : 0u;
          const bool match = tie && (udone == 0 || (u >> (32 - udone)) == uprefix);
          hist_add(hist, (u >> sh) & ((1u << nb) - 1u), match);
        }
        __syncthreads();
        find_bin(hist, urem, wsum, res);
        urem -= res[1];
        uprefix = (uprefix << nb) | res[0];
        udone += nb;
        __syncthreads();
      }
      c_last = ~uprefix;
      by_index = true;
    }
  }

  // 4. ordered output
  uint32_t taken = 0, eq_seen = 0;
  for (int base = 0; base < nC && taken < (uint32_t)keff; base += STEP) {
    const int c = base + 8 * tid;
    uint32_t kv[8];
    load8(keys, c, nC, kv);
    bool take[8];
    uint32_t nsel = 0;
    if (by_index) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        take[q] = c + q < nC && (kv[q] > T || (kv[q] == T && (uint32_t)(c + q) <= c_last));
        nsel += take[q] ? 1u : 0u;
      }
    } else {
      uint32_t neq = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) neq += (c + q < nC && kv[q] == T) ? 1u : 0u;
      uint32_t eq_tot;
      uint32_t eq_before = eq_seen + block_exscan(neq, wsum, &eq_tot);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool valid = c + q < nC;
        const bool eq = valid && kv[q] == T;
        take[q] = (valid && kv[q] > T) || (eq && eq_before < need_eq);
        if (eq) ++eq_before;
        nsel += take[q] ? 1u : 0u;
      }
      eq_seen += eq_tot;
    }
    uint32_t sel_tot;
    uint32_t at = taken + block_exscan(nsel, wsum, &sel_tot);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (take[q] && at < (uint32_t)keff) out[at++] = lo + c + q;
    taken += sel_tot;
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

size_t score_lds_bytes(int num_kv_heads, int num_q_heads, int nms_radius, int tile) {
  return sizeof(float) * ((size_t)num_kv_heads * (tile + 2 * (size_t)nms_radius) +
                          num_kv_heads + num_q_heads);
}

namespace {

template <int PPT>
void launch_score_g(const ScoreArgs& a, int n_seqs, size_t lds, hipStream_t st) {
  const dim3 grid(n_seqs * a.ntile), block(256);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((k_sel_score<1, PPT>), grid, block, lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_sel_score<2, PPT>), grid, block, lds, st, a); break;
    case 4: hipLaunchKernelGGL((k_sel_score<4, PPT>), grid, block, lds, st, a); break;
    case 8: hipLaunchKernelGGL((k_sel_score<8, PPT>), grid, block, lds, st, a); break;
    case 16: hipLaunchKernelGGL((k_sel_score<16, PPT>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((k_sel_score<0, PPT>), grid, block, lds, st, a); break;
  }
}

}  // namespace

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
  a.n_sink = prm.n_sink;
  a.n_recent = prm.n_recent;
  a.R = prm.nms_radius;
  a.lam = prm.lambda;
  a.a_soft = prm.alpha_soft;
  a.a_cross = prm.alpha_cross;
  // Wide tiles when their LDS fits, narrow ones otherwise.
  const size_t wide = score_lds_bytes(Hkv, Hq, prm.nms_radius, 1024);
  if (wide <= kScoreLdsLimit) {
    a.ntile = (max_seq_len + 1023) / 1024;
    launch_score_g<4>(a, n_seqs, wide, st);
  } else {
    a.ntile = (max_seq_len + 255) / 256;
    launch_score_g<1>(a, n_seqs, score_lds_bytes(Hkv, Hq, prm.nms_radius, 256), st);
  }
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
