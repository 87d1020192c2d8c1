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
//   k_sel_score  one block per tile of up to 256 positions with an R-position halo, all
//                KV heads at once (NMS couples neighbours, exclusivity couples heads):
//                logits and norms staged in LDS, s computed there, then the refined score
//                s' as an order-preserving uint32 key (s' >= 0, so its IEEE bits already
//                order like the value).
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
  int Hq, Hkv, G, nchunk, ntile, tile;
  int n_sink, n_recent, R;
  float lam, a_soft, a_cross;
};

// Row width of the staged tile: the halo on each side is padded to a multiple of four
// so the tile body keeps 16-byte alignment in LDS.
__host__ __device__ inline int score_pad(int R) { return (R + 3) & ~3; }

// One block per (row, tile of `tile` positions).  Stage the logits of every query head
// and the key norms of every KV head over the tile and an R-wide halo on each side into
// LDS, with all global loads issued before any arithmetic; then the fused score s of
// every KV head at every staged position; then, for the tile's candidates, the soft-NMS
// dominance (neighbours within R, same head) and ownership (all heads at the position)
// and the refined key.
template <int GT>
__global__ __launch_bounds__(256) void k_sel_score(ScoreArgs a) {
  extern __shared__ float4 lds4[];  // float4 keeps the staged rows 16-byte aligned
  float* lds = reinterpret_cast<float*>(lds4);
  const int G = GT > 0 ? GT : a.G;
  const int TILE = a.tile;
  const int P = score_pad(a.R);
  const int W = TILE + 2 * P;
  float* zt = lds;                    // [Hq][W]   logits
  float* nt = zt + a.Hq * W;          // [Hkv][W]  key norms
  float* s_t = nt + a.Hkv * W;        // [Hkv][W]  fused scores
  float* zs = s_t + a.Hkv * W;        // [Hkv]     prior normalisers
  float* lses = zs + a.Hkv;           // [Hq]
  const int tid = threadIdx.x;
  const int i = blockIdx.x / a.ntile;
  const int tile = blockIdx.x % a.ntile;
  const int b = a.seq_ids[i];
  const int N = a.seq_lens[b];
  const int t0 = tile * TILE;
  if (t0 >= N) return;  // block-uniform
  const int lo = a.n_sink;
  const int hi = max(lo, N - a.n_recent);

  // Stage the tile body (float4) and the halo (scalars) of logits and norms.
  const int q4 = TILE / 4;
  const int rows = a.Hq + a.Hkv;
  for (int e = tid; e < rows * q4; e += 256) {
    const int row = e / q4, c4 = e % q4;
    const int j = t0 + 4 * c4;
    const float* src = row < a.Hq
                           ? a.logits + ((size_t)b * a.Hq + row) * a.logits_stride + j
                           : a.key_norm + ((size_t)b * a.Hkv + (row - a.Hq)) * a.norm_stride + j;
    float4 v;
    if (j + 3 < N) {
      v = *reinterpret_cast<const float4*>(src);
    } else {
      v.x = j < N ? src[0] : 0.f;
      v.y = j + 1 < N ? src[1] : 0.f;
      v.z = j + 2 < N ? src[2] : 0.f;
      v.w = j + 3 < N ? src[3] : 0.f;
    }
    *reinterpret_cast<float4*>(zt + row * W + P + 4 * c4) = v;
  }
  for (int e = tid; e < rows * 2 * a.R; e += 256) {
    const int row = e / (2 * a.R), k = e % (2 * a.R);
    const bool left = k < a.R;
    const int j = left ? t0 - a.R + k : t0 + TILE + (k - a.R);
    const int col = left ? P - a.R + k : P + TILE + (k - a.R);
    float v = 0.f;
    if (j >= 0 && j < N)
      v = row < a.Hq ? a.logits[((size_t)b * a.Hq + row) * a.logits_stride + j]
                     : a.key_norm[((size_t)b * a.Hkv + (row - a.Hq)) * a.norm_stride + j];
    zt[row * W + col] = v;
  }
  for (int g = tid; g < a.Hkv; g += 256) {
    const float* zp = a.zpart + ((size_t)i * a.Hkv + g) * a.nchunk;
    float z = 0.f;
    for (int c = 0; c < a.nchunk; ++c) z += zp[c];
    zs[g] = z;
  }
  for (int h = tid; h < a.Hq; h += 256) lses[h] = a.lse[(size_t)b * a.Hq + h];
  __syncthreads();

  // Fused scores over the tile and its halo.
  const float invG = 1.f / (float)G;
  for (int col = P - a.R + tid; col < P + TILE + a.R; col += 256) {
    const int j = t0 - P + col;
    const bool in = j >= 0 && j < N;
    const float phi_pos = in ? 1.f + logf(1.f + (float)(N - 1 - j)) : 0.f;
    const bool body = col >= P && col < P + TILE;
    for (int g = 0; g < a.Hkv; ++g) {
      float s = -1.f;
      if (in) {
        float f = 0.f;
        if (GT > 0) {
#pragma unroll
          for (int hh = 0; hh < (GT > 0 ? GT : 1); ++hh)
            f += expf(zt[(g * G + hh) * W + col] - lses[g * G + hh]);
        } else {
          for (int hh = 0; hh < G; ++hh) f += expf(zt[(g * G + hh) * W + col] - lses[g * G + hh]);
        }
        f *= invG;
        const float r = (1.f / fmaxf(nt[g * W + col], 1e-6f)) * phi_pos / zs[g];
        s = (1.f - a.lam) * f + a.lam * r;
        if (a.dbg && body) a.dbg[((size_t)b * a.Hkv + g) * a.logits_stride + j] = s;
      }
      s_t[g * W + col] = s;
    }
  }
  __syncthreads();

  // Refinement decisions and keys for the tile's candidates.
  const float ws = 1.f - a.a_soft, wc = 1.f - a.a_cross;
  for (int col = P + tid; col < P + TILE; col += 256) {
    const int j = t0 - P + col;
    if (j < lo || j >= hi) continue;
    int own = 0;
    float best = s_t[col];
    for (int g = 1; g < a.Hkv; ++g) {
      const float v = s_t[g * W + col];
      if (v > best) {
        best = v;
        own = g;
      }
    }
    const int dlo = max(lo, j - a.R) - j;      // <= 0
    const int dhi = min(hi - 1, j + a.R) - j;  // >= 0
    for (int g = 0; g < a.Hkv; ++g) {
      const float* row = s_t + g * W + col;
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
// Every pass over global keys reads 16 keys per thread per chunk with the next chunk in
// flight.
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

constexpr int kKeysPerThread = 16;
constexpr int kPassStep = kKeysPerThread * kTopkThreads;

// keys[c .. c+16) as four 16-byte loads.  The read is clamped into the row
// [0, kstride) (kstride is a multiple of 64), so it is issued unconditionally; entries at
// or past the candidate count are masked by the caller through their index.
__device__ __forceinline__ void load16(const uint32_t* keys, int64_t kstride, int c,
                                       uint32_t kv[kKeysPerThread]) {
  const int cl = (int)min((int64_t)c, kstride - kKeysPerThread);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(keys + cl + 4 * w);
    kv[4 * w] = x[0];
    kv[4 * w + 1] = x[1];
    kv[4 * w + 2] = x[2];
    kv[4 * w + 3] = x[3];
  }
}

// Visit keys [0, n) in chunks of 16 per thread; the next chunk is requested before the
// current one is processed (two register buffers, unrolled so they swap roles without
// copies).  f(c, kv) sees the keys at candidate indices c .. c+15 and is called by every
// thread the same number of times (it may contain block barriers).
template <typename F>
__device__ __forceinline__ void pass16(const uint32_t* keys, int64_t kstride, int n, F&& f) {
  const int off = kKeysPerThread * (int)threadIdx.x;
  uint32_t A[kKeysPerThread], B[kKeysPerThread];
  load16(keys, kstride, off, A);
  for (int base = 0; base < n; base += 2 * kPassStep) {
    load16(keys, kstride, base + kPassStep + off, B);
    f(base + off, A);
    if (base + kPassStep >= n) break;
    load16(keys, kstride, base + 2 * kPassStep + off, A);
    f(base + kPassStep + off, B);
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
  // 1. global histogram passes
  uint32_t prefix = 0, krem = (uint32_t)keff, cnt = 0;
  int done = 0;  // resolved top bits
  while (true) {
    const int nb = min(11, 32 - done);
    const int sh = 32 - done - nb;
    for (int k = tid; k < kHistBins; k += kTopkThreads) hist[k] = 0;
    __syncthreads();
    pass16(keys, a.kstride, nC, [&](int c, const uint32_t* kv) {
#pragma unroll
      for (int q = 0; q < kKeysPerThread; ++q) {
        const bool match = c + q < nC && (done == 0 || (kv[q] >> (32 - done)) == prefix);
        hist_add(hist, (kv[q] >> sh) & ((1u << nb) - 1u), match);
      }
    });
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
    pass16(keys, a.kstride, nC, [&](int c, const uint32_t* kv) {
#pragma unroll
      for (int q = 0; q < kKeysPerThread; ++q) {
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
    });
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
  pass16(keys, a.kstride, nC, [&](int c, const uint32_t* kv) {
    bool take[kKeysPerThread];
    uint32_t nsel = 0;
    if (by_index) {
#pragma unroll
      for (int q = 0; q < kKeysPerThread; ++q) {
        take[q] = c + q < nC && (kv[q] > T || (kv[q] == T && (uint32_t)(c + q) <= c_last));
        nsel += take[q] ? 1u : 0u;
      }
    } else {
      uint32_t neq = 0;
#pragma unroll
      for (int q = 0; q < kKeysPerThread; ++q) neq += (c + q < nC && kv[q] == T) ? 1u : 0u;
      uint32_t eq_tot;
      uint32_t eq_before = eq_seen + block_exscan(neq, wsum, &eq_tot);
#pragma unroll
      for (int q = 0; q < kKeysPerThread; ++q) {
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
    for (int q = 0; q < kKeysPerThread; ++q)
      if (take[q] && at < (uint32_t)keff) out[at++] = lo + c + q;
    taken += sel_tot;
  });
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
  const size_t W = (size_t)tile + 2 * (size_t)score_pad(nms_radius);
  return sizeof(float) * ((size_t)(num_q_heads + 2 * num_kv_heads) * W + num_kv_heads +
                          num_q_heads);
}

int score_tile(int num_kv_heads, int num_q_heads, int nms_radius) {
  for (int tile = 256; tile >= 64; tile /= 2)
    if (score_lds_bytes(num_kv_heads, num_q_heads, nms_radius, tile) <= kScoreLdsLimit)
      return tile;
  return 0;
}

namespace {

void launch_score(const ScoreArgs& a, int n_seqs, size_t lds, hipStream_t st) {
  const dim3 grid(n_seqs * a.ntile), block(256);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((k_sel_score<1>), grid, block, lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_sel_score<2>), grid, block, lds, st, a); break;
    case 4: hipLaunchKernelGGL((k_sel_score<4>), grid, block, lds, st, a); break;
    case 8: hipLaunchKernelGGL((k_sel_score<8>), grid, block, lds, st, a); break;
    case 16: hipLaunchKernelGGL((k_sel_score<16>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((k_sel_score<0>), grid, block, lds, st, a); break;
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
  a.tile = score_tile(Hkv, Hq, prm.nms_radius);
  a.ntile = (max_seq_len + a.tile - 1) / a.tile;
  launch_score(a, n_seqs, score_lds_bytes(Hkv, Hq, prm.nms_radius, a.tile), st);
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
