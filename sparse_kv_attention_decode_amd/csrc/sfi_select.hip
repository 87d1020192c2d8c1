// The SFI Selector on the device (zh "2.2 训练无感的 Selector", fr "2.B Le Sélecteur",
// nl "De Selector"), plus the cached key-norm statistic it reads.
//
// Per listed row b and KV head g at KV length N:
//   evidence  f(g,j) = (1/G) sum_h exp(z(h,j) - lse(h))           (slow-step softmax)
//   prior     r(g,j) = phi_key * phi_pos / Z_g,  phi_key = 1/max(||k||, 1e-6),
//             phi_pos = 1 + ln(1 + (N-1-j)),  Z_g = sum over [0, N)
//   fusion    s = (1 - lambda) f + lambda r                        (closed form); with
//             lambda_clip >= 0 the weight adapts per (b, g):
//             lambda_g = min(lambda_clip, H(f_g) / ln N), H(f) = -sum_j f_j ln f_j
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
//   k_sel_zsum   Z_g partial sums over chunks of 4096 positions (and, with an adaptive
//                weight, partial sums of f ln f).
//   k_sel_score  one block per tile of 256 - 2R positions plus an R-position halo, all
//                KV heads at once (NMS couples neighbours, exclusivity couples heads):
//                one thread per position computes s of every head into LDS, then the
//                refined score s' as an order-preserving uint32 key (s' >= 0, so its IEEE
//                bits already order like the value).
//   k_greedy_nms (greedy soft-NMS only) one workgroup per (row, KV head): the greedy
//                takes in rounds, keys rewritten in place with the taken scores.
//   k_topk_*     radix select of the K-th largest key spread over slices of 4096
//                candidates (histogram, boundary-bin gather, a one-block select on the
//                gathered bin in LDS, ordered parallel write); see the top-K section.
//                Rows of at most four slices take one block per (row, head) instead
//                (k_topk_small), which ranks the keys in a single launch.
#include "sfi_device.h"
#include "sfi_internal.h"

#include <math.h>

namespace sfi {

namespace {

constexpr int kZChunk = 4096;
constexpr int kCandCapBytes = 48 * 1024;
constexpr int kTopkHistWords = 2048;  // global radix histogram per (row, KV head)
constexpr int kTopkStateWords = 8;

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
  if (b < 0) return;  // unused slot of the row list
  const int N = seq_lens[b];
  const int j = pos_begin + pb * rows_per_block + (int)threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float ss = 0.f;
  const bool ok = j < pos_end && j < N;
  if (ok) {
    const int page = bt[(size_t)b * max_pages + j / kPage];
    const T* row = kc + (((size_t)page * Hkv + g) * kPage + (j % kPage)) * D + part * EPL;
    ss = sumsq16<T>(*reinterpret_cast<const u32x4_t*>(row));
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

struct ZsumArgs {
  const float* key_norm;
  int64_t norm_stride;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  int Hkv, nchunk;
  float* zpart;
  uint32_t* topk_hist;
  uint32_t* topk_state;
  // adaptive fusion weight only (hpart == nullptr otherwise): partial sums of f ln f
  const float* logits;
  int64_t logits_stride;
  const float* lse;
  int Hq, G;
  float* hpart;
};

// Evidence f at positions j .. j + 3 of KV head g (the same sum, in the same order, as the
// scoring kernel's): the mean over the group's rows of exp(z - lse).
__device__ __forceinline__ float4 evidence4(const ZsumArgs& a, int b, int g, int j) {
  float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int hh = 0; hh < a.G; ++hh) {
    const int h = g * a.G + hh;
    const float4 z = *reinterpret_cast<const float4*>(
        a.logits + ((size_t)b * a.Hq + h) * a.logits_stride + j);
    const float l = a.lse[(size_t)b * a.Hq + h];
    f.x += expf(z.x - l);
    f.y += expf(z.y - l);
    f.z += expf(z.z - l);
    f.w += expf(z.w - l);
  }
  const float invG = 1.f / (float)a.G;
  return make_float4(f.x * invG, f.y * invG, f.z * invG, f.w * invG);
}

__device__ __forceinline__ float flogf(float f) { return f > 0.f ? f * logf(f) : 0.f; }

__global__ __launch_bounds__(256) void k_sel_zsum(ZsumArgs za) {
  const float* __restrict__ key_norm = za.key_norm;
  const int64_t norm_stride = za.norm_stride;
  const int32_t* __restrict__ seq_lens = za.seq_lens;
  const int32_t* __restrict__ seq_ids = za.seq_ids;
  const int Hkv = za.Hkv, nchunk = za.nchunk;
  float* __restrict__ zpart = za.zpart;
  uint32_t* __restrict__ topk_hist = za.topk_hist;
  uint32_t* __restrict__ topk_state = za.topk_state;
  __shared__ float red[8];
  const int chunk = blockIdx.x % nchunk;
  const int ig = blockIdx.x / nchunk;
  if (seq_ids[ig / Hkv] < 0) return;  // unused slot of the row list (block-uniform)
  if (chunk == 0) {  // clear the top-K histogram and state of this (row, head)
    uint32_t* h = topk_hist + (size_t)ig * kTopkHistWords;
    for (int k = threadIdx.x; k < kTopkHistWords; k += 256) h[k] = 0;
    if (threadIdx.x < kTopkStateWords) topk_state[(size_t)ig * kTopkStateWords + threadIdx.x] = 0;
  }
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
  if (za.hpart) {
    float h = 0.f;
    for (int k = 0; k < 4; ++k) {
      const int j = j0 + 1024 * k;
      if (j + 3 < N) {
        const float4 f = evidence4(za, b, g, j);
        h += flogf(f.x) + flogf(f.y) + flogf(f.z) + flogf(f.w);
      } else if (j < N) {
        // the logits row holds at least N entries; read the tail one by one
        for (int q = 0; q < 4 && j + q < N; ++q) {
          float f = 0.f;
          for (int hh = 0; hh < za.G; ++hh) {
            const int hq = g * za.G + hh;
            f += expf(za.logits[((size_t)b * za.Hq + hq) * za.logits_stride + j + q] -
                      za.lse[(size_t)b * za.Hq + hq]);
          }
          h += flogf(f * (1.f / (float)za.G));
        }
      }
    }
    h = block_sum<256>(h, red);
    if (threadIdx.x == 0) za.hpart[blockIdx.x] = h;
  }
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
  const float* hpart;  // partial sums of f ln f (adaptive weight), or nullptr
  uint32_t* keys;
  int64_t kstride;
  float* dbg;
  int greedy;  // greedy soft-NMS: the keys carry s with exclusivity only
  int Hq, Hkv, G, nchunk, ntile, tile;
  int n_work;  // rows x tiles
  int n_sink, n_recent, R;
  float lam, a_soft, a_cross, lam_clip;
};

// One block per (row, tile of `tile` positions).  Every thread computes the fused score s
// of every KV head at one position of the tile or of the R-wide halo on either side,
// reading the logits of the position's query heads and the key norms straight from global
// memory (consecutive threads, consecutive positions), and leaves s in LDS.  Then, for the
// tile's candidates, the soft-NMS dominance (neighbours within R, same head), the
// ownership (all heads at the position) and the refined key.  Only s is staged, so the
// block needs little LDS and shares CUs well with attention running at the same time.
template <int GT>
__device__ __forceinline__ void score_block(const ScoreArgs& a, int work, float* lds) {
  const int G = GT > 0 ? GT : a.G;
  const int TILE = a.tile;
  const int R = a.R;
  const int W = TILE + 2 * R;
  float* s_t = lds;                   // [Hkv][W]  fused scores, column c = position t0 - R + c
  float* zs = s_t + a.Hkv * W;        // [Hkv]     prior normalisers
  float* lams = zs + a.Hkv;           // [Hkv]     fusion weights
  float* lses = lams + a.Hkv;         // [Hq]
  const int tid = threadIdx.x;
  const int i = work / a.ntile;
  const int tile = work % a.ntile;
  const int b = a.seq_ids[i];
  if (b < 0) return;  // unused slot of the row list (block-uniform)
  const int N = a.seq_lens[b];
  const int t0 = tile * TILE;
  if (t0 >= N) return;  // block-uniform
  const int lo = a.n_sink;
  const int hi = max(lo, N - a.n_recent);

  // Prior normalisers: eight lanes per KV head add every eighth chunk partial, then a
  // fixed-order reduction over the eight lanes (the same sum in every block).
  if (tid < 8 * a.Hkv) {
    const int g = tid >> 3, part = tid & 7;
    const float* zp = a.zpart + ((size_t)i * a.Hkv + g) * a.nchunk;
    float z = 0.f;
    for (int c = part; c < a.nchunk; c += 8) z += zp[c];
    z += __shfl_xor(z, 1, 8);
    z += __shfl_xor(z, 2, 8);
    z += __shfl_xor(z, 4, 8);
    if (part == 0) zs[g] = z;
    // fusion weight: fixed, or min(lambda_clip, H / ln N) from the f ln f partials
    float lam = a.lam;
    if (a.hpart) {
      const float* hp = a.hpart + ((size_t)i * a.Hkv + g) * a.nchunk;
      float t = 0.f;
      for (int c = part; c < a.nchunk; c += 8) t += hp[c];
      t += __shfl_xor(t, 1, 8);
      t += __shfl_xor(t, 2, 8);
      t += __shfl_xor(t, 4, 8);
      lam = N > 1 ? fminf(a.lam_clip, -t / logf((float)N)) : 0.f;
    }
    if (part == 0) lams[g] = lam;
  }
  for (int h = tid; h < a.Hq; h += 256) lses[h] = a.lse[(size_t)b * a.Hq + h];
  __syncthreads();

  // Fused scores over the tile and its halo.
  const float invG = 1.f / (float)G;
  for (int col = tid; col < W; col += 256) {
    const int j = t0 - R + col;
    const bool in = j >= 0 && j < N;
    const int jc = in ? j : 0;
    const float phi_pos = 1.f + logf(1.f + (float)(N - 1 - jc));
    const bool body = col >= R && col < R + TILE;
    const float* zrow = a.logits + (size_t)b * a.Hq * a.logits_stride + jc;
    const float* nrow = a.key_norm + (size_t)b * a.Hkv * a.norm_stride + jc;
    for (int g = 0; g < a.Hkv; ++g) {
      float f = 0.f;
      if (GT > 0) {
        float zv[GT > 0 ? GT : 1];
#pragma unroll
        for (int hh = 0; hh < (GT > 0 ? GT : 1); ++hh)
          zv[hh] = zrow[(size_t)(g * G + hh) * a.logits_stride];
#pragma unroll
        for (int hh = 0; hh < (GT > 0 ? GT : 1); ++hh) f += expf(zv[hh] - lses[g * G + hh]);
      } else {
        for (int hh = 0; hh < G; ++hh)
          f += expf(zrow[(size_t)(g * G + hh) * a.logits_stride] - lses[g * G + hh]);
      }
      f *= invG;
      const float r = (1.f / fmaxf(nrow[(size_t)g * a.norm_stride], 1e-6f)) * phi_pos / zs[g];
      const float s = (1.f - lams[g]) * f + lams[g] * r;
      if (in && a.dbg && body) a.dbg[((size_t)b * a.Hkv + g) * a.logits_stride + j] = s;
      s_t[g * W + col] = in ? s : -1.f;
    }
  }
  __syncthreads();

  // Refinement decisions and keys for the tile's candidates.
  const float ws = 1.f - a.a_soft, wc = 1.f - a.a_cross;
  for (int col = R + tid; col < R + TILE; col += 256) {
    const int j = t0 - R + col;
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
    const int dlo = max(lo, j - R) - j;      // <= 0
    const int dhi = min(hi - 1, j + R) - j;  // >= 0
    for (int g = 0; g < a.Hkv; ++g) {
      const float* row = s_t + g * W + col;
      const float sj = row[0];
      bool dom = false;
      if (!a.greedy)
        for (int d = dlo; d <= dhi; ++d) dom |= (d != 0) && (row[d] > sj);
      float sp = sj;
      if (dom) sp *= ws;
      if (a.Hkv > 1 && g != own) sp *= wc;
      a.keys[((size_t)i * a.Hkv + g) * a.kstride + (j - lo)] = f2u(sp) & 0x7fffffffu;
    }
  }
}

// Grid-stride over (row, tile) blocks: the grid is capped at one block per CU so the
// scoring leaves room for the attention that runs at the same time.
constexpr int kScoreMaxBlocks = 256;

// ------------------------------------------------------------------- greedy soft-NMS
// The greedy reading takes, per head, the candidate with the largest current score (the
// lower position on ties); it keeps that score, and every untaken candidate within R is
// scaled by 1 - alpha_soft; repeated until all are taken.  The takes are made here in
// rounds: a candidate that beats every untaken candidate within R (larger score, or equal
// score and lower position) is taken before any of them in the greedy order and keeps
// its current score, so every such local maximum is taken at once, and the untaken
// candidates are scaled once per neighbour taken in the round.  Every round takes the
// largest untaken candidate, so there are at most |C| rounds.  The result is the greedy
// one exactly: a candidate's score is scaled once for each neighbour taken before it in
// either order.
struct GreedyArgs {
  uint32_t* keys;   // in: s with exclusivity (IEEE bits of a score >= 0); out: taken scores
  int64_t kstride;
  int32_t* taken;   // [units][kstride]: round in which the candidate was taken, 0 = not yet
  int32_t* ready;   // [units][kstride]: round in which it was found ready
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  int Hkv, n_sink, n_recent, R;
  float decay;      // 1 - alpha_soft
};
constexpr int kGreedyThreads = 1024;

__global__ __launch_bounds__(kGreedyThreads) void k_greedy_nms(GreedyArgs a) {
  __shared__ int s_taken;
  const int ig = blockIdx.x;
  const int b = a.seq_ids[ig / a.Hkv];
  if (b < 0) return;  // unused slot of the row list (block-uniform)
  const int N = a.seq_lens[b];
  const int lo = a.n_sink, hi = max(lo, N - a.n_recent);
  const int n = hi - lo;
  const int R = a.R;
  uint32_t* key = a.keys + (size_t)ig * a.kstride;
  int32_t* tk = a.taken + (size_t)ig * a.kstride;
  int32_t* rd = a.ready + (size_t)ig * a.kstride;
  const int tid = threadIdx.x;
  for (int c = tid; c < n; c += kGreedyThreads) {
    tk[c] = 0;
    rd[c] = 0;
  }
  if (tid == 0) s_taken = 0;
  __syncthreads();
  int left = n;
  for (int round = 1; left > 0 && round <= n; ++round) {
    // Ready: untaken and larger than every untaken neighbour (lower position on ties).
    for (int c = tid; c < n; c += kGreedyThreads) {
      if (tk[c]) continue;
      const float vc = u2f(key[c]);
      bool ready = true;
      for (int d = -R; d <= R && ready; ++d) {
        const int k = c + d;
        if (d == 0 || k < 0 || k >= n || tk[k]) continue;
        const float vk = u2f(key[k]);
        if (vk > vc || (vk == vc && k < c)) ready = false;
      }
      if (ready) rd[c] = round;
    }
    __syncthreads();
    // Take the ready ones (their key is their final score); scale the others once per
    // neighbour taken now.
    int took = 0;
    for (int c = tid; c < n; c += kGreedyThreads) {
      if (tk[c]) continue;
      if (rd[c] == round) {
        tk[c] = round;
        ++took;
        continue;
      }
      int cnt = 0;
      for (int d = -R; d <= R; ++d) {
        const int k = c + d;
        cnt += (d != 0 && k >= 0 && k < n && rd[k] == round) ? 1 : 0;
      }
      if (cnt) {
        float v = u2f(key[c]);
        for (int q = 0; q < cnt; ++q) v *= a.decay;
        key[c] = f2u(v) & 0x7fffffffu;
      }
    }
    took = (int)wave_sum_xor((float)took, kWave);
    if ((tid & 63) == 0 && took) atomicAdd(&s_taken, took);
    __syncthreads();
    left = n - s_taken;
    __syncthreads();
  }
}

template <int GT>
__global__ __launch_bounds__(256) void k_sel_score(ScoreArgs a) {
  extern __shared__ float lds[];
  for (int work = blockIdx.x; work < a.n_work; work += gridDim.x) {
    score_block<GT>(a, work, lds);
    __syncthreads();  // the next block reuses the LDS
  }
}

// ------------------------------------------------------------------------------- top-K
// Radix selection of the K_eff-th largest refined key per (row, KV head), spread over the
// chip in slices of 4096 candidates:
//   k_topk_hist    per slice: LDS histogram of the top 11 key bits, flushed into a global
//                  2048-bin histogram of the (row, head);
//   k_topk_gather  per slice: locate the bin holding the K_eff-th key, count the slice's
//                  keys above that bin and append the keys inside it, with their
//                  candidate indices, to a short candidate list;
//   k_topk_final   per (row, head), 512 threads: resolve the remaining 21 bits on the
//                  candidate list in LDS, giving the exact threshold T and the number of
//                  keys equal to T still to take; the last of those ties (lowest
//                  positions first) is found by the same selection on the complemented
//                  candidate index; then the output offset of every slice.  If the bin
//                  holds more keys than the list takes, a single-block path selects from
//                  the keys in global memory instead and writes the result itself;
//   k_topk_write   per slice: every key above T and the taken ties, ascending.
constexpr int kTopkThreads = 512;   // one-block stages: fits beside attention on a CU
constexpr int kSliceThreads = 256;
constexpr int kKeysPerThread = 16;
constexpr int kSlice = kSliceThreads * kKeysPerThread;  // candidates per slice
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
static_assert(kHistBins == kTopkHistWords, "global histogram size");
constexpr int kCandCap = kCandCapBytes / 8;  // key + index per candidate
constexpr int kMaxSlices = 1024;
static_assert(kMaxSlices % kTopkThreads == 0, "slices per thread");

// Per-(row, head) state words.
constexpr int kStCount = 0;  // candidates appended by k_topk_gather
constexpr int kStMode = 1;   // kModeWrite: k_topk_write emits; kModeDone: already written
constexpr int kStT = 2;      // threshold key
constexpr int kStCLast = 3;  // last tie taken (candidate index)
constexpr int kStWords = kTopkStateWords;
constexpr uint32_t kModeWrite = 0, kModeDone = 1;

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

// Bin of hist[0..2048) holding the krem-th largest counted element; thread t owns the
// 2048 / BLOCK bins just below 2048 - t * (2048 / BLOCK).  Writes (bin, count above the
// bin) to res[0..1].  All threads call.
template <int BLOCK>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t krem, uint32_t* wsum,
                                         uint32_t* res) {
  constexpr int BPT = kHistBins / BLOCK;
  const int top = kHistBins - 1 - BPT * (int)threadIdx.x;
  uint32_t h[BPT], sum = 0;
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    h[k] = hist[top - k];
    sum += h[k];
  }
  uint32_t tot;
  uint32_t above = block_exscan<BLOCK>(sum, wsum, &tot);
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    if (above < krem && above + h[k] >= krem) {
      res[0] = top - k;
      res[1] = above;
    }
    above += h[k];
  }
  __syncthreads();
}

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

// Visit keys [0, n) in chunks of 16 per thread (kTopkThreads threads); the next chunk is
// requested before the current one is processed (two register buffers, unrolled so they
// swap roles without copies).  f(c, kv) sees the keys at candidate indices c .. c+15 and
// is called by every thread the same number of times (it may contain block barriers).
template <typename F>
__device__ __forceinline__ void pass16(const uint32_t* keys, int64_t kstride, int n, F&& f) {
  constexpr int STEP = kKeysPerThread * kTopkThreads;
  const int off = kKeysPerThread * (int)threadIdx.x;
  uint32_t A[kKeysPerThread], B[kKeysPerThread];
  load16(keys, kstride, off, A);
  for (int base = 0; base < n; base += 2 * STEP) {
    load16(keys, kstride, base + STEP + off, B);
    f(base + off, A);
    if (base + STEP >= n) break;
    load16(keys, kstride, base + 2 * STEP + off, A);
    f(base + STEP + off, B);
  }
}

struct TopkArgs {
  const uint32_t* keys;
  int64_t kstride;
  const int32_t* seq_lens;
  const int32_t* seq_ids;
  int32_t* sel;
  uint32_t* hist;         // [n_seqs * Hkv][2048]
  uint32_t* state;        // [n_seqs * Hkv][kStWords]
  uint32_t* slice_above;  // [n_seqs * Hkv][nslice]
  uint32_t* slice_off;    // [n_seqs * Hkv][nslice]
  uint32_t* cand_key;     // [n_seqs * Hkv][kCandCap]
  uint32_t* cand_idx;     // [n_seqs * Hkv][kCandCap]
  int Hkv, K, n_sink, n_recent, nslice;
};

struct TopkRow {
  int b, lo, nC, keff;
};

__device__ __forceinline__ TopkRow topk_row(const TopkArgs& a, int i) {
  TopkRow r;
  r.b = a.seq_ids[i];
  const int N = r.b < 0 ? 0 : a.seq_lens[r.b];  // an unused slot has no candidates
  r.lo = a.n_sink;
  const int hi = max(r.lo, N - a.n_recent);
  r.nC = hi - r.lo;
  r.keff = min(a.K, r.nC);
  return r;
}

__global__ __launch_bounds__(kSliceThreads) void k_topk_hist(TopkArgs a) {
  __shared__ uint32_t hist[kHistBins];
  const int tid = threadIdx.x;
  const int sl = blockIdx.x % a.nslice;
  const int ig = blockIdx.x / a.nslice;
  const TopkRow row = topk_row(a, ig / a.Hkv);
  const int c0 = sl * kSlice;
  if (row.keff == 0 || row.keff == row.nC || c0 >= row.nC) return;  // block-uniform
  for (int k = tid; k < kHistBins; k += kSliceThreads) hist[k] = 0;
  __syncthreads();
  const int c = c0 + kKeysPerThread * tid;
  uint32_t kv[kKeysPerThread];
  load16(a.keys + (size_t)ig * a.kstride, a.kstride, c, kv);
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q)
    hist_add(hist, kv[q] >> (32 - kHistBits), c + q < row.nC);
  __syncthreads();
  uint32_t* gh = a.hist + (size_t)ig * kHistBins;
  for (int k = tid; k < kHistBins; k += kSliceThreads) {
    const uint32_t h = hist[k];
    if (h) atomicAdd(&gh[k], h);
  }
}

__global__ __launch_bounds__(kSliceThreads) void k_topk_gather(TopkArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[kSliceThreads / 64 + 1];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x;
  const int sl = blockIdx.x % a.nslice;
  const int ig = blockIdx.x / a.nslice;
  const TopkRow row = topk_row(a, ig / a.Hkv);
  const int c0 = sl * kSlice;
  if (row.keff == 0 || row.keff == row.nC || c0 >= row.nC) return;  // block-uniform
  const uint32_t* gh = a.hist + (size_t)ig * kHistBins;
  for (int k = tid; k < kHistBins; k += kSliceThreads) hist[k] = gh[k];
  __syncthreads();
  find_bin<kSliceThreads>(hist, (uint32_t)row.keff, wsum, res);
  const uint32_t d = res[0];
  const bool list_ok = hist[d] <= (uint32_t)kCandCap;
  const int c = c0 + kKeysPerThread * tid;
  uint32_t kv[kKeysPerThread];
  load16(a.keys + (size_t)ig * a.kstride, a.kstride, c, kv);
  uint32_t n_above = 0, n_in = 0;
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) {
    const bool valid = c + q < row.nC;
    const uint32_t bin = kv[q] >> (32 - kHistBits);
    n_above += (valid && bin > d) ? 1u : 0u;
    n_in += (valid && bin == d) ? 1u : 0u;
  }
  // One scan for both counts (each at most 4096 per block): above in the high half.
  uint32_t tot;
  const uint32_t pre = block_exscan<kSliceThreads>((n_above << 16) | n_in, wsum, &tot);
  if (tid == 0) a.slice_above[(size_t)ig * a.nslice + sl] = tot >> 16;
  if (list_ok) {
    if (tid == 0) res[2] = atomicAdd(&a.state[(size_t)ig * kStWords + kStCount], tot & 0xffffu);
    __syncthreads();
    uint32_t slot = res[2] + (pre & 0xffffu);
    uint32_t* ck = a.cand_key + (size_t)ig * kCandCap;
    uint32_t* ci = a.cand_idx + (size_t)ig * kCandCap;
#pragma unroll
    for (int q = 0; q < kKeysPerThread; ++q) {
      if (c + q < row.nC && (kv[q] >> (32 - kHistBits)) == d && slot < (uint32_t)kCandCap) {
        ck[slot] = kv[q];
        ci[slot] = (uint32_t)(c + q);
        ++slot;
      }
    }
  }
}

// Radix selection on the candidate list in LDS: resolves the key bits below `done` and
// then the last tie by candidate index.  Returns T, need_eq and c_last.
__device__ void select_in_lds(const uint32_t* ckey, const uint32_t* cidx, int n, uint32_t prefix,
                              int done, uint32_t krem, uint32_t* hist, uint32_t* wsum,
                              uint32_t* res, uint32_t& T, uint32_t& c_last) {
  const int tid = threadIdx.x;
  uint32_t n_eq = 0;  // candidates equal to the prefix once all 32 bits are fixed
  while (done < 32) {
    const int nb = min(kHistBits, 32 - done);
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
    find_bin<kTopkThreads>(hist, krem, wsum, res);
    krem -= res[1];
    n_eq = hist[res[0]];
    prefix = (prefix << nb) | res[0];
    done += nb;
    __syncthreads();
  }
  T = prefix;
  if (n_eq == krem) {  // every tie at T is taken
    c_last = 0xffffffffu;
    return;
  }
  // ties at T: the krem-th smallest candidate index is the last one taken
  uint32_t uprefix = 0, urem = krem;
  int udone = 0;
  while (udone < 32) {
    const int nb = min(kHistBits, 32 - udone);
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
    find_bin<kTopkThreads>(hist, urem, wsum, res);
    urem -= res[1];
    uprefix = (uprefix << nb) | res[0];
    udone += nb;
    __syncthreads();
  }
  c_last = ~uprefix;
}

// Whole selection of one (row, head) by one block from the keys in global memory; the
// path for a boundary bin larger than the candidate list (massive ties, very flat
// scores).  Writes out[0 .. keff).
__device__ void topk_single_block(const uint32_t* keys, int64_t kstride, int nC, int keff,
                                  int lo, int32_t* out, uint32_t* hist, uint32_t* ckey,
                                  uint32_t* cidx, uint32_t* wsum, uint32_t* res) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, krem = (uint32_t)keff, cnt = 0;
  int done = 0;
  while (true) {
    const int nb = min(kHistBits, 32 - done);
    const int sh = 32 - done - nb;
    for (int k = tid; k < kHistBins; k += kTopkThreads) hist[k] = 0;
    __syncthreads();
    pass16(keys, kstride, nC, [&](int c, const uint32_t* kv) {
#pragma unroll
      for (int q = 0; q < kKeysPerThread; ++q) {
        const bool match = c + q < nC && (done == 0 || (kv[q] >> (32 - done)) == prefix);
        hist_add(hist, (kv[q] >> sh) & ((1u << nb) - 1u), match);
      }
    });
    __syncthreads();
    find_bin<kTopkThreads>(hist, krem, wsum, res);
    const uint32_t d = res[0];
    krem -= res[1];
    cnt = hist[d];
    prefix = (prefix << nb) | d;
    done += nb;
    __syncthreads();
    if (cnt <= (uint32_t)kCandCap || done == 32) break;
  }
  uint32_t T, need_eq = krem, c_last = 0xffffffffu;
  bool by_index = false;
  if (done == 32) {
    T = prefix;
  } else {
    if (tid == 0) res[2] = 0;
    __syncthreads();
    pass16(keys, kstride, nC, [&](int c, const uint32_t* kv) {
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
    select_in_lds(ckey, cidx, (int)res[2], prefix, done, krem, hist, wsum, res, T, c_last);
    by_index = true;
  }
  uint32_t taken = 0, eq_seen = 0;
  pass16(keys, kstride, nC, [&](int c, const uint32_t* kv) {
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
      uint32_t eq_before = eq_seen + block_exscan<kTopkThreads>(neq, wsum, &eq_tot);
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
    uint32_t at = taken + block_exscan<kTopkThreads>(nsel, wsum, &sel_tot);
#pragma unroll
    for (int q = 0; q < kKeysPerThread; ++q)
      if (take[q] && at < (uint32_t)keff) out[at++] = lo + c + q;
    taken += sel_tot;
  });
}

__global__ __launch_bounds__(kTopkThreads) void k_topk_final(TopkArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t ckey[kCandCap];
  __shared__ uint32_t cidx[kCandCap];
  __shared__ uint32_t cnt_sl[kMaxSlices];
  __shared__ uint32_t wsum[kTopkThreads / 64 + 1];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x;
  const int ig = blockIdx.x;
  const TopkRow row = topk_row(a, ig / a.Hkv);
  if (row.b < 0) return;  // unused slot of the row list
  const int g = ig % a.Hkv;
  int32_t* out = a.sel + ((size_t)row.b * a.Hkv + g) * a.K;
  uint32_t* st = a.state + (size_t)ig * kStWords;
  for (int k = row.keff + tid; k < a.K; k += kTopkThreads) out[k] = -1;
  if (row.keff == 0 || row.keff == row.nC) {  // nothing to rank: none or every candidate
    for (int k = tid; k < row.keff; k += kTopkThreads) out[k] = row.lo + k;
    if (tid == 0) st[kStMode] = kModeDone;
    return;
  }
  const uint32_t* gh = a.hist + (size_t)ig * kHistBins;
  for (int k = tid; k < kHistBins; k += kTopkThreads) hist[k] = gh[k];
  __syncthreads();
  find_bin<kTopkThreads>(hist, (uint32_t)row.keff, wsum, res);
  const uint32_t d = res[0];
  const uint32_t krem = (uint32_t)row.keff - res[1];
  const uint32_t cnt = hist[d];
  __syncthreads();
  const uint32_t* keys = a.keys + (size_t)ig * a.kstride;
  if (cnt > (uint32_t)kCandCap) {
    topk_single_block(keys, a.kstride, row.nC, row.keff, row.lo, out, hist, ckey, cidx, wsum,
                      res);
    if (tid == 0) st[kStMode] = kModeDone;
    return;
  }
  const int n = (int)cnt;
  const uint32_t* gk = a.cand_key + (size_t)ig * kCandCap;
  const uint32_t* gi = a.cand_idx + (size_t)ig * kCandCap;
  for (int e = tid; e < n; e += kTopkThreads) {
    ckey[e] = gk[e];
    cidx[e] = gi[e];
  }
  __syncthreads();
  uint32_t T, c_last;
  select_in_lds(ckey, cidx, n, d, kHistBits, krem, hist, wsum, res, T, c_last);
  // Selected count of every slice: keys above the bin plus the taken candidates.
  const int nsl = (row.nC + kSlice - 1) / kSlice;
  const uint32_t* above = a.slice_above + (size_t)ig * a.nslice;
  for (int k = tid; k < nsl; k += kTopkThreads) cnt_sl[k] = above[k];
  __syncthreads();
  for (int e = tid; e < n; e += kTopkThreads) {
    const uint32_t key = ckey[e], idx = cidx[e];
    if (key > T || (key == T && idx <= c_last)) atomicAdd(&cnt_sl[idx / kSlice], 1u);
  }
  __syncthreads();
  // Output offset of every slice: exclusive scan, kSlicesPerThread consecutive slices per
  // thread.
  constexpr int kSlicesPerThread = kMaxSlices / kTopkThreads;
  uint32_t v[kSlicesPerThread], sum = 0;
#pragma unroll
  for (int k = 0; k < kSlicesPerThread; ++k) {
    const int sl = kSlicesPerThread * tid + k;
    v[k] = sl < nsl ? cnt_sl[sl] : 0u;
    sum += v[k];
  }
  uint32_t tot;
  uint32_t off = block_exscan<kTopkThreads>(sum, wsum, &tot);
#pragma unroll
  for (int k = 0; k < kSlicesPerThread; ++k) {
    const int sl = kSlicesPerThread * tid + k;
    if (sl < nsl) a.slice_off[(size_t)ig * a.nslice + sl] = off;
    off += v[k];
  }
  if (tid == 0) {
    st[kStT] = T;
    st[kStCLast] = c_last;
    st[kStMode] = kModeWrite;
  }
}

// Rows of at most kSmallSlices slices (16384 positions): one block per (row, head) ranks
// the keys straight from global memory (topk_single_block), so the selection is one launch
// instead of the four-kernel chain above, whose launches dominate at this size.
constexpr int kSmallSlices = 4;

__global__ __launch_bounds__(kTopkThreads) void k_topk_small(TopkArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t ckey[kCandCap];
  __shared__ uint32_t cidx[kCandCap];
  __shared__ uint32_t wsum[kTopkThreads / 64 + 1];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x;
  const int ig = blockIdx.x;
  const TopkRow row = topk_row(a, ig / a.Hkv);
  if (row.b < 0) return;  // unused slot of the row list
  int32_t* out = a.sel + ((size_t)row.b * a.Hkv + ig % a.Hkv) * a.K;
  for (int k = row.keff + tid; k < a.K; k += kTopkThreads) out[k] = -1;
  if (row.keff == 0 || row.keff == row.nC) {  // nothing to rank: none or every candidate
    for (int k = tid; k < row.keff; k += kTopkThreads) out[k] = row.lo + k;
    return;
  }
  topk_single_block(a.keys + (size_t)ig * a.kstride, a.kstride, row.nC, row.keff, row.lo, out,
                    hist, ckey, cidx, wsum, res);
}

__global__ __launch_bounds__(kSliceThreads) void k_topk_write(TopkArgs a) {
  __shared__ uint32_t wsum[kSliceThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int sl = blockIdx.x % a.nslice;
  const int ig = blockIdx.x / a.nslice;
  const TopkRow row = topk_row(a, ig / a.Hkv);
  const int c0 = sl * kSlice;
  if (row.keff == 0 || row.keff == row.nC || c0 >= row.nC) return;  // block-uniform
  const uint32_t* st = a.state + (size_t)ig * kStWords;
  if (st[kStMode] != kModeWrite) return;
  const uint32_t T = st[kStT], c_last = st[kStCLast];
  const int c = c0 + kKeysPerThread * tid;
  uint32_t kv[kKeysPerThread];
  load16(a.keys + (size_t)ig * a.kstride, a.kstride, c, kv);
  bool take[kKeysPerThread];
  uint32_t nsel = 0;
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) {
    take[q] = c + q < row.nC && (kv[q] > T || (kv[q] == T && (uint32_t)(c + q) <= c_last));
    nsel += take[q] ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t at = a.slice_off[(size_t)ig * a.nslice + sl] +
                block_exscan<kSliceThreads>(nsel, wsum, &tot);
  int32_t* out = a.sel + ((size_t)row.b * a.Hkv + ig % a.Hkv) * a.K;
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q)
    if (take[q] && at < (uint32_t)row.keff) out[at++] = row.lo + c + q;
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

SelectLayout select_layout(const sfi_shape& s, int n_seqs, int max_seq_len, bool greedy) {
  SelectLayout L;
  L.nchunk = (max_seq_len + kZChunk - 1) / kZChunk;
  L.kstride = ((int64_t)max_seq_len + 63) / 64 * 64;
  L.nslice = (max_seq_len + kSlice - 1) / kSlice;
  const size_t units = (size_t)n_seqs * s.num_kv_heads;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  L.zpart_off = take(units * L.nchunk * sizeof(float));
  L.hpart_off = take(units * L.nchunk * sizeof(float));
  L.keys_off = take(units * (size_t)L.kstride * sizeof(uint32_t));
  if (greedy) {
    L.taken_off = take(units * (size_t)L.kstride * sizeof(int32_t));
    L.ready_off = take(units * (size_t)L.kstride * sizeof(int32_t));
  }
  L.hist_off = take(units * kHistBins * sizeof(uint32_t));
  L.state_off = take(units * kStWords * sizeof(uint32_t));
  L.above_off = take(units * L.nslice * sizeof(uint32_t));
  L.sloff_off = take(units * L.nslice * sizeof(uint32_t));
  L.ckey_off = take(units * kCandCap * sizeof(uint32_t));
  L.cidx_off = take(units * kCandCap * sizeof(uint32_t));
  L.total = off;
  return L;
}

size_t score_lds_bytes(int num_kv_heads, int num_q_heads, int nms_radius, int tile) {
  const size_t W = (size_t)tile + 2 * (size_t)nms_radius;
  return sizeof(float) * ((size_t)num_kv_heads * W + 2 * num_kv_heads + num_q_heads);
}

int score_tile(int num_kv_heads, int num_q_heads, int nms_radius) {
  // One position per thread when the halo allows it (256 - 2R), else 64 positions.
  const int tile = nms_radius <= 96 ? 256 - 2 * nms_radius : 64;
  return score_lds_bytes(num_kv_heads, num_q_heads, nms_radius, tile) <= kScoreLdsLimit ? tile
                                                                                     : 0;
}

namespace {

void launch_score(ScoreArgs a, int n_seqs, size_t lds, hipStream_t st) {
  a.n_work = n_seqs * a.ntile;
  const dim3 grid(a.n_work < kScoreMaxBlocks ? a.n_work : kScoreMaxBlocks), block(256);
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
  const bool greedy = prm.nms_greedy != 0;
  const SelectLayout L = select_layout(s, n_seqs, max_seq_len, greedy);
  char* w = reinterpret_cast<char*>(ws);
  float* zpart = reinterpret_cast<float*>(w + L.zpart_off);
  const bool adaptive = prm.lambda_clip >= 0.f;
  float* hpart = adaptive ? reinterpret_cast<float*>(w + L.hpart_off) : nullptr;
  uint32_t* keys = reinterpret_cast<uint32_t*>(w + L.keys_off);
  const int Hkv = s.num_kv_heads, Hq = s.num_q_heads;
  ZsumArgs za;
  za.key_norm = key_norm;
  za.norm_stride = norm_stride;
  za.seq_lens = seq_lens;
  za.seq_ids = seq_ids;
  za.Hkv = Hkv;
  za.nchunk = L.nchunk;
  za.zpart = zpart;
  za.topk_hist = reinterpret_cast<uint32_t*>(w + L.hist_off);
  za.topk_state = reinterpret_cast<uint32_t*>(w + L.state_off);
  za.logits = logits;
  za.logits_stride = logits_stride;
  za.lse = lse;
  za.Hq = Hq;
  za.G = Hq / Hkv;
  za.hpart = hpart;
  hipLaunchKernelGGL(k_sel_zsum, dim3(n_seqs * Hkv * L.nchunk), dim3(256), 0, st, za);
  ScoreArgs a;
  a.logits = logits;
  a.logits_stride = logits_stride;
  a.lse = lse;
  a.key_norm = key_norm;
  a.norm_stride = norm_stride;
  a.seq_lens = seq_lens;
  a.seq_ids = seq_ids;
  a.zpart = zpart;
  a.hpart = hpart;
  a.keys = keys;
  a.kstride = L.kstride;
  a.dbg = dbg;
  a.greedy = greedy ? 1 : 0;
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
  a.lam_clip = prm.lambda_clip;
  a.tile = score_tile(Hkv, Hq, prm.nms_radius);
  a.ntile = (max_seq_len + a.tile - 1) / a.tile;
  launch_score(a, n_seqs, score_lds_bytes(Hkv, Hq, prm.nms_radius, a.tile), st);
  if (greedy) {
    GreedyArgs gr;
    gr.keys = keys;
    gr.kstride = L.kstride;
    gr.taken = reinterpret_cast<int32_t*>(w + L.taken_off);
    gr.ready = reinterpret_cast<int32_t*>(w + L.ready_off);
    gr.seq_lens = seq_lens;
    gr.seq_ids = seq_ids;
    gr.Hkv = Hkv;
    gr.n_sink = prm.n_sink;
    gr.n_recent = prm.n_recent;
    gr.R = prm.nms_radius;
    gr.decay = 1.f - prm.alpha_soft;
    hipLaunchKernelGGL(k_greedy_nms, dim3(n_seqs * Hkv), dim3(kGreedyThreads), 0, st, gr);
  }
  TopkArgs t;
  t.keys = keys;
  t.kstride = L.kstride;
  t.seq_lens = seq_lens;
  t.seq_ids = seq_ids;
  t.sel = sel_idx;
  t.hist = reinterpret_cast<uint32_t*>(w + L.hist_off);
  t.state = reinterpret_cast<uint32_t*>(w + L.state_off);
  t.slice_above = reinterpret_cast<uint32_t*>(w + L.above_off);
  t.slice_off = reinterpret_cast<uint32_t*>(w + L.sloff_off);
  t.cand_key = reinterpret_cast<uint32_t*>(w + L.ckey_off);
  t.cand_idx = reinterpret_cast<uint32_t*>(w + L.cidx_off);
  t.Hkv = Hkv;
  t.K = prm.top_k;
  t.n_sink = prm.n_sink;
  t.n_recent = prm.n_recent;
  t.nslice = L.nslice;
  if (L.nslice <= kSmallSlices) {
    hipLaunchKernelGGL(k_topk_small, dim3(n_seqs * Hkv), dim3(kTopkThreads), 0, st, t);
    return hipGetLastError();
  }
  const dim3 slices(n_seqs * Hkv * L.nslice);
  hipLaunchKernelGGL(k_topk_hist, slices, dim3(kSliceThreads), 0, st, t);
  hipLaunchKernelGGL(k_topk_gather, slices, dim3(kSliceThreads), 0, st, t);
  hipLaunchKernelGGL(k_topk_final, dim3(n_seqs * Hkv), dim3(kTopkThreads), 0, st, t);
  hipLaunchKernelGGL(k_topk_write, slices, dim3(kSliceThreads), 0, st, t);
  return hipGetLastError();
}

}  // namespace sfi
