// Split-K decode attention for SFI slow steps (dense, over the paged cache) and fast
// steps (two segments: the packed sink+selected buffer and the recent window in pages).
//
// Slow steps attend densely to the whole history and expose their logits as the
// Selector's evidence (es "2. Metodología", zh "2.1 慢快推理框架" and "2.2 训练无感的 Selector");
// fast steps attend to the compact contiguous buffer plus the recent tokens read straight
// from the paged cache (zh "2.3 系统级优化", nl "Systeemontwerp en Kernel-optimalisatie").
//
// One workgroup of four wavefronts owns one split: a run of 16-row tiles of one (row b,
// KV head g); the waves take every fourth tile and merge their results in LDS, so each
// split leaves one partial.  All G <= 16 query heads of g share the K/V reads.  bf16
// caches go through MFMA:
//   * logits   z[16 rows x 16 heads] = K_tile(16x D) * Q^T, as D/32 steps of
//     v_mfma_f32_16x16x32_bf16.  q is split exactly into three bf16 terms (hi+mid+lo,
//     truncation, so hi+mid+lo == q), and every bf16 x bf16 product is exact in fp32,
//     which keeps z at fp32 accuracy.
//   * V^T      the same MFMA against 0/1 selection matrices turns the row-major V tile
//     into the column layout the PV product needs (exact: one nonzero term per output).
//   * PV       O^T[dim][head] += V^T * P^T with v_mfma_f32_16x16x16bf16, P split into two
//     bf16 terms (relative error < 2^-16).
//   Lane l = 16*qd + r holds row r of each loaded K/V tile (16 B per 32-dim step: every
//   wave load reads 16 contiguous 64-byte segments) and, after the products, logits and
//   probabilities of head r at rows 4*qd .. 4*qd+3.
// fp32 caches use a plain VALU path with the same partial-result format.
// Each split writes its running (max m, sum l, unnormalised o); a merge kernel combines
// the splits of every query head with log-sum-exp weights.
#include "sfi_device.h"
#include "sfi_internal.h"

#include <math.h>

namespace sfi {

static_assert(kMaxG == kMaxGroup, "one MFMA tile covers every query head of a KV head");

constexpr int kMaxTilesPerSplit = 512;  // page indices of one split staged in LDS

namespace {

struct SplitRange {
  bool packed;
  int row_lo, row_hi;  // valid logical rows
  int t0, t1;          // tile range [t0, t1): rows [16 t, 16 t + 16)
};

__device__ __forceinline__ SplitRange split_range(const AttnParams& p, int b, int g, int split,
                                                  int N) {
  SplitRange sr;
  if (!p.fast) {
    sr.packed = false;
    sr.row_lo = 0;
    sr.row_hi = N;
    const int ntile = (N + kPage - 1) / kPage;
    sr.t0 = split * p.tps;
    sr.t1 = min(sr.t0 + p.tps, ntile);
  } else if (split < p.nsplit_a) {
    const int plen = min(max(uniform(p.packed_len[b * p.Hkv + g]), 0), p.packed_cap);
    sr.packed = true;
    sr.row_lo = 0;
    sr.row_hi = plen;
    const int ntile = (plen + kPage - 1) / kPage;
    sr.t0 = split * p.tps;
    sr.t1 = min(sr.t0 + p.tps, ntile);
  } else {
    const int rs = min(max(uniform(p.recent_start[b]), 0), N);
    sr.packed = false;
    sr.row_lo = rs;
    sr.row_hi = N;
    const int first = rs / kPage;
    const int last = (N + kPage - 1) / kPage;
    sr.t0 = first + (split - p.nsplit_a) * p.tps_b;
    sr.t1 = min(sr.t0 + p.tps_b, last);
  }
  return sr;
}

// Device-side contracts of row b (and KV head g): a broken one is clamped by the kernels
// and reported in the call's status word.  Called by one lane of the first split.
__device__ void report_contracts(const AttnParams& p, int b, int g) {
  uint32_t f = 0;
  const int raw_n = p.seq_lens[b];
  if (raw_n < 0 || raw_n > p.max_len) f |= SFI_DEV_SEQ_LEN;
  if (p.fast) {
    const int N = min(max(raw_n, 0), p.max_len);
    const int pl = p.packed_len[b * p.Hkv + g];
    if (pl < 0 || pl > p.packed_cap) f |= SFI_DEV_PACKED_LEN;
    const int rs = p.recent_start[b];
    if (rs < 0 || rs > N ||
        (N + kPage - 1) / kPage - rs / kPage > (p.nsplit - p.nsplit_a) * p.tps_b)
      f |= SFI_DEV_RECENT;
  }
  if (f) atomicOr(p.status, f);
}

__device__ __forceinline__ void write_empty_partial(const AttnParams& p, size_t pidx, int D,
                                                    int lane) {
  for (int h = lane; h < p.G; h += kWave) {
    p.part_m[pidx * p.G + h] = -INFINITY;
    p.part_l[pidx * p.G + h] = 0.f;
  }
  float* o = p.part_o + pidx * p.G * D;
  for (int k = lane; k < p.G * D; k += kWave) o[k] = 0.f;
}

// Split x into hi + mid + lo, three truncated bf16 values whose sum is exactly x.
__device__ __forceinline__ void split3(float x, float& hi, float& mid, float& lo) {
  hi = trunc_bf16(x);
  const float r1 = x - hi;
  mid = trunc_bf16(r1);
  lo = trunc_bf16(r1 - mid);
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

constexpr int kAttnWaves = 4;  // wavefronts per bf16 workgroup; they share one split

// LDS of one bf16 workgroup.
template <int D>
struct Bf16Lds {
  float m[kAttnWaves][kMaxG], l[kAttnWaves][kMaxG];
  float o[kAttnWaves - 1][kMaxG][D];
  int32_t page[kMaxTilesPerSplit];
};

// Split `work` of the call described by p (one workgroup).
template <int D, bool WRITE_Z>
__device__ __forceinline__ void attn_partial_bf16(AttnParams p, int work, Bf16Lds<D>& lds) {
  constexpr int NC = D / 32;   // 32-dim steps of the logit product
  constexpr int NT = D / 16;   // 16-dim output tiles of the PV product
  constexpr int NW = kAttnWaves;
  auto& sm_m = lds.m;
  auto& sm_l = lds.l;
  auto& sm_o = lds.o;
  auto& sm_page = lds.page;
  const int lane = threadIdx.x & 63;
  // Wave-uniform by construction; readfirstlane lets the compiler keep tile indices and
  // page-table reads scalar (s_load, counted by lgkmcnt) instead of vector loads whose
  // wait would also drain the in-flight K/V prefetch.
  const int wave = uniform(threadIdx.x >> 6);
  if (work >= p.n_seqs * p.Hkv * p.nsplit) return;  // workgroup-uniform
  const int split = work % p.nsplit;
  const int ig = work / p.nsplit;
  const int g = ig % p.Hkv;
  const int i = ig / p.Hkv;
  const int b = uniform(p.seq_ids[i]);
  if (b < 0) return;  // unused slot of the row list (workgroup-uniform)
  if (split == 0 && p.status && threadIdx.x == 0) report_contracts(p, b, g);
  const int r = lane & 15;
  const int qd = lane >> 4;
  const size_t pidx = (size_t)ig * p.nsplit + split;
  const int lane_off = r * D + 8 * qd;

  // Query of head r, dims 32c + 8qd .. +8 for c < NC: requested before any K/V tile, so it
  // is the first load of the wave to return (the wave's loads return in order) and the
  // first tile's products never wait for it behind the tile requests of the whole chip.
  float4 qraw[2 * NC];
  {
    const bool hv = r < p.G;
    const float* qrow = p.q + ((size_t)b * p.Hq + (size_t)g * p.G + (hv ? r : 0)) * D + 8 * qd;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qraw[2 * c] = *reinterpret_cast<const float4*>(qrow + 32 * c);
      qraw[2 * c + 1] = *reinterpret_cast<const float4*>(qrow + 32 * c + 4);
    }
  }

  const bool packed = p.fast && split < p.nsplit_a;
  const uint16_t* kbase;
  const uint16_t* vbase;
  if (packed) {
    const size_t off = ((size_t)b * p.Hkv + g) * (size_t)p.packed_cap * D;
    kbase = reinterpret_cast<const uint16_t*>(p.packed_k) + off;
    vbase = reinterpret_cast<const uint16_t*>(p.packed_v) + off;
  } else {
    kbase = reinterpret_cast<const uint16_t*>(p.k_cache);
    vbase = reinterpret_cast<const uint16_t*>(p.v_cache);
  }
  auto load_rows = [&](size_t off, u32x4_t* kk, u32x4_t* vv) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kk[c] = *reinterpret_cast<const u32x4_t*>(kbase + off + 32 * c);
      vv[c] = *reinterpret_cast<const u32x4_t*>(vbase + off + 32 * c);
    }
  };
  // A packed tile's address depends only on the row, the KV head and the tile index, so
  // a packed split requests its wave's first two tiles before the split's extent is known
  // (indices clamped to the split's share of the buffer's capacity, so no split fetches
  // another's tiles); their latency overlaps the set-up below.
  u32x4_t ka[NC], va[NC], kb[NC], vb[NC];
  if (packed) {
    const int last = min((split + 1) * p.tps, p.packed_cap / kPage) - 1;
    const int t0w = split * p.tps + wave;
    load_rows((size_t)min(t0w, last) * (kPage * D) + lane_off, ka, va);
    load_rows((size_t)min(t0w + NW, last) * (kPage * D) + lane_off, kb, vb);
  }
  // clamped: a length past the call's bound cannot send an index out of the buffers
  const int N = min(max(uniform(p.seq_lens[b]), 0), p.max_len);

  const SplitRange sr = split_range(p, b, g, split, N);
  if (sr.t0 >= sr.t1) {  // workgroup-uniform
    if (wave == 0) write_empty_partial(p, pidx, D, lane);
    return;
  }
  // Wave w takes tiles t0 + w, t0 + w + NW, ...
  const int wt0 = sr.t0 + wave;
  // Physical pages of the split, staged once in LDS: the per-tile lookups then wait on
  // the LDS counter only and never on the in-flight K/V loads.
  if (!packed) {
    const int32_t* btg = p.block_table + (size_t)b * p.max_pages + sr.t0;
    for (int k = threadIdx.x; k < sr.t1 - sr.t0; k += 256) sm_page[k] = btg[k];
  }
  __syncthreads();

  float* zrow = (WRITE_Z && r < p.G)
                    ? p.logits + ((size_t)b * p.Hq + (size_t)g * p.G + r) * p.logits_stride
                    : nullptr;

  auto tile_offset = [&](int t) -> size_t {
    if (packed) return (size_t)t * kPage * D;
    const int page = uniform(sm_page[t - sr.t0]);
    return ((size_t)page * p.Hkv + g) * (size_t)(kPage * D);
  };
  auto load_tile = [&](int t, u32x4_t* kk, u32x4_t* vv) {
    load_rows(tile_offset(t) + lane_off, kk, vv);
  };

  // Paged splits request their wave's first two tiles now, before the query is prepared.
  if (!packed && wt0 < sr.t1) {
    load_tile(wt0, ka, va);
    load_tile(min(wt0 + NW, sr.t1 - 1), kb, vb);
  }

  // Query operand of head r (lane (qd, r)), pre-scaled by 1/sqrt(D) and split into three
  // bf16 terms, held in registers for the whole split.  Rows past the group are zero.
  u32x4_t qh[NC], qm[NC], ql[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float x[8] = {qraw[2 * c].x, qraw[2 * c].y, qraw[2 * c].z, qraw[2 * c].w,
                  qraw[2 * c + 1].x, qraw[2 * c + 1].y, qraw[2 * c + 1].z, qraw[2 * c + 1].w};
    float h8[8], m8[8], l8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split3(r < p.G ? x[j] * p.scale : 0.f, h8[j], m8[j], l8[j]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      qh[c][w] = pack_hi16(h8[2 * w], h8[2 * w + 1]);
      qm[c][w] = pack_hi16(m8[2 * w], m8[2 * w + 1]);
      ql[c][w] = pack_hi16(l8[2 * w], l8[2 * w + 1]);
    }
  }
  // Selection matrices E_e[k][n] = (k == n + 16 e), lane (qd, r): k = 8qd + j, n = r.
  u32x4_t sel[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int k0 = 8 * qd + 2 * w;
      const uint32_t lo = (k0 == r + 16 * e) ? 0x3f80u : 0u;
      const uint32_t hi = (k0 + 1 == r + 16 * e) ? 0x3f80u : 0u;
      sel[e][w] = lo | (hi << 16);
    }
  }

  f32x4_t O[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) O[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // One tile step: request the wave's next tile t + NW into (kpf, vpf), then consume
  // tile t from (kr, vr).  The two buffers swap roles by unrolling the loop twice, so no
  // register copy ever waits on an outstanding load.
  // The request is unconditional (the last tile is re-read at the end of the run) so the
  // number of loads in flight, and with it the wait before tile t's products, does not
  // depend on a branch.
  auto step = [&](auto prefetch, int t, u32x4_t* kr, u32x4_t* vr, u32x4_t* kpf,
                  u32x4_t* vpf) {
    if constexpr (decltype(prefetch)::value) load_tile(min(t + NW, sr.t1 - 1), kpf, vpf);
    const int pos0 = t * kPage;
    const bool full = pos0 >= sr.row_lo && pos0 + kPage <= sr.row_hi;
    if (!full) {
      const int pr = pos0 + r;
      if (pr < sr.row_lo || pr >= sr.row_hi) {
#pragma unroll
        for (int c = 0; c < NC; ++c) vr[c] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    // Logits: D[m = row][n = head].  Accumulate the small terms first.
    f32x4_t za = {0.f, 0.f, 0.f, 0.f}, zb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) zb = mfma32(kr[c], ql[c], zb);
#pragma unroll
    for (int c = 0; c < NC; ++c) zb = mfma32(kr[c], qm[c], zb);
#pragma unroll
    for (int c = 0; c < NC; ++c) za = mfma32(kr[c], qh[c], za);
    float z[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) z[k] = za[k] + zb[k];
    if (!full) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pr = pos0 + 4 * qd + k;
        if (pr < sr.row_lo || pr >= sr.row_hi) z[k] = -INFINITY;
      }
    }
    if (WRITE_Z && zrow) {
      if (full) {
        *reinterpret_cast<float4*>(zrow + pos0 + 4 * qd) = make_float4(z[0], z[1], z[2], z[3]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pr = pos0 + 4 * qd + k;
          if (pr >= sr.row_lo && pr < sr.row_hi) zrow[pr] = z[k];
        }
      }
    }
    // V^T tiles: lane (qd, r) gets V[row 4qd + k][dim 16 tt + r], k = 0..3.
    u32x2_t vt[NT];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const f32x4_t tr = mfma32(vr[c], sel[e], f32x4_t{0.f, 0.f, 0.f, 0.f});
        vt[2 * c + e] = u32x2_t{pack_hi16(tr[0], tr[1]), pack_hi16(tr[2], tr[3])};
      }
    }
    // Online softmax of head r over this tile.
    float mt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __expf(m_run - m_use);
    float pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = __expf(z[k] - m_use);
    l_run = l_run * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
        for (int k = 0; k < 4; ++k) O[tt][k] *= alpha;
      }
    }
    m_run = m_new;
    // P^T operand, split into hi + lo bf16 terms.
    float pl[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pl[k] = pv[k] - trunc_bf16(pv[k]);
    const u32x2_t ph2 = {pack_hi16(pv[0], pv[1]), pack_hi16(pv[2], pv[3])};
    const u32x2_t pl2 = {pack_hi16(pl[0], pl[1]), pack_hi16(pl[2], pl[3])};
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      O[tt] = mfma16(vt[tt], pl2, O[tt]);
      O[tt] = mfma16(vt[tt], ph2, O[tt]);
    }
  };
  // The first tile's successor is already in flight; every later step requests the
  // wave's tile after next.
  if (wt0 < sr.t1) {
    step(Flag<false>{}, wt0, ka, va, kb, vb);
    for (int t = wt0 + NW; t < sr.t1; t += 2 * NW) {
      step(Flag<true>{}, t, kb, vb, ka, va);
      if (t + NW >= sr.t1) break;
      step(Flag<true>{}, t + NW, ka, va, kb, vb);
    }
  }

  // Merge the four waves of the workgroup: common max, rescaled sums, one partial.
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (qd == 0) {
    sm_m[wave][r] = m_run;
    sm_l[wave][r] = l_tot;
  }
  __syncthreads();
  float M = sm_m[0][r];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][r]);
  const float M_use = (M == -INFINITY) ? 0.f : M;
  const float sc = __expf(m_run - M_use);
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
    for (int k = 0; k < 4; ++k) O[tt][k] *= sc;
  }
  if (wave > 0 && r < p.G) {
    float* so = &sm_o[wave - 1][r][4 * qd];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<float4*>(so + 16 * tt) = make_float4(O[tt][0], O[tt][1], O[tt][2], O[tt][3]);
  }
  __syncthreads();
  if (wave == 0 && r < p.G) {
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) L += sm_l[w][r] * __expf(sm_m[w][r] - M_use);
    if (qd == 0) {
      p.part_m[pidx * p.G + r] = M;
      p.part_l[pidx * p.G + r] = L;
    }
    float* o = p.part_o + (pidx * p.G + r) * D + 4 * qd;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      float4 a = make_float4(O[tt][0], O[tt][1], O[tt][2], O[tt][3]);
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) {
        const float4 c = *reinterpret_cast<const float4*>(&sm_o[w][r][16 * tt + 4 * qd]);
        a.x += c.x;
        a.y += c.y;
        a.z += c.z;
        a.w += c.w;
      }
      *reinterpret_cast<float4*>(o + 16 * tt) = a;
    }
  }
}

template <int D, bool WRITE_Z>
__global__ __launch_bounds__(256) void k_attn_partial_bf16(AttnParams p) {
  __shared__ Bf16Lds<D> lds;
  attn_partial_bf16<D, WRITE_Z>(p, blockIdx.x, lds);
}

// The slow rows and the fast rows of one decode step in one launch: workgroups below the
// slow call's split count run its splits, the others the fast call's.  The slow call's
// workgroups come first: it plans one per CU, and dispatched first onto an idle chip they
// land one per CU as in a launch of their own (behind the fast call's workgroups, which
// exit at once on a slow step, they were measured 35% slower).
template <int D>
__global__ __launch_bounds__(256) void k_attn_partial_bf16_pair(AttnParams pf, AttnParams ps) {
  __shared__ Bf16Lds<D> lds;
  const int ns = ps.n_seqs * ps.Hkv * ps.nsplit;
  if ((int)blockIdx.x < ns)
    attn_partial_bf16<D, true>(ps, blockIdx.x, lds);
  else
    attn_partial_bf16<D, false>(pf, blockIdx.x - ns, lds);
}

// LDS of one fp32 workgroup.
template <int D>
struct F32Lds {
  float qs[kMaxG][D];
  float zt[kMaxG][kPage];
};

// fp32 caches: one wavefront per split, VALU only.
template <int D, bool WRITE_Z>
__device__ __forceinline__ void attn_partial_f32(AttnParams p, int work, F32Lds<D>& lds) {
  constexpr int DD = D / kWave;
  auto& qs = lds.qs;
  auto& zt = lds.zt;
  const int lane = threadIdx.x;
  if (work >= p.n_seqs * p.Hkv * p.nsplit) return;
  const int split = work % p.nsplit;
  const int ig = work / p.nsplit;
  const int g = ig % p.Hkv;
  const int i = ig / p.Hkv;
  const int b = uniform(p.seq_ids[i]);
  if (b < 0) return;  // unused slot of the row list
  if (split == 0 && p.status && threadIdx.x == 0) report_contracts(p, b, g);
  // clamped: a length past the call's bound cannot send an index out of the buffers
  const int N = min(max(uniform(p.seq_lens[b]), 0), p.max_len);
  const size_t pidx = (size_t)ig * p.nsplit + split;
  const SplitRange sr = split_range(p, b, g, split, N);
  if (sr.t0 >= sr.t1) {
    write_empty_partial(p, pidx, D, lane);
    return;
  }
  const int G = p.G;
  for (int k = lane; k < G * D; k += kWave) {
    const int h = k / D, d = k % D;
    qs[h][d] = p.q[((size_t)b * p.Hq + (size_t)g * G + h) * D + d] * p.scale;
  }
  __syncthreads();

  const float* kbase;
  const float* vbase;
  if (sr.packed) {
    const size_t off = ((size_t)b * p.Hkv + g) * (size_t)p.packed_cap * D;
    kbase = reinterpret_cast<const float*>(p.packed_k) + off;
    vbase = reinterpret_cast<const float*>(p.packed_v) + off;
  } else {
    kbase = reinterpret_cast<const float*>(p.k_cache);
    vbase = reinterpret_cast<const float*>(p.v_cache);
  }
  const int32_t* bt = p.block_table + (size_t)b * p.max_pages;

  float m_run[kMaxG], l_run[kMaxG], acc[kMaxG][DD];
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) acc[h][dd] = 0.f;
  }
  const int r = lane & 15, hq = lane >> 4;
  for (int t = sr.t0; t < sr.t1; ++t) {
    size_t toff;
    if (sr.packed) {
      toff = (size_t)t * kPage * D;
    } else {
      const int page = uniform(bt[t]);
      toff = ((size_t)page * p.Hkv + g) * (size_t)(kPage * D);
    }
    const int pos0 = t * kPage;
    for (int hb = 0; hb < G; hb += 4) {
      const int h = hb + hq;
      if (h < G) {
        const int pr = pos0 + r;
        float z = -INFINITY;
        if (pr >= sr.row_lo && pr < sr.row_hi) {
          const float* krow = kbase + toff + (size_t)r * D;
          float a = 0.f;
          for (int d = 0; d < D; ++d) a = fmaf(krow[d], qs[h][d], a);
          z = a;
          if (WRITE_Z && p.logits)
            p.logits[((size_t)b * p.Hq + (size_t)g * G + h) * p.logits_stride + pr] = z;
        }
        zt[h][r] = z;
      }
    }
    __syncthreads();
    float v[kPage][DD];
#pragma unroll
    for (int rr = 0; rr < kPage; ++rr) {
      const int pr = pos0 + rr;
      const bool ok = pr >= sr.row_lo && pr < sr.row_hi;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd)
        v[rr][dd] = ok ? vbase[toff + (size_t)rr * D + lane + kWave * dd] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
      if (h < G) {
        float mt = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < kPage; ++rr) mt = fmaxf(mt, zt[h][rr]);
        const float m_new = fmaxf(m_run[h], mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = expf(m_run[h] - m_use);
        float ls = 0.f;
#pragma unroll
        for (int dd = 0; dd < DD; ++dd) acc[h][dd] *= alpha;
#pragma unroll
        for (int rr = 0; rr < kPage; ++rr) {
          const float pr = expf(zt[h][rr] - m_use);
          ls += pr;
#pragma unroll
          for (int dd = 0; dd < DD; ++dd) acc[h][dd] = fmaf(pr, v[rr][dd], acc[h][dd]);
        }
        l_run[h] = l_run[h] * alpha + ls;
        m_run[h] = m_new;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < kMaxG; ++h) {
    if (h < G) {
      if (lane == 0) {
        p.part_m[pidx * G + h] = m_run[h];
        p.part_l[pidx * G + h] = l_run[h];
      }
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) p.part_o[(pidx * G + h) * D + lane + kWave * dd] = acc[h][dd];
    }
  }
}

template <int D, bool WRITE_Z>
__global__ __launch_bounds__(64) void k_attn_partial_f32(AttnParams p) {
  __shared__ F32Lds<D> lds;
  attn_partial_f32<D, WRITE_Z>(p, blockIdx.x, lds);
}

template <int D>
__global__ __launch_bounds__(64) void k_attn_partial_f32_pair(AttnParams pf, AttnParams ps) {
  __shared__ F32Lds<D> lds;
  const int ns = ps.n_seqs * ps.Hkv * ps.nsplit;
  if ((int)blockIdx.x < ns)
    attn_partial_f32<D, true>(ps, blockIdx.x, lds);
  else
    attn_partial_f32<D, false>(pf, blockIdx.x - ns, lds);
}

struct MergeArgs {
  const float* pm;
  const float* pl;
  const float* po;
  int nsplit, Hq, Hkv, G, D, win;
  const int32_t* seq_ids;
  float* out;
  float* lse;
};

MergeArgs merge_args(const AttnParams& p, int D, float* out, float* lse) {
  return MergeArgs{p.part_m, p.part_l, p.part_o, p.nsplit, p.Hq, p.Hkv, p.G, D, p.win,
                   p.seq_ids, out, lse};
}

struct MergeLds {
  float gm[64], gl[64];
  float4 acc4[256];
};

// One block per (listed row, query head): log-sum-exp merge of the split partials.
__device__ __forceinline__ void attn_merge(MergeArgs a, int blk, MergeLds& lds) {
  const float* __restrict__ pm = a.pm;
  const float* __restrict__ pl = a.pl;
  const float* __restrict__ po = a.po;
  const int nsplit = a.nsplit, Hq = a.Hq, Hkv = a.Hkv, G = a.G, D = a.D, win = a.win;
  const int32_t* __restrict__ seq_ids = a.seq_ids;
  float* __restrict__ out = a.out;
  float* __restrict__ lse = a.lse;
  auto& gm = lds.gm;
  auto& gl = lds.gl;
  auto& acc4 = lds.acc4;
  // Thread (grp, col) folds splits grp, grp + ngrp, ... of column block col into a running
  // (max, sum, weighted o); the loads of kUnroll splits are issued together.  The groups
  // are then combined in LDS.
  //
  // With a query window (win > 1) the G rows of a KV head are win slots of G / win heads;
  // lse is written for every row, the output only for slot 0 (the current query), into
  // the [batch][Hq / win][D] layout of the model's own heads.
  constexpr int kUnroll = 8;
  const int tid = threadIdx.x;
  const int i = blk / Hq;
  const int h = blk % Hq;
  const int g = h / G, hh = h % G;
  const int b = seq_ids[i];
  if (b < 0) return;  // unused slot of the row list (block-uniform)
  const size_t base = ((size_t)i * Hkv + g) * nsplit;
  const int cols = D / 4;
  const int ngrp = 256 / cols;
  const int col = tid % cols, grp = tid / cols;
  const float4* po4 = reinterpret_cast<const float4*>(po);
  float mt = -INFINITY, lt = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = grp; s0 < nsplit; s0 += kUnroll * ngrp) {
    float m[kUnroll], l[kUnroll];
    float4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int s = s0 + k * ngrp;
      const size_t u = (base + min(s, nsplit - 1)) * G + hh;
      m[k] = s < nsplit ? pm[u] : -INFINITY;
      l[k] = pl[u];
      v[k] = po4[u * cols + col];
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      if (m[k] == -INFINITY) continue;  // empty split (or past the end): weight 0
      const float mn = fmaxf(mt, m[k]);
      const float co = __expf(mt - mn);  // 0 while mt is -inf
      const float cn = __expf(m[k] - mn);
      lt = lt * co + l[k] * cn;
      acc.x = acc.x * co + v[k].x * cn;
      acc.y = acc.y * co + v[k].y * cn;
      acc.z = acc.z * co + v[k].z * cn;
      acc.w = acc.w * co + v[k].w * cn;
      mt = mn;
    }
  }
  if (col == 0) {
    gm[grp] = mt;
    gl[grp] = lt;
  }
  acc4[tid] = acc;
  __syncthreads();
  if (grp == 0) {
    float M = -INFINITY;
    for (int q = 0; q < ngrp; ++q) M = fmaxf(M, gm[q]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Lt = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q = 0; q < ngrp; ++q) {
      if (gm[q] == -INFINITY) continue;
      const float w = __expf(gm[q] - Mu);
      const float4 x = acc4[q * cols + col];
      Lt += w * gl[q];
      o.x += w * x.x;
      o.y += w * x.y;
      o.z += w * x.z;
      o.w += w * x.w;
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    const int G0 = G / win;
    if (hh < G0)
      reinterpret_cast<float4*>(out + ((size_t)b * (Hq / win) + g * G0 + hh) * D)[col] =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (col == 0 && lse) lse[(size_t)b * Hq + h] = Lt > 0.f ? Mu + logf(Lt) : -INFINITY;
  }
}

__global__ __launch_bounds__(256) void k_attn_merge(MergeArgs a) {
  __shared__ MergeLds lds;
  attn_merge(a, blockIdx.x, lds);
}

// Merge blocks of the slow call, then of the fast call.
__global__ __launch_bounds__(256) void k_attn_merge_pair(MergeArgs af, MergeArgs as, int ns) {
  __shared__ MergeLds lds;
  if ((int)blockIdx.x < ns)
    attn_merge(as, blockIdx.x, lds);
  else
    attn_merge(af, blockIdx.x - ns, lds);
}

template <int D>
hipError_t launch_partial(const AttnParams& p, int dtype, hipStream_t stream) {
  const int works = p.n_seqs * p.Hkv * p.nsplit;
  const bool wz = p.logits != nullptr;
  if (dtype == SFI_BF16) {
    // one workgroup (four wavefronts) per split
    if (wz)
      hipLaunchKernelGGL((k_attn_partial_bf16<D, true>), dim3(works), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((k_attn_partial_bf16<D, false>), dim3(works), dim3(256), 0, stream, p);
  } else {
    if (wz)
      hipLaunchKernelGGL((k_attn_partial_f32<D, true>), dim3(works), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((k_attn_partial_f32<D, false>), dim3(works), dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

// Tiles per split for about `target` workgroups per call.  Fast calls aim at two workgroups per CU (256 CUs), which fills the chip in
// one wave of workgroups.  Slow calls aim at one per CU: the dense pass stays HBM-bound
// (the same duration as with two), and half of every CU stays free for the Selector and
// pack of the previous layer, which run at the same time on another stream.
// Small calls are latency-bound, so the floor is low: one tile per wavefront (four per
// bf16 workgroup) or two tiles for the one-wavefront fp32 workgroup, and the many short
// splits start at once.
constexpr long kFastTargetSplits = 512;
constexpr long kSlowTargetSplits = 256;
constexpr int kMaxTps = kMaxTilesPerSplit;

static int tiles_per_split(const sfi_shape& s, long total, long target) {
  const int min_tps = s.dtype == SFI_BF16 ? 4 : 2;
  long tps = (total + target - 1) / target;
  return (int)(tps < min_tps ? min_tps : (tps > kMaxTps ? kMaxTps : tps));
}

SplitPlan plan_slow(const sfi_shape& s, int n_seqs, int max_seq_len) {
  SplitPlan sp;
  const int ntile = (max_seq_len + kPage - 1) / kPage;
  const int tps = tiles_per_split(s, (long)n_seqs * s.num_kv_heads * ntile, kSlowTargetSplits);
  sp.tps = tps;
  sp.nsplit = (ntile + tps - 1) / tps;
  sp.nsplit_a = 0;
  return sp;
}

// A paged split stages its page table in LDS before its first K/V request, so it starts
// later than a packed split, whose first requests go out at once: it gets half the tiles,
// and the packed splits share the rest of the workgroup target.
SplitPlan plan_fast(const sfi_shape& s, int n_seqs, int packed_cap, int max_recent) {
  SplitPlan sp;
  const int ta = packed_cap / kPage;
  const int tb = (max_recent + kPage - 1) / kPage + 1;  // +1: the window need not start on a page
  const long units = (long)n_seqs * s.num_kv_heads;
  const int tps0 = tiles_per_split(s, units * (ta + tb), kFastTargetSplits);
  const int min_tps = s.dtype == SFI_BF16 ? 4 : 2;
  const int tps_b = (tps0 + 1) / 2 < min_tps ? min_tps : (tps0 + 1) / 2;
  const int nsb = (tb + tps_b - 1) / tps_b;
  long per_unit = units > 0 ? kFastTargetSplits / units : kFastTargetSplits;
  if (per_unit < 1) per_unit = 1;
  const long rem = per_unit - nsb > 1 ? per_unit - nsb : 1;
  long tps_a = (ta + rem - 1) / rem;
  if (tps_a < tps0) tps_a = tps0;
  if (tps_a > kMaxTps) tps_a = kMaxTps;
  sp.tps = (int)tps_a;
  sp.tps_b = tps_b;
  sp.nsplit_a = (ta + sp.tps - 1) / sp.tps;
  sp.nsplit = sp.nsplit_a + nsb;
  return sp;
}

size_t partial_bytes(const sfi_shape& s, int n_seqs, int nsplit) {
  const size_t G = (size_t)(s.num_q_heads / s.num_kv_heads);
  const size_t units = (size_t)n_seqs * s.num_kv_heads * nsplit * G;
  const size_t ml = ((units * sizeof(float) + 255) / 256) * 256;
  return 2 * ml + units * s.head_dim * sizeof(float);
}

hipError_t launch_attention(const AttnParams& p0, int head_dim, int dtype, float* out,
                            float* lse, hipStream_t stream) {
  AttnParams p = p0;
  hipError_t e = head_dim == 64 ? launch_partial<64>(p, dtype, stream)
                                : launch_partial<128>(p, dtype, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_merge, dim3(p.n_seqs * p.Hq), dim3(256), 0, stream,
                     merge_args(p, head_dim, out, lse));
  return hipGetLastError();
}

hipError_t launch_attention_pair(const AttnParams& pf, const AttnParams& ps, int head_dim,
                                 int dtype, float* out, float* lse_slow, hipStream_t stream) {
  const int works = pf.n_seqs * pf.Hkv * pf.nsplit + ps.n_seqs * ps.Hkv * ps.nsplit;
  if (dtype == SFI_BF16) {
    if (head_dim == 64)
      hipLaunchKernelGGL(k_attn_partial_bf16_pair<64>, dim3(works), dim3(256), 0, stream, pf, ps);
    else
      hipLaunchKernelGGL(k_attn_partial_bf16_pair<128>, dim3(works), dim3(256), 0, stream, pf,
                         ps);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL(k_attn_partial_f32_pair<64>, dim3(works), dim3(64), 0, stream, pf, ps);
    else
      hipLaunchKernelGGL(k_attn_partial_f32_pair<128>, dim3(works), dim3(64), 0, stream, pf, ps);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ns = ps.n_seqs * ps.Hq;
  hipLaunchKernelGGL(k_attn_merge_pair, dim3(pf.n_seqs * pf.Hq + ns), dim3(256), 0, stream,
                     merge_args(pf, head_dim, out, nullptr),
                     merge_args(ps, head_dim, out, lse_slow), ns);
  return hipGetLastError();
}

}  // namespace sfi
