// Compaction of the fast-step memory: sink rows and Selector-chosen rows are copied from
// the paged cache into one contiguous buffer per (row b, KV head g), so fast steps read
// them sequentially instead of gathering scattered pages (zh "2.3 系统级优化",
// nl "Systeemontwerp en Kernel-optimalisatie", fr "2.C Optimisations Système").
//
// Each wavefront moves a run of consecutive packed rows.  The lanes first look up one row
// each (selected position, then its page), then every load instruction covers whole rows
// with consecutive lanes on consecutive 16-byte words: LPR = row bytes / 16 lanes per row,
// 64 / LPR rows per instruction, eight instructions per wavefront for K and eight for V,
// all issued before any store.  Packed row i holds position packed_pos[i] = i for
// i < n_sink and sel_idx[i - n_sink] after; rows without a position are zero-filled.
#include "sfi_device.h"
#include "sfi_internal.h"

namespace sfi {

namespace {

struct PackArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  const int32_t* sel;
  const int32_t* seq_ids;
  uint8_t* pk;
  uint8_t* pv;
  int32_t* ppos;
  int32_t* plen;
  int Hkv, max_pages, K, n_sink, cap, row_bytes;
  int n_work;  // row blocks in all
};

__device__ __forceinline__ int packed_source(const PackArgs& a, const int32_t* selrow, int row) {
  if (row < a.n_sink) return row;
  const int k = row - a.n_sink;
  return k < a.K ? selrow[k] : -1;
}

constexpr int kPackInstr = 8;   // load instructions per wavefront and tensor
constexpr int kPackWaves = 4;   // wavefronts per block
// At most this many blocks (one per CU), each looping over row blocks: the copy keeps the
// HBM busy while leaving room on every CU for the attention that runs at the same time.
constexpr int kPackMaxBlocks = 256;

template <int LPR>
__global__ __launch_bounds__(64 * kPackWaves) void k_pack(PackArgs a) {
  constexpr int RPI = 64 / LPR;          // rows per load instruction
  constexpr int RW = kPackInstr * RPI;   // rows per wavefront
  constexpr int RB = kPackWaves * RW;    // rows per block
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = (a.cap + RB - 1) / RB;
  // Grid-stride over the row blocks: the grid is capped (see launch_pack).
  for (int work = blockIdx.x; work < a.n_work; work += gridDim.x) {
    const int blk = work % nblk;
    const int ig = work / nblk;
    const int g = ig % a.Hkv, i = ig / a.Hkv;
    const int b = a.seq_ids[i];
    if (b < 0) continue;  // unused slot of the row list (wavefront-uniform)
    const size_t bg = (size_t)b * a.Hkv + g;
    const int32_t* selrow = a.sel + bg * a.K;
    const int row0 = blk * RB + wv * RW;
    if (row0 >= a.cap) continue;  // wavefront-uniform; the kernel has no block barrier
    // Lane r < RW resolves row row0 + r: its position and page.
    const int my_row = row0 + lane;
    const bool own = lane < RW && my_row < a.cap;
    const int pos = own ? packed_source(a, selrow, my_row) : -1;
    const int page = pos >= 0 ? a.bt[(size_t)b * a.max_pages + pos / kPage] : 0;
    if (own) {
      a.ppos[bg * a.cap + my_row] = pos;
      // Valid rows form a prefix: the last valid row (or row 0 when none is valid) records
      // the packed length.
      const int next = my_row + 1 < a.cap ? packed_source(a, selrow, my_row + 1) : -1;
      if (pos >= 0 && next < 0) a.plen[bg] = my_row + 1;
      if (my_row == 0 && pos < 0) a.plen[bg] = 0;
    }
    const int sub = lane % LPR, rsub = lane / LPR;
    const size_t rb = (size_t)a.row_bytes;
    u32x4_t kv[kPackInstr], vv[kPackInstr];
    bool valid[kPackInstr];
#pragma unroll
    for (int j = 0; j < kPackInstr; ++j) {
      const int r = j * RPI + rsub;
      const int pr = __shfl(pos, r), pg = __shfl(page, r);
      valid[j] = pr >= 0;
      // Rows without a position read row 0 of page 0 (always present) and store zeros.
      const size_t src = valid[j] ? (((size_t)pg * a.Hkv + g) * kPage + pr % kPage) * rb : 0;
      kv[j] = *reinterpret_cast<const u32x4_t*>(a.kc + src + 16 * sub);
      vv[j] = *reinterpret_cast<const u32x4_t*>(a.vc + src + 16 * sub);
    }
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kPackInstr; ++j) {
      const int row = row0 + j * RPI + rsub;
      if (row < a.cap) {
        const size_t dst = (bg * a.cap + row) * rb + 16 * sub;
        *reinterpret_cast<u32x4_t*>(a.pk + dst) = valid[j] ? kv[j] : zero;
        *reinterpret_cast<u32x4_t*>(a.pv + dst) = valid[j] ? vv[j] : zero;
      }
    }
  }
}

// ----------------------------------------------------------------- incremental update
// The fast step's softmax does not depend on the order of the packed rows, so the packed
// buffer can be kept as a set: an update keeps every row whose position stays selected in
// its slot and copies only the newly selected rows, into the slots of the dropped ones (and,
// as K_eff grows with N, past the old end).  slot_map[b][g][j] holds the slot of position j
// (or -1), so membership is one load.
//
// Each (listed row, KV head) "ig" has two lists: its selection (K entries) and its slots
// (n_sink + K).  Both are cut into chunks of kChunk entries, one workgroup per chunk, so the
// scattered map accesses of one ig spread over many CUs.  The map (one word per position,
// megabytes per layer) is read at scattered places once per update, by kernel 1, and
// written only where a row changes hands; the other kernels read two small per-ig lists
// in the workspace instead: the old slot of each selection entry, and for each slot the
// index of the selection entry that claimed it.  Four kernels, each needing the previous
// one complete:
//   1. mark     sel chunks record each entry's old slot (map value, -1 if not held), claim
//               that slot with the entry's index, and count the entries not held and the
//               valid ones per chunk;
//   2. count    slot chunks find the held rows whose position is no longer selected: a
//               slot is kept when its claim names a selection entry holding its position
//               (a claim left over from an earlier update passes that test only if its
//               position is selected again, so the claims need no clearing); dropped
//               positions leave the map, and each chunk counts its free slots;
//   3. free     slot chunks write their free slots at (earlier chunks' count + in-chunk
//               prefix), so the free list is in slot order;
//   4. assign   sel chunks give the j-th new position the j-th free slot (past the old end
//               once the freed slots are used up), record it, and copy its K/V rows.
// Kernel 4 publishes the new packed length from one chunk while the other chunks of the
// same ig may not have started, so no chunk of it reads packed_len: kernel 3 keeps a copy
// of the old length for it.
// Chunk prefixes are sums over at most a few dozen per-chunk counts, so every assignment is
// deterministic.  An empty buffer (packed_len 0) or a selection smaller than the rows held
// is rebuilt in sfi_pack's order by kernels 3 and 4.

constexpr int kChunk = 1024;           // list entries per workgroup
constexpr int kChunkThreads = 256;     // four consecutive entries per thread

struct UpdArgs {
  const int32_t* sel;
  const int32_t* seq_ids;
  const uint8_t* kc;
  const uint8_t* vc;
  const int32_t* bt;
  uint8_t* pk;
  uint8_t* pv;
  int32_t* ppos;
  int32_t* plen;
  int32_t* map;
  int64_t map_stride;  // >= every N and >= n_sink
  int32_t* cnt_free;   // [n_ig][nc_slot]
  int32_t* cnt_add;    // [n_ig][nc_sel]
  int32_t* cnt_valid;  // [n_ig][nc_sel]
  int32_t* free_slot;  // [n_ig][K]
  int32_t* plen_old;   // [n_ig] held length before this update (written by kernel 3)
  int32_t* old_slot;   // [n_ig][K]: slot of each selection entry before the update, or -1
  int32_t* claim;      // [n_ig][nc_slot * kChunk]: index of the selection entry holding the
                       // slot's position (valid only where it says so, see is_kept)
  uint32_t* status;    // device contract flags, may be null
  int Hkv, K, n_sink, cap, nc_sel, nc_slot, max_pages, row_bytes;
};

struct Ig {
  int ig, chunk, b, g;
  size_t bg;
};

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();  // red may still be read by an earlier call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < kChunkThreads / 64; ++w) t += red[w];
  return t;
}

// Workgroup x of a grid of n_ig * nc chunks; b < 0 for an unused slot of the row list.
__device__ __forceinline__ Ig ig_of(const UpdArgs& a, int x, int nc) {
  Ig r;
  r.ig = x / nc;
  r.chunk = x % nc;
  r.g = r.ig % a.Hkv;
  r.b = a.seq_ids[r.ig / a.Hkv];
  r.bg = (size_t)(r.b < 0 ? 0 : r.b) * a.Hkv + r.g;
  return r;
}

// The held length as these kernels maintain it (clamped, so that a corrupted value cannot
// send the loops out of the lists).
__device__ __forceinline__ int held_len(const UpdArgs& a, size_t bg) {
  return min(max(a.plen[bg], 0), a.n_sink + a.K);
}

__device__ __forceinline__ bool in_map(const UpdArgs& a, int p) {
  return p >= 0 && p < a.map_stride;
}

// Slots of one ig's claim list.
__device__ __forceinline__ int claim_len(const UpdArgs& a) { return a.nc_slot * kChunk; }

// Whether held slot sl, holding position q, keeps its row: q is in the map and the slot's
// claim names a selection entry equal to q.  Kernel 1 claimed sl for the entry holding q if
// there is one; a claim from an earlier update that still names an entry equal to q is
// equally right, and any other value fails the test.
__device__ __forceinline__ bool is_kept(const UpdArgs& a, const Ig& r, int sl, int q) {
  if (!in_map(a, q)) return false;
  const int c = a.claim[(size_t)r.ig * claim_len(a) + sl];
  return c >= 0 && c < a.K && a.sel[r.bg * a.K + c] == q;
}

// Kernel 1: mark (sel chunks).
__global__ __launch_bounds__(kChunkThreads) void k_upd_mark(UpdArgs a) {
  __shared__ uint32_t red[kChunkThreads / 64];
  const Ig r = ig_of(a, blockIdx.x, a.nc_sel);
  if (r.b < 0) return;
  const int32_t* sel = a.sel + r.bg * a.K;
  const int32_t* map = a.map + r.bg * a.map_stride;
  int32_t* old_slot = a.old_slot + (size_t)r.ig * a.K;
  int32_t* claim = a.claim + (size_t)r.ig * claim_len(a);
  const int k0 = r.chunk * kChunk + 4 * (int)threadIdx.x;
  int q[4], v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = k0 + i < a.K ? sel[k0 + i] : -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = in_map(a, q[i]) ? map[q[i]] : -1;
  uint32_t c_add = 0, c_valid = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (k0 + i < a.K) old_slot[k0 + i] = v[i] >= 0 ? v[i] : -1;
    if (v[i] >= 0 && v[i] < claim_len(a)) claim[v[i]] = k0 + i;
    c_add += (q[i] >= 0 && v[i] < 0) ? 1u : 0u;  // selected, not held
    c_valid += q[i] >= 0 ? 1u : 0u;              // valid entry
  }
  const uint32_t t1 = block_sum_u32(c_add, red), t2 = block_sum_u32(c_valid, red);
  if (threadIdx.x == 0) {
    a.cnt_add[(size_t)r.ig * a.nc_sel + r.chunk] = (int32_t)t1;
    a.cnt_valid[(size_t)r.ig * a.nc_sel + r.chunk] = (int32_t)t2;
  }
}

// Kernel 2: count (slot chunks).
__global__ __launch_bounds__(kChunkThreads) void k_upd_count(UpdArgs a) {
  __shared__ uint32_t red[kChunkThreads / 64];
  const Ig r = ig_of(a, blockIdx.x, a.nc_slot);
  if (r.b < 0) return;
  int32_t* map = a.map + r.bg * a.map_stride;
  const int k0 = r.chunk * kChunk + 4 * (int)threadIdx.x;
  const int plen = held_len(a, r.bg);
  const int32_t* ppos = a.ppos + r.bg * a.cap;
  int q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sl = k0 + i;
    q[i] = (sl >= a.n_sink && sl < plen) ? ppos[sl] : -2;
  }
  uint32_t c_free = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (q[i] == -2) continue;
    if (!is_kept(a, r, k0 + i, q[i])) {
      if (in_map(a, q[i])) map[q[i]] = -1;
      ++c_free;
    }
  }
  const uint32_t t = block_sum_u32(c_free, red);
  if (threadIdx.x == 0) a.cnt_free[(size_t)r.ig * a.nc_slot + r.chunk] = (int32_t)t;
}

// Sums of one ig's chunk counts: before chunk `upto` and in all.
struct Pref {
  int before, total;
};
__device__ __forceinline__ Pref chunk_prefix(const int32_t* cnt, int nc, int upto) {
  Pref p{0, 0};
  for (int c = 0; c < nc; ++c) {
    const int v = cnt[c];
    p.before += c < upto ? v : 0;
    p.total += v;
  }
  return p;
}

__device__ __forceinline__ bool rebuild_of(int plen_old, int n_sink, int keff) {
  const int nsel_old = plen_old > n_sink ? plen_old - n_sink : 0;
  return plen_old == 0 || keff < nsel_old;
}

// Kernel 3: the free list (slot chunks).  For a rebuilt ig: drop every listed position
// from the map and clear the slots past the new length.
__global__ __launch_bounds__(kChunkThreads) void k_upd_free(UpdArgs a) {
  __shared__ uint32_t wsum[kChunkThreads / 64 + 1];
  __shared__ int sh[3];
  const Ig r = ig_of(a, blockIdx.x, a.nc_slot);
  if (r.b < 0) return;
  if (threadIdx.x == 0) {
    const Pref f = chunk_prefix(a.cnt_free + (size_t)r.ig * a.nc_slot, a.nc_slot, r.chunk);
    const Pref v = chunk_prefix(a.cnt_valid + (size_t)r.ig * a.nc_sel, a.nc_sel, 0);
    sh[0] = f.before;
    sh[1] = v.total;  // K_eff
    sh[2] = held_len(a, r.bg);
    if (r.chunk == 0) a.plen_old[r.ig] = sh[2];
  }
  __syncthreads();
  const int keff = sh[1], plen = sh[2];
  int32_t* ppos = a.ppos + r.bg * a.cap;
  int32_t* map = a.map + r.bg * a.map_stride;
  const int k0 = r.chunk * kChunk + 4 * (int)threadIdx.x;
  int q[4];
  if (rebuild_of(plen, a.n_sink, keff)) {
    const int n = a.n_sink + keff;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (k0 + i >= a.n_sink && k0 + i < a.cap) ? ppos[k0 + i] : -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (in_map(a, q[i])) map[q[i]] = -1;
      if (k0 + i >= n && k0 + i < a.cap) ppos[k0 + i] = -1;
    }
    return;
  }
  // free slots of this chunk: the held rows that kernel 2 found not kept
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sl = k0 + i;
    q[i] = (sl >= a.n_sink && sl < plen) ? ppos[sl] : -2;
  }
  uint32_t fmask = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (q[i] == -2) continue;
    if (!is_kept(a, r, k0 + i, q[i])) fmask |= 1u << i;
  }
  uint32_t tot;
  uint32_t j = (uint32_t)sh[0] +
               block_exscan<kChunkThreads>(__builtin_popcount(fmask), wsum, &tot);
  int32_t* fslot = a.free_slot + (size_t)r.ig * a.K;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (fmask & (1u << i)) fslot[j++] = k0 + i;
}

// Kernel 4: assign and copy (sel chunks).  LPR lanes copy one row (16 bytes each).
template <int LPR>
__global__ __launch_bounds__(kChunkThreads) void k_upd_assign(UpdArgs a) {
  __shared__ uint32_t wsum[kChunkThreads / 64 + 1];
  __shared__ int sh[5];
  __shared__ int l_pos[kChunk];
  __shared__ int l_slot[kChunk];
  __shared__ int l_page[kChunk];
  const Ig r = ig_of(a, blockIdx.x, a.nc_sel);
  if (r.b < 0) return;
  if (threadIdx.x == 0) {
    const Pref ad = chunk_prefix(a.cnt_add + (size_t)r.ig * a.nc_sel, a.nc_sel, r.chunk);
    const Pref fr = chunk_prefix(a.cnt_free + (size_t)r.ig * a.nc_slot, a.nc_slot, a.nc_slot);
    const Pref v = chunk_prefix(a.cnt_valid + (size_t)r.ig * a.nc_sel, a.nc_sel, 0);
    sh[0] = ad.before;
    sh[1] = ad.total;
    sh[2] = fr.total;
    sh[3] = v.total;  // K_eff
    sh[4] = a.plen_old[r.ig];  // not packed_len: chunk 0 of this kernel overwrites it
  }
  __syncthreads();
  const int keff = sh[3], plen = sh[4];
  const bool rebuild = rebuild_of(plen, a.n_sink, keff);
  const int32_t* sel = a.sel + r.bg * a.K;
  int32_t* ppos = a.ppos + r.bg * a.cap;
  int32_t* map = a.map + r.bg * a.map_stride;
  const int k0 = r.chunk * kChunk + 4 * (int)threadIdx.x;
  int q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = k0 + i < keff ? sel[k0 + i] : -1;
  uint32_t amask = 0;
  if (rebuild) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (q[i] >= 0) amask |= 1u << i;
  } else {
    const int32_t* old_slot = a.old_slot + (size_t)r.ig * a.K;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (q[i] >= 0 && old_slot[k0 + i] < 0) amask |= 1u << i;
  }
  uint32_t tot;
  const uint32_t first = block_exscan<kChunkThreads>(__builtin_popcount(amask), wsum, &tot);
  uint32_t j = (uint32_t)sh[0] + first;  // rank among the ig's new positions
  uint32_t li = first;                   // rank within this chunk
  const int32_t* fslot = a.free_slot + (size_t)r.ig * a.K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (amask & (1u << i)) {
      int slot;
      if (rebuild)
        slot = a.n_sink + k0 + i;  // the full pack's order
      else
        slot = j < (uint32_t)sh[2] ? fslot[j] : plen + (int)(j - (uint32_t)sh[2]);
      ++j;
      // The counts make every slot < n_sink + K_eff <= cap; a slot outside the buffer can
      // only come from state these calls did not maintain: it is dropped (position -1 in
      // the copy list) rather than written, and reported in the status word.
      const bool in_buf = slot >= a.n_sink && slot < a.cap;
      if (!in_buf && a.status) atomicOr(a.status, (uint32_t)SFI_DEV_PACK_SLOT);
      if (in_buf) {
        ppos[slot] = q[i];
        if (in_map(a, q[i])) map[q[i]] = slot;
      }
      l_pos[li] = in_buf ? q[i] : -1;
      l_slot[li] = slot;
      ++li;
    }
  }
  if (threadIdx.x == 0 && r.chunk == 0) a.plen[r.bg] = a.n_sink + keff;
  __syncthreads();
  // physical page of every listed row, staged once: the copy loop below then issues its
  // row loads without waiting for a block-table load first
  const int32_t* btb = a.bt + (size_t)r.b * a.max_pages;
  for (int e = threadIdx.x; e < (int)tot; e += kChunkThreads)
    l_page[e] = l_pos[e] >= 0 ? btb[l_pos[e] / kPage] : 0;
  __syncthreads();
  // copy the rows listed in LDS (and, for a rebuild, the sink rows in chunk 0): LPR lanes
  // per row, 16 bytes per lane
  constexpr int RPB = kChunkThreads / LPR;
  const int sub = threadIdx.x % LPR, rsub = threadIdx.x / LPR;
  const size_t rb = (size_t)a.row_bytes;
  const int n_sink_copy = (rebuild && r.chunk == 0) ? a.n_sink : 0;
  const int nl = (int)tot + n_sink_copy;
  // kCopyBatch rows per lane group are loaded before any of them is stored (a rebuild
  // copies a whole chunk)
  constexpr int kCopyBatch = 8;
  for (int e0 = rsub; e0 < nl; e0 += kCopyBatch * RPB) {
    u32x4_t kv[kCopyBatch], vv[kCopyBatch];
    size_t dst[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      const int e = e0 + u * RPB;
      dst[u] = ~(size_t)0;
      if (e < nl && (e >= (int)tot || l_pos[e] >= 0)) {
        const bool sink = e >= (int)tot;
        const int pos = sink ? e - (int)tot : l_pos[e];
        const int slot = sink ? pos : l_slot[e];
        if (sink && sub == 0) {
          ppos[pos] = pos;
          if (in_map(a, pos)) map[pos] = pos;
        }
        const int page = sink ? btb[pos / kPage] : l_page[e];
        const size_t src =
            (((size_t)page * a.Hkv + r.g) * kPage + pos % kPage) * rb + 16 * sub;
        dst[u] = (r.bg * a.cap + slot) * rb + 16 * sub;
        kv[u] = *reinterpret_cast<const u32x4_t*>(a.kc + src);
        vv[u] = *reinterpret_cast<const u32x4_t*>(a.vc + src);
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      if (dst[u] != ~(size_t)0) {
        *reinterpret_cast<u32x4_t*>(a.pk + dst[u]) = kv[u];
        *reinterpret_cast<u32x4_t*>(a.pv + dst[u]) = vv[u];
      }
    }
  }
}

}  // namespace

static int ceil_div(int x, int y) { return (x + y - 1) / y; }

size_t pack_update_ws(const sfi_shape& s, const sfi_select_params& prm, int n_seqs) {
  const size_t n_ig = (size_t)n_seqs * s.num_kv_heads;
  const size_t nc_sel = ceil_div(prm.top_k, kChunk);
  const size_t nc_slot = ceil_div(prm.n_sink + prm.top_k + 15, kChunk);  // >= packed_cap
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  return r256(n_ig * nc_slot * 4) + 2 * r256(n_ig * nc_sel * 4) +
         2 * r256(n_ig * (size_t)prm.top_k * 4) + r256(n_ig * 4) +
         r256(n_ig * nc_slot * kChunk * 4);
}

hipError_t launch_pack_update(const sfi_shape& s, const sfi_select_params& prm,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* sel_idx,
                              const int32_t* seq_ids, int n_seqs, void* packed_k, void* packed_v,
                              int32_t* packed_pos, int32_t* packed_len, int packed_cap,
                              int32_t* slot_map, int64_t map_stride, uint32_t* status, void* ws,
                              hipStream_t stream) {
  const int n_ig = n_seqs * s.num_kv_heads;
  UpdArgs a;
  a.nc_sel = ceil_div(prm.top_k, kChunk);
  a.nc_slot = ceil_div(packed_cap, kChunk);
  auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = reinterpret_cast<char*>(ws);
  a.cnt_free = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)n_ig * a.nc_slot * 4);
  a.cnt_add = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)n_ig * a.nc_sel * 4);
  a.cnt_valid = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)n_ig * a.nc_sel * 4);
  a.free_slot = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)n_ig * prm.top_k * 4);
  a.plen_old = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)n_ig * 4);
  a.old_slot = reinterpret_cast<int32_t*>(w);
  w += r256((size_t)n_ig * prm.top_k * 4);
  a.claim = reinterpret_cast<int32_t*>(w);
  a.sel = sel_idx;
  a.seq_ids = seq_ids;
  a.kc = reinterpret_cast<const uint8_t*>(k_cache);
  a.vc = reinterpret_cast<const uint8_t*>(v_cache);
  a.bt = block_table;
  a.pk = reinterpret_cast<uint8_t*>(packed_k);
  a.pv = reinterpret_cast<uint8_t*>(packed_v);
  a.ppos = packed_pos;
  a.plen = packed_len;
  a.map = slot_map;
  a.map_stride = map_stride;
  a.status = status;
  a.Hkv = s.num_kv_heads;
  a.K = prm.top_k;
  a.n_sink = prm.n_sink;
  a.cap = packed_cap;
  a.max_pages = s.max_pages_per_seq;
  a.row_bytes = s.head_dim * (s.dtype == SFI_BF16 ? 2 : 4);
  const dim3 blk(kChunkThreads);
  hipLaunchKernelGGL(k_upd_mark, dim3(n_ig * a.nc_sel), blk, 0, stream, a);
  hipLaunchKernelGGL(k_upd_count, dim3(n_ig * a.nc_slot), blk, 0, stream, a);
  hipLaunchKernelGGL(k_upd_free, dim3(n_ig * a.nc_slot), blk, 0, stream, a);
  const dim3 g_sel(n_ig * a.nc_sel);
  switch (a.row_bytes / 16) {
    case 8: hipLaunchKernelGGL(k_upd_assign<8>, g_sel, blk, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(k_upd_assign<16>, g_sel, blk, 0, stream, a); break;
    default: hipLaunchKernelGGL(k_upd_assign<32>, g_sel, blk, 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_pack(const sfi_shape& s, const sfi_select_params& prm, const void* k_cache,
                       const void* v_cache, const int32_t* block_table, const int32_t* sel_idx,
                       const int32_t* seq_ids, int n_seqs, void* packed_k, void* packed_v,
                       int32_t* packed_pos, int32_t* packed_len, int packed_cap,
                       hipStream_t stream) {
  PackArgs a;
  a.kc = reinterpret_cast<const uint8_t*>(k_cache);
  a.vc = reinterpret_cast<const uint8_t*>(v_cache);
  a.bt = block_table;
  a.sel = sel_idx;
  a.seq_ids = seq_ids;
  a.pk = reinterpret_cast<uint8_t*>(packed_k);
  a.pv = reinterpret_cast<uint8_t*>(packed_v);
  a.ppos = packed_pos;
  a.plen = packed_len;
  a.Hkv = s.num_kv_heads;
  a.max_pages = s.max_pages_per_seq;
  a.K = prm.top_k;
  a.n_sink = prm.n_sink;
  a.cap = packed_cap;
  a.row_bytes = s.head_dim * (s.dtype == SFI_BF16 ? 2 : 4);
  const int lpr = a.row_bytes / 16;  // 8, 16 or 32 lanes per row
  const int rb = kPackWaves * kPackInstr * (64 / lpr);
  a.n_work = n_seqs * s.num_kv_heads * ((packed_cap + rb - 1) / rb);
  const dim3 grid(a.n_work < kPackMaxBlocks ? a.n_work : kPackMaxBlocks);
  const dim3 block(64 * kPackWaves);
  switch (lpr) {
    case 8: hipLaunchKernelGGL(k_pack<8>, grid, block, 0, stream, a); break;
    case 16: hipLaunchKernelGGL(k_pack<16>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(k_pack<32>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace sfi
