// Compaction of the fast-step memory: sink rows and Selector-chosen rows are copied from
// the paged cache into one contiguous buffer per (row b, KV head g), so fast steps read
// them sequentially instead of gathering scattered pages (zh "2.3 显存合并的内核",
// nl "Memory-Coalesced Kernel", fr "2.C Kernels Mémoire-Coalescés").
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

}  // namespace

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
