// Compaction of the fast-step memory: sink rows and Selector-chosen rows are copied from
// the paged cache into one contiguous buffer per (row b, KV head g), so fast steps read
// them sequentially instead of gathering scattered pages (zh "2.3 显存合并的内核",
// nl "Memory-Coalesced Kernel", fr "2.C Kernels Mémoire-Coalescés").
//
// One wavefront per group of 16 packed rows: the four lanes l = 4 r .. 4 r + 3 copy row r
// of K and V, 64 contiguous bytes per step.  Packed row i holds position packed_pos[i] = i for i < n_sink and
// sel_idx[i - n_sink] after; rows without a position are zero-filled.
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
};

__device__ __forceinline__ int packed_source(const PackArgs& a, const int32_t* selrow, int row) {
  if (row < a.n_sink) return row;
  const int k = row - a.n_sink;
  return k < a.K ? selrow[k] : -1;
}

__global__ __launch_bounds__(64) void k_pack(PackArgs a) {
  const int lane = threadIdx.x;
  const int ngrp = a.cap / kPage;
  const int grp = blockIdx.x % ngrp;
  const int ig = blockIdx.x / ngrp;
  const int g = ig % a.Hkv, i = ig / a.Hkv;
  const int b = a.seq_ids[i];
  const size_t bg = (size_t)b * a.Hkv + g;
  const int32_t* selrow = a.sel + bg * a.K;
  const int row = grp * kPage + lane / 4;
  const int quarter = lane % 4;
  const int pos = packed_source(a, selrow, row);
  // The four lanes of a row copy 64 contiguous bytes per step.
  uint8_t* dk = a.pk + (bg * a.cap + row) * a.row_bytes + quarter * 16;
  uint8_t* dv = a.pv + (bg * a.cap + row) * a.row_bytes + quarter * 16;
  if (pos >= 0) {
    const int page = a.bt[(size_t)b * a.max_pages + pos / kPage];
    const size_t src = (((size_t)page * a.Hkv + g) * kPage + pos % kPage) * a.row_bytes +
                       quarter * 16;
    // All loads of the row first, then all stores (rows are at most 512 bytes).
    constexpr int kMaxSteps = 8;
    const int steps = a.row_bytes / 64;
    u32x4_t kv[kMaxSteps], vv[kMaxSteps];
#pragma unroll
    for (int k = 0; k < kMaxSteps; ++k) {
      if (k < steps) {
        kv[k] = *reinterpret_cast<const u32x4_t*>(a.kc + src + 64 * k);
        vv[k] = *reinterpret_cast<const u32x4_t*>(a.vc + src + 64 * k);
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxSteps; ++k) {
      if (k < steps) {
        *reinterpret_cast<u32x4_t*>(dk + 64 * k) = kv[k];
        *reinterpret_cast<u32x4_t*>(dv + 64 * k) = vv[k];
      }
    }
  } else {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int o = 0; o < a.row_bytes; o += 64) {
      *reinterpret_cast<u32x4_t*>(dk + o) = zero;
      *reinterpret_cast<u32x4_t*>(dv + o) = zero;
    }
  }
  if (quarter == 0) {
    a.ppos[bg * a.cap + row] = pos;
    // Valid rows form a prefix: the last valid row (or group 0 when none is valid)
    // records the packed length.
    const int next = row + 1 < a.cap ? packed_source(a, selrow, row + 1) : -1;
    if (pos >= 0 && next < 0) a.plen[bg] = row + 1;
    if (row == 0 && pos < 0) a.plen[bg] = 0;
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
  const int blocks = n_seqs * s.num_kv_heads * (packed_cap / kPage);
  hipLaunchKernelGGL(k_pack, dim3(blocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sfi
