// sfi_fast_attn_noalloc: the fast-step attention call for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses that forbid
// hipMalloc).  It runs the kernels of sfi_fast_attn with their split partials in a
// file-scope device array instead of a caller workspace.
//
// The array lives in the library's code object: every GPU the library runs on holds its
// own copy, at its own address, until the process ends.  In host code the array's name is
// only a host-side stand-in, so its device address is resolved once per device with
// hipGetSymbolAddress (with that device current) and every launch receives that address.
#include "sfi_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = SFI_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once resolved

// Device address of this device's copy of `scratch`, resolved on first use.  The calling
// thread's current device must be the device of the call's stream.
int scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SFI_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SFI_E_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SFI_E_HIP;
    if (sdev != dev) return SFI_E_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SFI_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SFI_OK;
}

}  // namespace

extern "C" {

int sfi_fast_attn_noalloc(const sfi_shape* shape, const float* q, const void* packed_k,
                          const void* packed_v, const int32_t* packed_len, int32_t packed_cap,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          const int32_t* recent_start, const int32_t* seq_lens,
                          const int32_t* seq_ids, int32_t n_seqs, int32_t max_recent,
                          float* out, float* lse, uint32_t* status, void* stream) {
  // Validate every argument against a stand-in workspace of the maximum size (never
  // dereferenced) before touching the device, so argument errors come back exactly as
  // sfi_fast_attn returns them; then reject calls whose partials do not fit the array.
  static_assert(kScratchBytes % 256 == 0, "scratch size");
  void* const probe = reinterpret_cast<void*>(uintptr_t(256));
  int rc = sfi_fast_attn(shape, q, packed_k, packed_v, packed_len, packed_cap, k_cache,
                         v_cache, block_table, recent_start, seq_lens, seq_ids, 0, max_recent,
                         out, lse, status, probe, kScratchBytes, stream);
  if (rc) return rc;
  if (n_seqs < 0 || n_seqs > shape->batch) return SFI_E_ARG;
  if (n_seqs == 0) return SFI_OK;
  const size_t need = sfi_fast_attn_ws(shape, n_seqs, packed_cap, max_recent);
  if (need == 0 || need > kScratchBytes) return SFI_E_WORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = scratch_for(s, &ws))) return rc;
  return sfi_fast_attn(shape, q, packed_k, packed_v, packed_len, packed_cap, k_cache, v_cache,
                       block_table, recent_start, seq_lens, seq_ids, n_seqs, max_recent, out,
                       lse, status, ws, kScratchBytes, stream);
}

}  // extern "C"
