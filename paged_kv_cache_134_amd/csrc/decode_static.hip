// pa_decode for callers that cannot allocate device memory: the split-K
// workspace is a file-scope device array of PA_STATIC_SCRATCH_BYTES per GPU
// (partials, their (max, sum) records and the dispatch list), otherwise the
// call is pa_decode itself.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <string>

#include "pa.h"
#include "pa_internal.h"

namespace {

// One array per GPU, held until the process ends.  On the host its name is
// only a stand-in: its device address comes from hipGetSymbolAddress, once
// per device, and every use (the kernels' workspace argument) takes that
// address.
__device__ __align__(256) char scratch[PA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

pa_status fail_hip(hipError_t e, const char* what) {
  const std::string msg = std::string("pa_decode_static_scratch: ") + what + ": " + hipGetErrorString(e);
  return pa_fail(PA_ERR_HIP, msg.c_str());
}

// Device address of the current device's array (resolved on the first call
// made on that device).
pa_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return pa_fail(PA_ERR_UNSUPPORTED, "pa_decode_static_scratch: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail_hip(hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_static_scratch(void* out, pa_dtype out_dtype, const void* query,
                                              const void* key_cache, const void* value_cache,
                                              pa_dtype kv_dtype, pa_layout layout,
                                              const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens,
                                              int32_t max_context_len, int32_t num_seqs,
                                              int32_t num_heads, int32_t num_kv_heads,
                                              int32_t head_size, int32_t block_size,
                                              int32_t num_blocks, float scale,
                                              int32_t partition_size, void* stream) {
  // the partition size pa_decode would resolve, and the workspace it needs,
  // checked before any device call
  int32_t ps = partition_size;
  if (ps < 0 && num_seqs > 0 && num_heads > 0 && num_kv_heads > 0)
    ps = pa_decode_auto_partition(num_seqs, num_heads, num_kv_heads, kv_dtype, max_context_len, 0);
  void* ws = nullptr;
  if (ps > 0 && num_seqs > 0) {
    const size_t need = pa_decode_workspace_size(num_seqs, num_heads, head_size, max_context_len, ps);
    if (need > (size_t)PA_STATIC_SCRATCH_BYTES) {
      char msg[200];
      std::snprintf(msg, sizeof msg,
                    "pa_decode_static_scratch: split-K needs %zu workspace bytes, the static "
                    "scratch holds %zu (pa_decode takes a caller workspace)",
                    need, (size_t)PA_STATIC_SCRATCH_BYTES);
      return pa_fail(PA_ERR_WORKSPACE_TOO_SMALL, msg);
    }
    const pa_status st = scratch_of_current_device(&ws);
    if (st != PA_OK) return st;
  }
  return pa_decode(out, out_dtype, query, key_cache, value_cache, kv_dtype, layout, block_tables,
                   max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_heads,
                   num_kv_heads, head_size, block_size, num_blocks, scale, ps, ws,
                   ws ? (size_t)PA_STATIC_SCRATCH_BYTES : 0, stream);
}
