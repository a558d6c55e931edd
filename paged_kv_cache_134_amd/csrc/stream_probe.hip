// Streaming-read probe: a measurement aid, not a step of the method.  It
// reads a device buffer once with the loads the decode kernels use for K/V
// rows (16-byte, non-temporal) and keeps nothing but a digest, so its rate
// is the practical ceiling of HBM reads on this GPU, against which the
// decode kernels' algorithmic bandwidth is also reported.
#include <hip/hip_runtime.h>

#include <string>

#include "kernel_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;        // independent 16-byte loads in flight per thread
constexpr int kProbeBlocksPerCu = 2;

// Workgroup b reads one contiguous slab of the buffer; its threads take
// consecutive 16-byte chunks (each wave's load covers whole cache lines),
// kProbeUnroll of them in flight per thread.  Of the patterns measured on
// MI355X (grid-strided or slabbed, 1-16 loads in flight, 2-32 workgroups per
// CU, plain or non-temporal loads) this one read fastest.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ buf,
                                                                    int64_t chunks,
                                                                    uint32_t* __restrict__ sink) {
  const int64_t slab = (chunks + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * slab;
  const int64_t hi = min(chunks, lo + slab);
  uint32_t x = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < hi; i += kProbeUnroll * kProbeThreads) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load_nt(buf + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += kProbeThreads) {
    const uint4 v = load_nt(buf + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one digest per workgroup (a lane-0 vector store after a wave reduction
  // is enough to keep every load live)
  for (int d = 1; d < kWave; d <<= 1) x ^= __shfl_xor(x, d);
  __shared__ uint32_t red[kProbeThreads / kWave];
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / kWave; ++w) y ^= red[w];
    sink[blockIdx.x] = y;
  }
}

int probe_blocks() { return device_cus() * kProbeBlocksPerCu; }

}  // namespace
}  // namespace pa

extern "C" int32_t pa_stream_read_probe_sink_words(void) { return pa::probe_blocks(); }

extern "C" pa_status pa_stream_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                          void* stream) {
  if (bytes == 0 || bytes % 16 != 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_stream_read_probe: bytes must be a positive multiple of 16");
  if (!buf || !sink) return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_stream_read_probe: null pointer");
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return pa_fail(PA_ERR_INVALID_ARGUMENT, "pa_stream_read_probe: buf must be 16-byte aligned");
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3(pa::probe_blocks()), dim3(pa::kProbeThreads), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(buf), (int64_t)(bytes / 16),
                     sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    std::string msg = std::string("pa_stream_read_probe: ") + hipGetErrorString(e);
    return pa_fail(PA_ERR_HIP, msg.c_str());
  }
  return PA_OK;
}
