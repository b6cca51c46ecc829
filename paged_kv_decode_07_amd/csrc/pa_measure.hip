// Streaming-read helper behind include/pa_measure.h: the achievable HBM read
// bandwidth of the device, reported beside the published peak.
#include <hip/hip_runtime.h>

#include "pa_decode.h"
#include "pa_host.h"
#include "pa_measure.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

// Each work-group reads 16 KiB chunks (256 lanes x 4 loads of 16 bytes, the
// 4 loads of a lane 4 KiB apart, all issued before any use) and strides over
// the chunks of the buffer; one folded word per work-group.  The loads carry
// the non-temporal policy, the fastest plain streaming read measured on this
// part (about 10% above the default policy).
constexpr int kUnroll = 4;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4v* __restrict__ buf, size_t n,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t chunk = 256 * kUnroll;                       // words per chunk
  const size_t stride = (size_t)gridDim.x * chunk;
  for (size_t base = (size_t)blockIdx.x * chunk + threadIdx.x; base < n; base += stride) {
    u32x4v v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = i < n ? __builtin_nontemporal_load(buf + i) : u32x4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

}  // namespace

PA_API int pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t groups,
                          void* stream) {
  if (!buf || !sink) return PA_ERR_NULL;
  if (!pa_host::aligned(buf, 16) || !pa_host::aligned(sink, 4)) return PA_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 != 0 || groups < 0 || groups > 65536) return PA_ERR_VALUE;
  if (groups == 0) {
    int cu = 0;
    const int rc = pa_host::current_cu_count(&cu);
    if (rc != PA_OK) return rc;
    groups = 4 * cu;
    if (groups > 65536) groups = 65536;
  }
  hipLaunchKernelGGL(stream_read_kernel, dim3(groups), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4v*)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
