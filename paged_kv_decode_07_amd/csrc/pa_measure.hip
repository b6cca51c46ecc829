// Measurement helpers behind include/pa_measure.h: the achievable HBM read
// bandwidth of the device, reported beside the published peak, and the page
// stream of the decode kernels without their arithmetic.
#include <hip/hip_runtime.h>

#include "pa_decode.h"
#include "pa_decode_kernel.h"
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


// Page stream.  One work-group per sequence, WPH wavefronts per KV head (the
// two of a head take the first and the second half of the sequence's pages),
// RING page slots per wavefront.  Each page is requested with the decode
// kernels' own direct-to-LDS loads for page format FMT (page_dma and
// page_fetch: the same lane-to-address maps and cache policy; the same ring
// waits), read back from LDS in full once it has landed, and folded into one
// XOR word per wavefront; the slot is then refilled.  Nothing else is
// computed.
constexpr int kStreamWindow = 256;               // pages of one wavefront's block-table window

struct PageStreamArgs {
  const char* k_pool;
  const char* v_pool;
  const char* scales;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  uint32_t* sink;
  int32_t num_pages;
  int32_t max_blocks;
};

template <int FMT>
struct StreamFormat {
  static constexpr int kSlot = FMT == pa::kFmtBF16 ? 4096 : FMT == pa::kFmtINT8 ? pa::kSlotQ8 : pa::kSlotQ4;
  static constexpr int kLoads = FMT == pa::kFmtBF16 ? 4 : FMT == pa::kFmtINT8 ? 3 : 2;
};

// The rings of a work-group within the 160 KiB of LDS of a CU.
constexpr int kStreamMaxRingBytes = 160 * 1024;

template <int FMT, int WPH, int RING>
constexpr bool stream_fits() {
  return RING * pa::kWaves * WPH * StreamFormat<FMT>::kSlot <= kStreamMaxRingBytes;
}

__device__ __forceinline__ uint32_t fold4(pa::u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

template <int FMT, int WPH, int RING>
__global__ __launch_bounds__(pa::kWaves * WPH * 64) void page_stream_kernel(PageStreamArgs a) {
  using namespace pa;
  using F = StreamFormat<FMT>;
  __shared__ __attribute__((aligned(16))) char ring[RING][kWaves * WPH][F::kSlot];
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = wave / WPH, part = wave % WPH;
  int L = a.seq_lens[b];
  if (L < 0 || L > a.max_blocks * kPage) L = 0;
  const int n = (L + kPage - 1) / kPage;
  const int p0 = n * part / WPH, p1 = n * (part + 1) / WPH;
  const int32_t* row = a.block_tables + (int64_t)b * a.max_blocks;
  int ent[kStreamWindow / 64];
#pragma unroll
  for (int c = 0; c < kStreamWindow / 64; ++c)
    ent[c] = p0 + c * 64 + lane < p1 ? row[p0 + c * 64 + lane] : 0;
  auto page_id = [&](int i) -> int64_t {
    const int j = i - p0;
    int id = __builtin_amdgcn_readlane(ent[0], j & 63);
#pragma unroll
    for (int c = 1; c < kStreamWindow / 64; ++c)
      if ((j >> 6) == c) id = __builtin_amdgcn_readlane(ent[c], j & 63);
    return (unsigned)id < (unsigned)a.num_pages ? id : 0;   // an id outside the pool reads page 0
  };
  // the decode kernels' own lane maps and loads for this format
  const PageDma dma = page_dma<FMT>(g, lane, a.k_pool, a.v_pool);
  auto fetch = [&](int i, int slot) {
    page_fetch<FMT>(dma, a.k_pool, a.v_pool, a.scales, page_id(i), 0u, 0u, &ring[slot][wave][0]);
  };
  // the slot read back: every code byte once; the scale line once (lanes 32..63
  // hold a second copy of it).  The outputs are early-clobber: a later read of
  // the same asm statement must not take its address from a register an
  // earlier read is already writing.
  auto fold_slot = [&](uint32_t addr) -> uint32_t {
    if constexpr (FMT == kFmtBF16) {
      u32x4 x0, x1, x2, x3;
      asm volatile(
          "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
          "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
          : "v"(addr + 16 * lane)
          : "memory");
      return fold4(x0) ^ fold4(x1) ^ fold4(x2) ^ fold4(x3);
    } else if constexpr (FMT == kFmtINT8) {
      u32x4 x0, x1;
      uint32_t s;
      asm volatile(
          "ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:1024\n\t"
          "ds_read_b32 %2, %4 offset:2048\n\ts_waitcnt lgkmcnt(0)"
          : "=&v"(x0), "=&v"(x1), "=&v"(s)
          : "v"(addr + 16 * lane), "v"(addr + 4 * lane)
          : "memory");
      return fold4(x0) ^ fold4(x1) ^ (lane < 32 ? s : 0u);
    } else {
      u32x4 x0;
      uint32_t s;
      asm volatile("ds_read_b128 %0, %2\n\tds_read_b32 %1, %3 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(x0), "=&v"(s)
                   : "v"(addr + 16 * lane), "v"(addr + 4 * lane)
                   : "memory");
      return fold4(x0) ^ (lane < 32 ? s : 0u);
    }
  };

  const uint32_t slot0 = lds_address(&ring[0][wave][0]);
  constexpr uint32_t kRingSlotBytes = kWaves * WPH * F::kSlot;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // the block-table window has landed
  uint32_t acc = 0;
#pragma unroll
  for (int r = 0; r < RING; ++r)
    if (p0 + r < p1) fetch(p0 + r, r);
  for (int i = p0; i < p1; ++i) {
    const int slot = (i - p0) % RING;
    if constexpr (RING == 1) wait_vmem<0>();
    else wait_page<F::kLoads, RING>(min(p1 - 1 - i, RING - 1));   // page i landed
    acc ^= fold_slot(slot0 + slot * kRingSlotBytes);
    if (i + RING < p1) fetch(i + RING, slot);
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) acc ^= __shfl_xor(acc, s);
  if (lane == 0) a.sink[(int64_t)b * kWaves * WPH + wave] = acc;
}

template <int FMT, int WPH, int RING>
void launch_page_stream(int batch, const PageStreamArgs& a, hipStream_t st) {
  if constexpr (stream_fits<FMT, WPH, RING>())
    hipLaunchKernelGGL((page_stream_kernel<FMT, WPH, RING>), dim3(batch),
                       dim3(pa::kWaves * WPH * 64), 0, st, a);
}

template <int FMT>
int dispatch_page_stream(int batch, int wph, int ring, const PageStreamArgs& a, hipStream_t st) {
  bool fits;
  if (wph == 1) {
    fits = ring == 1 ? stream_fits<FMT, 1, 1>() : ring == 2 ? stream_fits<FMT, 1, 2>() : stream_fits<FMT, 1, 3>();
  } else {
    fits = ring == 1 ? stream_fits<FMT, 2, 1>() : ring == 2 ? stream_fits<FMT, 2, 2>() : stream_fits<FMT, 2, 3>();
  }
  if (!fits) return PA_ERR_VALUE;
  if (wph == 1) {
    if (ring == 1) launch_page_stream<FMT, 1, 1>(batch, a, st);
    else if (ring == 2) launch_page_stream<FMT, 1, 2>(batch, a, st);
    else launch_page_stream<FMT, 1, 3>(batch, a, st);
  } else {
    if (ring == 1) launch_page_stream<FMT, 2, 1>(batch, a, st);
    else if (ring == 2) launch_page_stream<FMT, 2, 2>(batch, a, st);
    else launch_page_stream<FMT, 2, 3>(batch, a, st);
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
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

PA_API int pa_page_stream(const pa_shape* shape, int32_t batch, const void* k_pool,
                          const void* v_pool, const void* kv_scales, int32_t page_format,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          int32_t waves_per_head, int32_t ring, uint32_t* sink, void* stream) {
  int rc = pa_host::check_shape(shape);
  if (rc != PA_OK) return rc;
  if (page_format < 0 || page_format > 2 || waves_per_head < 1 || waves_per_head > 2 || ring < 1 ||
      ring > 3 || batch < 0 || shape->max_blocks_per_seq > kStreamWindow)
    return PA_ERR_VALUE;
  if (!k_pool || !v_pool || !block_tables || !seq_lens || !sink ||
      (page_format != pa::kFmtBF16 && !kv_scales))
    return PA_ERR_NULL;
  if (!pa_host::aligned(k_pool, 16) || !pa_host::aligned(v_pool, 16) ||
      (page_format != pa::kFmtBF16 && !pa_host::aligned(kv_scales, 16)) ||
      !pa_host::aligned(block_tables, 4) || !pa_host::aligned(seq_lens, 4) ||
      !pa_host::aligned(sink, 4))
    return PA_ERR_ALIGN;
  if (batch == 0) return PA_OK;
  PageStreamArgs a{static_cast<const char*>(k_pool), static_cast<const char*>(v_pool),
                   static_cast<const char*>(kv_scales), block_tables, seq_lens, sink,
                   shape->num_pages, shape->max_blocks_per_seq};
  const hipStream_t st = (hipStream_t)stream;
  if (page_format == pa::kFmtBF16) return dispatch_page_stream<pa::kFmtBF16>(batch, waves_per_head, ring, a, st);
  if (page_format == pa::kFmtINT8) return dispatch_page_stream<pa::kFmtINT8>(batch, waves_per_head, ring, a, st);
  return dispatch_page_stream<pa::kFmtINT4>(batch, waves_per_head, ring, a, st);
}
