// Streaming-read ceiling (measurement only, not part of the method).  A plain
// kernel that reads a device buffer once with 16-byte loads and folds it into
// per-workgroup XOR checksums: the read rate it reaches on a buffer larger than
// the last-level cache is the ceiling a bandwidth-bound kernel can approach on
// this device, reported beside the published HBM peak.  The fold keeps the
// loads from being optimised away and gives a test an exact result (the XOR of
// all checksums equals the XOR of the buffer's 32-bit words).
#include "seedlm_internal.h"

namespace seedlm {
namespace {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread

// Workgroup b reads the contiguous range [b per, min(n, (b+1) per)) of 16-byte
// words: contiguous ranges per workgroup measured faster on this device than a
// grid-stride walk (about 6.3 against 5.5 TB/s on 2 GiB).
__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const uint4* __restrict__ p,
                                                                   int64_t n,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kReadThreads / 64];
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n ? beg + per : n;
  int64_t i = beg + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * kReadThreads < end; i += kReadUnroll * kReadThreads) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) v[k] = p[i + k * kReadThreads];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < end; i += kReadThreads) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / 64; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

}  // namespace

int launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s) {
  int grid = 32 * device_cu_count();
  if (grid > SEEDLM_STREAM_READ_SINK) grid = SEEDLM_STREAM_READ_SINK;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, s,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
