// fp16 GEMV baseline (measurement only, not part of the method): the speed-up
// denominator for the compressed path, standing in on this chip for the FP16
// reference design the pages compare against (atlas.scime.ai, "Key results").
//
// y[b][r] = sum_c W[r][c] * x[b][c], W and x fp16, fp32 accumulation, y fp16.
// Each wave owns RW rows; the workgroup walks the columns in 512-column chunks,
// staging x[:, chunk] in LDS once per chunk so every W byte is read once from
// HBM with 16-byte loads, and multiplies with v_dot2_f32_f16.
#include <hip/hip_fp16.h>

#include "seedlm_internal.h"

namespace seedlm {
namespace {

constexpr int kChunk = 512;  // columns per chunk: 64 lanes x 8 halves

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ inline float dot8(const uint4& a, const uint4& b, float acc) {
  const uint32_t av[4] = {a.x, a.y, a.z, a.w};
  const uint32_t bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int k = 0; k < 4; ++k)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, av[k]),
                                 __builtin_bit_cast(half2v, bv[k]), acc, false);
  return acc;
}

template <int RW, int B>
__global__ void __launch_bounds__(256) fp16_gemv_kernel(const uint4* __restrict__ W,
                                                        const __half* __restrict__ x,
                                                        __half* __restrict__ y, int64_t rows,
                                                        int64_t cols, int batch) {
  __shared__ uint4 xs[B][kChunk / 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RW;
  const int64_t cw = cols / 8;  // uint4 per row
  float acc[RW][B];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[i][b] = 0.f;

  for (int64_t c0 = 0; c0 < cols; c0 += kChunk) {
    __syncthreads();
    for (int k = threadIdx.x; k < B * (kChunk / 8); k += blockDim.x) {
      const int b = k / (kChunk / 8), j = k % (kChunk / 8);
      const int64_t c = c0 + (int64_t)j * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (b < batch && c < cols) v = *reinterpret_cast<const uint4*>(x + (int64_t)b * cols + c);
      xs[b][j] = v;
    }
    __syncthreads();
    const int64_t cj = c0 / 8 + lane;
    if (cj < cw) {
      uint4 wv[RW];
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int64_t r = row0 + i;
        wv[i] = (r < rows) ? W[r * cw + cj] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint4 xv = xs[b][lane];
#pragma unroll
        for (int i = 0; i < RW; ++i) acc[i][b] = dot8(wv[i], xv, acc[i][b]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RW; ++i) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = acc[i][b];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      const int64_t r = row0 + i;
      if (lane == 0 && r < rows && b < batch) y[(int64_t)b * rows + r] = __float2half_rn(v);
    }
  }
}

template <int RW, int B>
void launch_rb(const void* W, const void* x, void* y, int64_t rows, int64_t cols, int batch,
               hipStream_t s) {
  const int64_t grid = (rows + 4 * RW - 1) / (4 * RW);
  hipLaunchKernelGGL((fp16_gemv_kernel<RW, B>), dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const uint4*>(W), static_cast<const __half*>(x),
                     static_cast<__half*>(y), rows, cols, batch);
}

template <int RW>
void launch_r(const void* W, const void* x, void* y, int64_t rows, int64_t cols, int batch,
              hipStream_t s) {
  if (batch == 1) launch_rb<RW, 1>(W, x, y, rows, cols, batch, s);
  else if (batch <= 2) launch_rb<RW, 2>(W, x, y, rows, cols, batch, s);
  else if (batch <= 4) launch_rb<RW, 4>(W, x, y, rows, cols, batch, s);
  else if (batch <= 8) launch_rb<RW, 8>(W, x, y, rows, cols, batch, s);
  else launch_rb<RW, 16>(W, x, y, rows, cols, batch, s);
}

}  // namespace

int launch_fp16_gemv(const void* W, const void* x, void* y, int64_t rows, int64_t cols, int batch,
                     hipStream_t s) {
  // Enough workgroups to fill the chip: 4 rows per wave only for tall matrices.
  const int64_t cus = device_cu_count();
  if (rows / 16 >= 2 * cus) launch_r<4>(W, x, y, rows, cols, batch, s);
  else if (rows / 8 >= 2 * cus) launch_r<2>(W, x, y, rows, cols, batch, s);
  else launch_r<1>(W, x, y, rows, cols, batch, s);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
