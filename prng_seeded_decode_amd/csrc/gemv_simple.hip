// Reference-grade fused decode-GEMV: one wavefront per output row, each lane
// rebuilds whole blocks (exact integer reconstruction, as in decode) and
// multiplies them with x.  Every packed format, batch 1..16, any dtype pair.  This is
// the correctness anchor for the faster kernels and the SIMPLE variant of the
// A/B measurements.  SeedLM's inference step: fetch s and t, rebuild the
// weights on the fly, use them to compute the activations (paperhub.cn
// rebuttal text before Eq. (1)).
#include <hip/hip_fp16.h>

#include "lfsr_device.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

template <typename T>
__device__ inline float to_f32(T v);
template <>
__device__ inline float to_f32<float>(float v) { return v; }
template <>
__device__ inline float to_f32<__half>(__half v) { return __half2float(v); }

template <typename T>
__device__ inline void store_out(T* p, float v);
template <>
__device__ inline void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void store_out<__half>(__half* p, float v) { *p = __float2half_rn(v); }

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int C, int P, int K, int Q, int B, typename XT, typename YT>
__global__ void __launch_bounds__(256) gemv_simple_kernel(const uint32_t* __restrict__ words,
                                                          const uint16_t* __restrict__ exps,
                                                          const XT* __restrict__ x,
                                                          YT* __restrict__ y, int64_t rows,
                                                          int64_t cols, int64_t nb, int64_t Mp,
                                                          int batch) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;
  float acc[B];
#pragma unroll
  for (int k = 0; k < B; ++k) acc[k] = 0.f;
  constexpr int PB = panel_blocks(C);
  for (int64_t b = lane; b < nb; b += 64) {
    const uint32_t w = words[word_index(r, b, Mp, nb, PB)];
    int g;
    if constexpr (C == 8) {
      g = (int)(w >> 28);
    } else {
      g = (exps[exp_index(r, b, Mp, nb, PB)] >> (4 * exp_nibble(r, b, PB))) & 0xF;
    }
    const uint64_t stream = lfsr_stream_k<K, C * P + K - 1>(w);
    int t[P];
#pragma unroll
    for (int j = 0; j < P; ++j) t[j] = ((int)(w << (32 - K - Q * (j + 1)))) >> (32 - Q);
    const float scale = __int_as_float((g - 14 - K + 127) << 23);  // 2^(e - (K-1))
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int64_t c = b * C + i;
      if (c >= cols) break;
      int I = 0;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int z = (int)((stream >> (j * C + i)) & ((1u << K) - 1u));
        I += t[j] * (z - (1 << (K - 1)));
      }
      const float wv = (float)I * scale;
#pragma unroll
      for (int k = 0; k < B; ++k)
        if (k < batch) acc[k] = fmaf(wv, to_f32(x[(int64_t)k * cols + c]), acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < B; ++k) {
    if (k < batch) {
      const float s = wave_sum(acc[k]);
      if (lane == 0) store_out(y + (int64_t)k * rows + r, s);
    }
  }
}

template <int C, int P, int K, int Q, typename XT, typename YT>
int launch_typed(const seedlm_matrix* h, const void* x, void* y, int batch, hipStream_t s) {
  const int waves = 4;
  const int64_t grid = (h->rows + waves - 1) / waves;
  const uint32_t* words = static_cast<const uint32_t*>(h->d_buf);
  const uint16_t* exps =
      reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(h->d_buf) + h->exp_off);
  const XT* xp = static_cast<const XT*>(x);
  YT* yp = static_cast<YT*>(y);
  if (batch == 1)
    hipLaunchKernelGGL((gemv_simple_kernel<C, P, K, Q, 1, XT, YT>), dim3((unsigned)grid),
                       dim3(64 * waves), 0, s, words, exps, xp, yp, h->rows, h->cols, h->nb,
                       h->Mp, batch);
  else
    hipLaunchKernelGGL((gemv_simple_kernel<C, P, K, Q, SEEDLM_MAX_BATCH, XT, YT>),
                       dim3((unsigned)grid),
                       dim3(64 * waves), 0, s, words, exps, xp, yp, h->rows, h->cols, h->nb,
                       h->Mp, batch);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

template <int C, int P, int K, int Q>
int launch_cp(const seedlm_matrix* h, const void* x, void* y, int batch, int xdt, int ydt,
              hipStream_t s) {
  if (xdt == SEEDLM_F32 && ydt == SEEDLM_F32)
    return launch_typed<C, P, K, Q, float, float>(h, x, y, batch, s);
  if (xdt == SEEDLM_F32 && ydt == SEEDLM_F16)
    return launch_typed<C, P, K, Q, float, __half>(h, x, y, batch, s);
  if (xdt == SEEDLM_F16 && ydt == SEEDLM_F32)
    return launch_typed<C, P, K, Q, __half, float>(h, x, y, batch, s);
  return launch_typed<C, P, K, Q, __half, __half>(h, x, y, batch, s);
}

}  // namespace

int launch_gemv_simple(const seedlm_matrix* h, const void* x, void* y, int batch, int xdt,
                       int ydt, hipStream_t s) {
  if (h->is_4bit()) return launch_cp<8, 3, 16, 4>(h, x, y, batch, xdt, ydt, s);
  if (h->is_3bit()) return launch_cp<12, 4, 16, 4>(h, x, y, batch, xdt, ydt, s);
  if (h->C == 8) return launch_cp<8, 4, 16, 3>(h, x, y, batch, xdt, ydt, s);
  return launch_cp<12, 3, 20, 4>(h, x, y, batch, xdt, ydt, s);
}

}  // namespace seedlm
