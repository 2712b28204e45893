// seedlm_decode: dense fp32 weights from the packed records, bit-exact.
//
// Per block (SeedLM: w = 2^e * U(s) * t, U(s) the C x P matrix the seeded LFSR
// emits; paperdance.org abstract, atlas.scime.ai "Approach"):
//   I_i = sum_j t_j * (z_{j*C+i} - 2^15)      exact int32, |I_i| < 2^24
//   w_i = I_i * 2^(e-15) = I_i * 2^(g-30)     exact in fp32 (power-of-two scale)
// The kernel is bound by the 4-byte-per-weight writes; one thread rebuilds one
// block and writes it with 16-byte stores where the row allows.
#include "lfsr_device.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

__device__ inline float pow2f(int k) { return __int_as_float((k + 127) << 23); }

template <int C, int P>
__global__ void __launch_bounds__(256) decode_kernel(const uint32_t* __restrict__ words,
                                                     const uint16_t* __restrict__ exps,
                                                     float* __restrict__ W, int64_t rows,
                                                     int64_t cols, int64_t nb, int64_t Mp,
                                                     bool vec_ok) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * nb) return;
  const int64_t r = gid / nb, b = gid - r * nb;
  const uint32_t w = words[word_index(r, b, Mp, nb)];
  int g;
  if constexpr (P == 3) {
    g = (int)(w >> 28);
  } else {
    g = (exps[exp_index(r, b, Mp, nb)] >> (4 * exp_nibble(r, b))) & 0xF;
  }
  const uint64_t stream = lfsr_stream<C * P + 15>(w);
  int t[P];
#pragma unroll
  for (int j = 0; j < P; ++j) t[j] = ((int)(w << (12 - 4 * j))) >> 28;  // sign-extend nibble
  const float scale = pow2f(g - 30);
  float out[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    int I = 0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int z = (int)((stream >> (j * C + i)) & 0xFFFFu);
      I += t[j] * (z - (int)kHalf);
    }
    out[i] = (float)I * scale;
  }
  float* dst = W + r * cols + b * C;
  const int64_t valid = cols - b * C;
  if (vec_ok && valid >= C) {
#pragma unroll
    for (int i = 0; i < C; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(out[i], out[i + 1], out[i + 2], out[i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < C; ++i)
      if (i < valid) dst[i] = out[i];
  }
}

}  // namespace

int launch_decode(const seedlm_matrix* h, float* W, hipStream_t s) {
  const int64_t n = h->rows * h->nb;
  const int threads = 256;
  const int64_t grid = (n + threads - 1) / threads;
  if (grid > 0x7FFFFFFF) return SEEDLM_E_INVALID;
  const bool vec_ok = (h->cols % 4 == 0) && ((uintptr_t)W % 16 == 0);
  const uint32_t* words = static_cast<const uint32_t*>(h->d_buf);
  const uint16_t* exps =
      reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(h->d_buf) + h->exp_off);
  if (h->C == 8)
    hipLaunchKernelGGL((decode_kernel<8, 3>), dim3((unsigned)grid), dim3(threads), 0, s, words,
                       exps, W, h->rows, h->cols, h->nb, h->Mp, vec_ok);
  else
    hipLaunchKernelGGL((decode_kernel<12, 4>), dim3((unsigned)grid), dim3(threads), 0, s, words,
                       exps, W, h->rows, h->cols, h->nb, h->Mp, vec_ok);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
