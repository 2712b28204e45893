// seedlm_decode: dense fp32 weights from the packed records, bit-exact.
//
// Per block (SeedLM: w = 2^e * U(s) * t, U(s) the C x P matrix the seeded LFSR
// emits; paperdance.org abstract, atlas.scime.ai "Approach"):
//   I_i = sum_j t_j * (z_{j*C+i} - 2^(K-1))      exact int32, |I_i| < 2^24
//   w_i = I_i * 2^(e-(K-1)) = I_i * 2^(g-14-K)   exact in fp32 (power-of-two scale)
// for every packed format (K = 16 or 20, Q-bit coefficients).
// The kernel is bound by the 4-byte-per-weight writes, so the thread mapping
// follows the output: thread k of a row writes columns 4k .. 4k+3 with one
// 16-byte nontemporal store (the output is not re-read here), and consecutive
// lanes write consecutive 16-byte chunks (C is a multiple of 4, so a chunk
// never straddles two blocks).  The stream bits
// past the seed come from GF(2) byte tables in LDS (ext(s) = T0[s & 255] ^
// T1[(s >> 8) & 255] ^ T2[s >> 16]); z_n is the K-bit window of the stream at
// bit n.
#include <type_traits>

#include "lfsr_device.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

constexpr int kThreads = 256;
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ inline float pow2f(int k) { return __int_as_float((k + 127) << 23); }

// Stream words of a block: bits 0 .. K + C*P - 2 of its LFSR stream are the
// seed and its extension; Ext holds the extension bits K .. (32 or 64 of them).
template <int C, int P, int K>
using DecExt = typename std::conditional<(C * P - 1 <= 32), uint32_t, uint64_t>::type;

template <int C, int P, int K, int Q>
__global__ void __launch_bounds__(kThreads) decode_kernel(const uint32_t* __restrict__ words,
                                                          const uint16_t* __restrict__ exps,
                                                          float* __restrict__ W, int rows,
                                                          int cols, int nb, int Mp, bool vec_ok) {
  using Ext = DecExt<C, P, K>;
  constexpr int PB = panel_blocks(C);
  constexpr uint32_t kSeedMask = (1u << K) - 1u;
  // GF(2) tables of the extension bits, one per seed byte (K = 20: three, the
  // third indexed by the seed's top nibble).
  __shared__ Ext T[3][256];
  for (int e = threadIdx.x; e < 768; e += kThreads) {
    const uint32_t u = (uint32_t)e & 255u, k = (uint32_t)e >> 8;
    T[k][u] = (k == 2 && K <= 16) ? Ext(0) : ext_bits_k<K, Ext>(u << (8 * k));
  }
  __syncthreads();
  const int col0 = 4 * (blockIdx.x * kThreads + threadIdx.x);
  if (col0 >= cols) return;
  const int b = col0 / C, i0 = col0 - b * C;  // block, first weight inside it
  const int p = b / PB, q = b % PB;
  const int Wp = (int)panel_stored_width(p, nb, PB);
  const int valid = cols - col0;  // >= 1
  // Rows y, y + gy, ...: the record words of the next kRing rows are loaded
  // ahead (clamped to a valid row, so no load is conditional) to keep enough
  // reads in flight; each thread reads only 4 bytes per row.
  const int gy = (int)gridDim.y;
  const int64_t wbase = (int64_t)p * Mp * PB + (q & ~3);
  const int64_t ebase = (int64_t)p * Mp * (PB / 4) + q / 4;
  auto word_at = [&](int r) { return words[wbase + (int64_t)r * Wp + ((q - r) & 3)]; };
  auto exp_at = [&](int r) -> uint32_t {
    if constexpr (C == 8) return 0u;
    else return exps[ebase + (int64_t)r * (Wp / 4)];
  };
  constexpr int kRing = 4;
  uint32_t wr[kRing], er[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) {
    const int rr = min((int)blockIdx.y + k * gy, rows - 1);
    wr[k] = word_at(rr);
    er[k] = exp_at(rr);
  }
  for (int r0 = blockIdx.y; r0 < rows; r0 += kRing * gy) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int r = r0 + k * gy;
      if (r >= rows) break;
      const uint32_t w = wr[k];
      const uint32_t ev = er[k];
      {
        const int rn = min(r + kRing * gy, rows - 1);
        wr[k] = word_at(rn);
        er[k] = exp_at(rn);
      }
      int g;
      if constexpr (C == 8) {
        g = (int)(w >> 28);
      } else {
        g = (int)(ev >> (4 * ((q - r) & 3))) & 0xF;
      }
      Ext ext = T[0][w & 0xFFu] ^ T[1][(w >> 8) & 0xFFu];
      if constexpr (K > 16) ext ^= T[2][(w >> 16) & 0xFu];
      // stream bits 0..63, shifted so that bit 0 is window i0's first bit
      const uint64_t S = ((uint64_t)(w & kSeedMask) | ((uint64_t)ext << K)) >> i0;
      int t[P];
      int base = 0;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        t[j] = ((int)(w << (32 - K - Q * (j + 1)))) >> (32 - Q);  // sign-extend t_j
        base -= t[j] * (1 << (K - 1));
      }
      const float scale = pow2f(g - 14 - K);  // 2^(e - (K-1)), e = g - 15
      float out[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int I = base;
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const int n = j * C + u;  // window offset from bit i0
          uint32_t z;
          if constexpr (K == 16) {
            const uint32_t s0 = (uint32_t)S, s1 = (uint32_t)(S >> 16), s2 = (uint32_t)(S >> 32);
            z = n <= 16 ? __builtin_amdgcn_ubfe(s0, n, 16)
                        : (n <= 32 ? __builtin_amdgcn_ubfe(s1, n - 16, 16)
                                   : __builtin_amdgcn_ubfe(s2, n - 32, 16));
          } else {
            z = (uint32_t)(S >> n) & kSeedMask;
          }
          I += t[j] * (int)z;
        }
        out[u] = (float)I * scale;
      }
      float* dst = W + (int64_t)r * cols + col0;
      if (vec_ok && valid >= 4) {
        __builtin_nontemporal_store(f4{out[0], out[1], out[2], out[3]}, reinterpret_cast<f4*>(dst));
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (u < valid) dst[u] = out[u];
      }
    }
  }
}

}  // namespace

int launch_decode(const seedlm_matrix* h, float* W, hipStream_t s) {
  if (h->rows >= (1LL << 31) || h->cols >= (1LL << 31) - 4 || h->Mp >= (1LL << 31))
    return SEEDLM_E_UNSUPPORTED;
  const int64_t chunks = (h->cols + 3) / 4;
  const int64_t gx = (chunks + kThreads - 1) / kThreads;
  // Up to 2048 row slots; a workgroup handles rows y, y + 2048, ... (its GF(2)
  // tables are built once for all of them).
  const int64_t gy = h->rows < 2048 ? h->rows : 2048;
  const bool vec_ok = (h->cols % 4 == 0) && ((uintptr_t)W % 16 == 0);
  const uint32_t* words = static_cast<const uint32_t*>(h->d_buf);
  const uint16_t* exps =
      reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(h->d_buf) + h->exp_off);
  const dim3 grid((unsigned)gx, (unsigned)gy);
  const int R = (int)h->rows, Cn = (int)h->cols, nb = (int)h->nb, Mp = (int)h->Mp;
  if (h->is_4bit())
    hipLaunchKernelGGL((decode_kernel<8, 3, 16, 4>), grid, dim3(kThreads), 0, s, words, exps, W,
                       R, Cn, nb, Mp, vec_ok);
  else if (h->is_3bit())
    hipLaunchKernelGGL((decode_kernel<12, 4, 16, 4>), grid, dim3(kThreads), 0, s, words, exps, W,
                       R, Cn, nb, Mp, vec_ok);
  else if (h->C == 8)
    hipLaunchKernelGGL((decode_kernel<8, 4, 16, 3>), grid, dim3(kThreads), 0, s, words, exps, W,
                       R, Cn, nb, Mp, vec_ok);
  else
    hipLaunchKernelGGL((decode_kernel<12, 3, 20, 4>), grid, dim3(kThreads), 0, s, words, exps, W,
                       R, Cn, nb, Mp, vec_ok);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
