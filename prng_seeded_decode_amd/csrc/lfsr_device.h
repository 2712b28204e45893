// Device-side LFSR helpers for libseedlm.
//
// The 16-bit Fibonacci LFSR of the format (feedback bit0 ^ bit2 ^ bit3 ^ bit5,
// entering at bit 15) makes every state a 16-bit window of one bit stream b:
// b[0..15] are the seed bits (LSB first), b[m+16] = b[m]^b[m+2]^b[m+3]^b[m+5],
// and state z_n = sum_k b[n+k] 2^k.  A block needs b[0 .. C*P+14]: 39 bits for
// (C,P) = (8,3), 63 bits for (12,4).  SeedLM generates the block's random
// matrix from the seed with an LFSR (paperdance.org abstract; atlas.scime.ai
// "Approach"); the word-level stepping and the GF(2) jump tables below are this
// library's way of producing that stream on a GPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seedlm {

// Feedback of the K-bit Fibonacci LFSRs of the packed formats, as a word-level
// map: bit m of next(b) is b[m+K] wherever b[m .. m+kMaxTap] are known.
//   K = 16: b[m+16] = b[m] ^ b[m+2] ^ b[m+3] ^ b[m+5]   (x^16 + x^5 + x^3 + x^2 + 1)
//   K = 20: b[m+20] = b[m] ^ b[m+3]                      (x^20 + x^3 + 1)
template <int K>
struct LfsrTaps;
template <>
struct LfsrTaps<16> {
  static constexpr int kMaxTap = 5;
  __host__ __device__ static uint64_t next(uint64_t b) { return b ^ (b >> 2) ^ (b >> 3) ^ (b >> 5); }
};
template <>
struct LfsrTaps<20> {
  static constexpr int kMaxTap = 3;
  __host__ __device__ static uint64_t next(uint64_t b) { return b ^ (b >> 3); }
};

// Stream bits b[0 .. NBITS-1] (NBITS <= 64) of the K-bit LFSR from a seed,
// K - kMaxTap new bits per round (11 for K = 16, 17 for K = 20): with L bits
// known, next(b) has bits m <= L-1-kMaxTap right, which are b[K .. L-1-kMaxTap+K].
template <int K, int NBITS>
__host__ __device__ inline uint64_t lfsr_stream_k(uint32_t seed) {
  constexpr int kNew = K - LfsrTaps<K>::kMaxTap;
  uint64_t b = seed & ((1u << K) - 1u);
#pragma unroll
  for (int L = K; L < NBITS; L += kNew) {
    const uint64_t x = LfsrTaps<K>::next(b);
    b |= ((x >> (L - K)) & ((1ull << kNew) - 1ull)) << L;
  }
  return b;
}

// The 16-bit LFSR of the pages' two formats.
template <int NBITS>
__host__ __device__ inline uint64_t lfsr_stream(uint32_t seed) {
  return lfsr_stream_k<16, NBITS>(seed);
}

// The stream is GF(2)-linear in the seed, so its extension bits b[16..] split
// over the seed bytes: ext(s) = ext(s & 0xFF) ^ ext(s & 0xFF00).  T0 and T1 hold
// those two 256-entry halves (32 extension bits each, or 64 for 64-bit entries).
template <typename T>
__host__ __device__ inline T ext_bits(uint32_t seed16) {
  constexpr int kBits = 16 + 8 * (int)sizeof(T) > 64 ? 64 : 16 + 8 * (int)sizeof(T);
  return (T)(lfsr_stream<kBits>(seed16) >> 16);
}

// The same for a K-bit seed: stream bits K .. K + 8*sizeof(T) - 1 (at most bit
// 63), linear in the seed, so a seed's extension is the XOR of its bytes' ones.
template <int K, typename T>
__host__ __device__ inline T ext_bits_k(uint32_t seed) {
  constexpr int kBits = K + 8 * (int)sizeof(T) > 64 ? 64 : K + 8 * (int)sizeof(T);
  return (T)(lfsr_stream_k<K, kBits>(seed) >> K);
}

}  // namespace seedlm
