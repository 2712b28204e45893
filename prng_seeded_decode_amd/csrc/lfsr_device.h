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

// Stream bits b[0 .. nbits-1] (nbits <= 64) from a seed, 11 new bits per round:
// x = b ^ b>>2 ^ b>>3 ^ b>>5 has bit m equal to b[m+16] wherever b[m..m+5] are
// known, i.e. for m <= L-6 once L bits are known.
template <int NBITS>
__host__ __device__ inline uint64_t lfsr_stream(uint32_t seed) {
  uint64_t b = seed & 0xFFFFu;
#pragma unroll
  for (int L = 16; L < NBITS; L += 11) {
    const uint64_t x = b ^ (b >> 2) ^ (b >> 3) ^ (b >> 5);
    b |= ((x >> (L - 16)) & 0x7FFull) << L;
  }
  return b;
}

// The stream is GF(2)-linear in the seed, so its extension bits b[16..] split
// over the seed bytes: ext(s) = ext(s & 0xFF) ^ ext(s & 0xFF00).  T0 and T1 hold
// those two 256-entry halves (32 extension bits each, or 64 for 64-bit entries).
template <typename T>
__host__ __device__ inline T ext_bits(uint32_t seed16) {
  constexpr int kBits = 16 + 8 * (int)sizeof(T) > 64 ? 64 : 16 + 8 * (int)sizeof(T);
  return (T)(lfsr_stream<kBits>(seed16) >> 16);
}

}  // namespace seedlm
