// Exact decode of packed blocks into fp16 operands for the matrix cores, shared
// by the skinny decode-GEMM (gemv_mfma.hip) and the prefill GEMM (gemm.hip).
//
// A block is rebuilt exactly as an integer sum, I_i = sum_j t_j (z_{jC+i} - 2^15)
// (SeedLM: paperdance.org abstract; atlas.scime.ai "Approach"), and enters the
// MFMA as fp16(I_i * 2^(e-15) * 2^10) = fp16(w_i * 2^10): |w * 2^10| <= 32767,
// so nothing overflows, and the products are scaled back by 2^-10 afterwards.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace seedlm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

__device__ inline uint32_t ubfe(uint32_t v, uint32_t off, uint32_t w) {
  return __builtin_amdgcn_ubfe(v, off, w);
}

// 2^(g - 20) for g in [0, 15]: the block scale 2^(e - 15) = 2^(g - 30) times
// the fp16 range factor 2^10.
__device__ inline float block_scale(uint32_t g) { return __uint_as_float((g + 107u) << 23); }

// a * b + c for a, b within 24-bit signed range (a coefficient and a 16-bit
// window): one v_mad_i32_i24, which the compiler does not form by itself (it
// emits v_mul_i32_i24 and sums with v_add3_u32, two instructions more per
// weight).
__device__ inline int mad24(int a, int b, int c) {
  int d;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// The integer sums start from kMagic, the bits of the float 1.5 * 2^23: for
// |I| < 2^22 the bits of kMagic + I are the float 1.5 * 2^23 + I, exactly, so
// fma(bits as float, scale, -1.5 * 2^23 * scale) is I * scale before its one
// rounding, to fp16 -- the same value as converting I and scaling, in one
// instruction (v_fma_mixlo_f16) instead of a conversion and a multiply.
constexpr int kMagic = 0x4B400000;
constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23

// Stream bits 16..47 of a 4-bit block's seed from the two GF(2) byte tables.
__device__ inline uint32_t ext_c8(uint32_t w, const uint32_t* T0, const uint32_t* T1) {
  return T0[w & 0xFFu] ^ T1[(w >> 8) & 0xFFu];
}

// Eight fp16 weights (x 2^10) of a 4-bit block, in column order, given its
// stream bits 16..47.
__device__ inline half8 decode_c8_ext(uint32_t w, uint32_t ext) {
  const uint32_t lo = (w & 0xFFFFu) | (ext << 16);             // stream bits 0..31
  const int t0 = ((int)(w << 12)) >> 28;
  const int t1 = ((int)(w << 8)) >> 28;
  const int t2 = ((int)(w << 4)) >> 28;
  const int base = kMagic - 32768 * (t0 + t1 + t2);
  const float sc = block_scale(w >> 28);
  const float off = -kMagicF * sc;
  half8 out;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int z0 = (int)ubfe(lo, i, 16);       // z_i
    const int z1 = (int)ubfe(lo, 8 + i, 16);   // z_{8+i}
    const int z2 = (int)ubfe(ext, i, 16);      // z_{16+i}
    const int I = mad24(t2, z2, mad24(t1, z1, mad24(t0, z0, base)));
    out[i] = (_Float16)__builtin_fmaf(__int_as_float(I), sc, off);
  }
  return out;
}

// Eight fp16 weights (x 2^10) of a 4-bit block, in column order.
__device__ inline half8 decode_c8(uint32_t w, const uint32_t* T0, const uint32_t* T1) {
  return decode_c8_ext(w, ext_c8(w, T0, T1));
}

// Decode state of a 3-bit block: its stream bits 0..63, coefficients, the
// offset term and the scale.  dec12_quad then produces the weights four at a
// time, so that a caller can spread one block's decode over other work.
struct Dec12 {
  uint32_t s0, s1, s2;  // stream bits 0..31, 16..47, 32..63
  int t[4];
  int base;             // kMagic - 2^15 (t0 + t1 + t2 + t3)
  float sc;
  float off;            // -1.5 * 2^23 * sc
};

__device__ inline Dec12 dec12_setup(uint32_t w, uint32_t g, const uint64_t* T0,
                                    const uint64_t* T1) {
  Dec12 d;
  const uint64_t ext = T0[w & 0xFFu] ^ T1[(w >> 8) & 0xFFu];  // stream bits 16..79
  d.s0 = (w & 0xFFFFu) | ((uint32_t)ext << 16);
  d.s1 = (uint32_t)ext;
  d.s2 = (uint32_t)(ext >> 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) d.t[j] = ((int)(w << (12 - 4 * j))) >> 28;
  d.base = kMagic - 32768 * (d.t[0] + d.t[1] + d.t[2] + d.t[3]);
  d.sc = block_scale(g);
  d.off = -kMagicF * d.sc;
  return d;
}

// Ties a block's decode state to this point of the program: the compiler must
// assume the stream words, offset and scale change here, so weights computed
// from them are not moved above it (and the scheduler can interleave them with
// the MFMAs that follow).  The coefficients stay out of it, so that the
// compiler still knows they are 4-bit and multiplies with v_mul_i32_i24.
// Emits no instruction.
__device__ inline void dec12_pin(Dec12& d) {
  asm volatile("" : "+v"(d.s0), "+v"(d.s1), "+v"(d.s2), "+v"(d.base), "+v"(d.sc));
}

typedef _Float16 half4 __attribute__((ext_vector_type(4)));

// fp16 weights I0 .. I0+3 (x 2^10) of a decoded block, lowest column in the low
// 16 bits.
template <int I0>
__device__ inline uint64_t dec12_quad(const Dec12& d) {
  half4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = I0 + k;
    int I = d.base;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 12 * j + i;  // state index, window b[n .. n+15]
      const int z = n <= 16 ? (int)ubfe(d.s0, n, 16)
                            : (n <= 32 ? (int)ubfe(d.s1, n - 16, 16) : (int)ubfe(d.s2, n - 32, 16));
      I = mad24(d.t[j], z, I);
    }
    o[k] = (_Float16)__builtin_fmaf(__int_as_float(I), d.sc, d.off);
  }
  return __builtin_bit_cast(uint64_t, o);
}

}  // namespace seedlm
