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
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short2v __attribute__((ext_vector_type(2)));

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
// fma(bits as float, scale, -1.5 * 2^23 * scale) is I * scale, exact in fp32
// (the scale is a power of two); its conversion to fp16 is the one rounding.
// That is one FMA per weight in place of a conversion and a multiply.  (The
// fused v_fma_mixlo/hi_f16, one instruction per weight instead of 1.5, made
// the batch-8 layer step 6% slower in an interleaved A/B, so the conversion
// stays a separate pack.)
constexpr int kMagic = 0x4B400000;
constexpr float kMagicF = 12582912.0f;  // 1.5 * 2^23

typedef _Float16 half2x __attribute__((ext_vector_type(2)));

// The fp16 pair (I0 * sc, I1 * sc) of two magic-offset integer sums.
__device__ inline uint32_t to_f16_pair(int I0, int I1, float sc, float off) {
  half2x h;
  h[0] = (_Float16)__builtin_fmaf(__int_as_float(I0), sc, off);
  h[1] = (_Float16)__builtin_fmaf(__int_as_float(I1), sc, off);
  return __builtin_bit_cast(uint32_t, h);
}

// The GF(2) byte tables of the 4-bit decode hold their 32 extension bits
// rotated by 16 (the XOR of two rotated words is the rotated XOR), so that
// one word is both halves a block needs: its high half completes stream bits
// 0..31 beside the seed, and its low half is stream bits 32..47, the high word
// of every v_alignbit below (which reads only its low i < 8 bits).
template <typename Ext>
__device__ inline Ext c8_table_word(Ext e) {
  if constexpr (sizeof(Ext) == 4) return (e >> 16) | (e << 16);
  else return e;
}

// Stream bits 16..47 of a 4-bit block's seed, rotated by 16, from the tables.
__device__ inline uint32_t ext_c8(uint32_t w, const uint32_t* T0, const uint32_t* T1) {
  return T0[w & 0xFFu] ^ T1[(w >> 8) & 0xFFu];
}

// Eight fp16 weights (x 2^10) of a 4-bit block, in column order, given its
// stream bits 16..47 rotated by 16 (ext_c8).  Weight i needs the windows z_i, z_{8+i} and z_{16+i}
// (bits i.., 8+i.., 16+i.. of the stream, 16 each).  V = stream bits i..i+31
// (one v_alignbit) holds z_i in its low half and z_{16+i} in its high half;
// XOR with 0x80008000 turns both into z - 2^15 as signed 16-bit values, so one
// v_dot2_i32_i16 against (t0, t2) adds t0 (z_i - 2^15) + t2 (z_{16+i} - 2^15)
// to the middle term t1 z_{8+i} (bits 8..23 of V, one bfe and one mad24 onto
// kMagic - 2^15 t1).  Five integer instructions per weight instead of six
// (three bfe, three mad24); 4% off the batch-8 layer step in an interleaved
// A/B, with identical results.
__device__ inline half8 decode_c8_ext(uint32_t w, uint32_t ext) {
  // stream bits 0..31: the seed, then the rotated word's high half (one v_perm_b32)
  const uint32_t lo = __builtin_amdgcn_perm(ext, w, 0x07060100u);
  const uint32_t hi = ext;  // stream bits 32..47 in its low half
  const int t0 = ((int)(w << 12)) >> 28;
  const int t1 = ((int)(w << 8)) >> 28;
  const int t2 = ((int)(w << 4)) >> 28;
  const short2v t02 = short2v{(short)t0, (short)t2};
  const int base = mad24(t1, -32768, kMagic);
  // 2^(g - 20) and -1.5 * 2^23 * 2^(g - 20) as two v_ldexp_f32 of g = w >> 28
  const int g = (int)(w >> 28);
  const float sc = __builtin_amdgcn_ldexpf(0x1p-20f, g);
  const float off = __builtin_amdgcn_ldexpf(-kMagicF * 0x1p-20f, g);
  int I[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t V = i == 0 ? lo : __builtin_amdgcn_alignbit(hi, lo, i);
    const int mid = mad24(t1, (int)ubfe(V, 8, 16), base);
    I[i] = __builtin_amdgcn_sdot2(__builtin_bit_cast(short2v, V ^ 0x80008000u), t02, mid, false);
  }
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = to_f16_pair(I[2 * k], I[2 * k + 1], sc, off);
  return __builtin_bit_cast(half8, o);
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
  d.s0 = __builtin_amdgcn_perm((uint32_t)ext, w, 0x05040100u);  // seed, ext bits 0..15
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

// fp16 weights I0 .. I0+3 (x 2^10) of a decoded block, lowest column in the low
// 16 bits.
template <int I0>
__device__ inline uint64_t dec12_quad(const Dec12& d) {
  int I[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = I0 + k;
    I[k] = d.base;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 12 * j + i;  // state index, window b[n .. n+15]
      const int z = n <= 16 ? (int)ubfe(d.s0, n, 16)
                            : (n <= 32 ? (int)ubfe(d.s1, n - 16, 16) : (int)ubfe(d.s2, n - 32, 16));
      I[k] = mad24(d.t[j], z, I[k]);
    }
  }
  const uint64_t lo = to_f16_pair(I[0], I[1], d.sc, d.off);
  const uint64_t hi = to_f16_pair(I[2], I[3], d.sc, d.off);
  return lo | (hi << 32);
}

}  // namespace seedlm
