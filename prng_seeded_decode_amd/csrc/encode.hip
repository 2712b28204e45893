// seedlm_encode: exhaustive seed search on the matrix cores.
//
// SeedLM compresses a block w of C weights by finding, over every K-bit seed s,
// the P coefficients and the shared exponent that bring 2^e U(s) t closest to w,
// and storing the best seed with them (atlas.scime.ai "Approach").  The
// pseudo-inverses of all seeds are computed once and cached, and the error
// minimisation runs in parallel over blocks and seeds (paperhub.cn rebuttal on
// compression cost).  For one seed the score is fixed as follows: least squares
// t* = pinv(U) w; e = the smallest exponent in [-15, 0] at which every
// round-half-even(t*_j / 2^e) lies in [-8, 7] (e = 0 if none does);
// t = clamp(round-half-even(t* / 2^e), -8, 7); score ||w - 2^e U t||^2.  The
// lowest score wins, the smaller seed on ties.
//
// How the kernels get there.  Per seed, U = Q R is a thin QR factorisation (Q
// is C x P with orthonormal columns, R is upper triangular); seed_table_kernel
// builds it once per encoder in fp64 (pinv(U) = R^-1 Q^T).  Then for any w
//   c = Q^T w,   t* = R^-1 c,   ||w||^2 - ||c||^2 = least-squares residual,
//   ||w - U tau||^2 = (||w||^2 - ||c||^2) + ||c - R tau||^2        (Pythagoras)
// The least-squares residual is a lower bound on the score of every
// quantisation, so a seed whose residual is not below the block's best score so
// far cannot win and is dropped after three FMAs; only the rest (well under one
// seed in a thousand on Gaussian blocks) is quantised and scored.  The score is
// computed as residual + ||c - R tau||^2, which in fp32 can never come out
// below the residual (rounding is monotone), so the dropping is exact for the
// kernel's own arithmetic: the result is the exhaustive minimum of its fp32
// scores.
//
// c = Q^T w for 16 seeds x 16 blocks is one MFMA per column j of Q:
// v_mfma_f32_16x16x32_bf16 with A = the 16 seeds' column j (rows = seeds) and
// B = 16 blocks (columns = blocks).  Weights come in as bf16, exact in the
// operand.  Each Q entry is stored as the sum of three bf16 parts (hi + mid +
// lo, about 24 significant bits) laid out along K, with the block's weights
// repeated along K to match, so every product is exact and the sum is
// accumulated in fp32.  For C = 8 the three parts fill K slots 0..23 of one
// MFMA; for C = 12 hi and mid fill slots 0..23 of a 16x16x32 MFMA and lo slots
// 0..11 of a v_mfma_f32_16x16x16_bf16, whose result is added on the VALU.  K
// slots 24..31 (lanes 48..63) carry zero weights, so whatever finite A values
// those lanes hold do not matter.
//
// Operand layout (wave64): lane l supplies K slots 8*(l/16) .. 8*(l/16)+7
// (4*(l/16) .. +3 for the 16x16x16 form) of A row l%16 and of B column l%16;
// the result gives lane l rows 4*(l/16)+v (v = 0..3) of column l%16.  So lane
// l sees block (l%16) of the tile against seeds 4*(l/16) .. 4*(l/16)+3.
//
// Work split: a wave owns kTiles tiles of 16 consecutive blocks for the whole
// search and keeps, per block, the best score, seed and record in registers;
// the four lanes that share a block merge their bests after every tile step in
// which any of them improved.  A workgroup (8 waves) streams the seed table
// through LDS in stages of a few 16-seed tiles, double-buffered, one barrier per
// stage; two workgroups share a CU (four waves per SIMD).
#include <hip/hip_runtime.h>

#include "seedlm_internal.h"

namespace seedlm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kEncThreads = 512;  // 8 waves

// The K-bit LFSR: z' = (z >> 1) | (f << (K - 1)), f the XOR of a few bits of z
// (characteristic polynomials x^12 + x^6 + x^4 + x + 1, x^16 + x^5 + x^3 +
// x^2 + 1 -- the format's -- and x^20 + x^3 + 1, all primitive).
template <int K>
__device__ inline uint32_t lfsr_next(uint32_t z) {
  static_assert(K == 12 || K == 16 || K == 20, "seed widths");
  uint32_t f;
  if constexpr (K == 12) f = z ^ (z >> 1) ^ (z >> 4) ^ (z >> 6);
  else if constexpr (K == 16) f = z ^ (z >> 2) ^ (z >> 3) ^ (z >> 5);
  else f = z ^ (z >> 3);
  return (z >> 1) | ((f & 1u) << (K - 1));
}

// A format: C weights per block, P coefficients per block, K-bit seeds, Q-bit
// coefficients.  The two packed formats, (8,3) and (12,4) with K = 16 and
// Q = 4, keep their tuned work split; the others serve the design-space study
// (records only).
template <int C, int P, int K, int Q>
struct EncFmt {
  static_assert(C >= 2 && C <= 12 && P >= 1 && P <= 7 && P < C, "supported formats");
  static_assert(Q == 3 || Q == 4, "coefficients fit a nibble");
  static constexpr int kSeedTiles = (1 << K) / 16;  // seeds 1 .. 2^K (2^K is padding)
  static constexpr int kLastSeed = (1 << K) - 1;
  // Q's three bf16 parts along K: all in one 16x16x32 MFMA when 3C <= 32, else
  // hi and mid there and lo in a 16x16x16 MFMA.
  static constexpr bool kSplit = 3 * C > 32;
  static constexpr int kSlots = kSplit ? 2 * C : 3 * C;  // used K slots of the 32-wide operand
  static constexpr int kGroups = (kSlots + 7) / 8;       // lane groups (8 slots each) holding them
  // Table columns store 48 lanes when lane group 3 is unused (lanes 48..63
  // then re-read lanes 0..15: finite values against zero weights), else 64.
  static constexpr int kALanes = kGroups == 4 ? 64 : 48;
  static constexpr int kQBytes = kALanes * 16 + (kSplit ? 48 * 8 : 0);  // one column j of a tile
  static constexpr bool kPacked83 = C == 8 && P == 3 && K == 16 && Q == 4;
  static constexpr int kTiles = kPacked83 ? 8 : (P >= 6 ? 2 : 4);  // block tiles per wave
  static constexpr int kStage = kPacked83 ? 8 : 4;   // seed tiles per LDS stage
};

template <int C, int P, int K, int Q>
struct EncLayout {
  using F = EncFmt<C, P, K, Q>;
  static constexpr int NR = P * (P + 1) / 2;           // entries of an upper triangle
  static constexpr int kRBytes = 2 * NR * 4;           // R^-1 then R, fp32, per seed
  static constexpr int kROff = P * F::kQBytes;         // R data of the 16 seeds of a tile
  static constexpr int kTileBytes = (kROff + 16 * kRBytes + 255) / 256 * 256;
  static constexpr int kStageBytes = F::kStage * kTileBytes;
  static constexpr int kStages = F::kSeedTiles / F::kStage;
  static constexpr int kChunks = kStageBytes / 16;     // 16-byte pieces per stage
  static constexpr int kChunksPerThread = (kChunks + kEncThreads - 1) / kEncThreads;
  static constexpr int kBlocksPerWave = 16 * F::kTiles;
  static constexpr int kBlocksPerGroup = (kEncThreads / 64) * kBlocksPerWave;
  static_assert(kChunks % 64 == 0, "a stage splits into whole 1 KiB wave pieces");
  static_assert(F::kSeedTiles % F::kStage == 0 && kStages % 2 == 0, "stages alternate");
};

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline double bf16_value(uint16_t h) {
  return (double)__uint_as_float((uint32_t)h << 16);
}

// One thread per seed: U(s) from the LFSR, thin QR by Gram-Schmidt with one
// re-orthogonalisation pass (fp64), R^-1 by back substitution; Q's columns go
// out as three bf16 parts each in the MFMA operand layout, R^-1 and R as fp32
// upper triangles (row-major).  Seed 2^K (padding of the last tile) gets
// zeros; the search never accepts it.
template <int C, int P, int K, int Q>
__global__ void __launch_bounds__(256) seed_table_kernel(uint8_t* __restrict__ table) {
  using L = EncLayout<C, P, K, Q>;
  using F = EncFmt<C, P, K, Q>;
  constexpr int NR = L::NR;
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= 16 * F::kSeedTiles) return;
  const int seed = m + 1, tile = m >> 4, n = m & 15;
  double Qm[C][P], R[P][P], Ri[P][P];
  for (int i = 0; i < P; ++i)
    for (int j = 0; j < P; ++j) R[i][j] = Ri[i][j] = 0.0;
  if (seed <= F::kLastSeed) {
    uint32_t z = (uint32_t)seed;
    for (int k = 0; k < C * P; ++k) {  // column-major fill: U[i][j] = v_{jC+i}
      Qm[k % C][k / C] = ((double)z - (double)(1 << (K - 1))) / (double)(1 << (K - 1));
      z = lfsr_next<K>(z);
    }
    for (int j = 0; j < P; ++j) {
      for (int pass = 0; pass < 2; ++pass)
        for (int k = 0; k < j; ++k) {
          double r = 0.0;
          for (int i = 0; i < C; ++i) r += Qm[i][k] * Qm[i][j];
          for (int i = 0; i < C; ++i) Qm[i][j] -= r * Qm[i][k];
          R[k][j] += r;
        }
      double nn = 0.0;
      for (int i = 0; i < C; ++i) nn += Qm[i][j] * Qm[i][j];
      R[j][j] = sqrt(nn);
      for (int i = 0; i < C; ++i) Qm[i][j] /= R[j][j];
    }
    for (int i = P - 1; i >= 0; --i) {
      Ri[i][i] = 1.0 / R[i][i];
      for (int j = i + 1; j < P; ++j) {
        double s = 0.0;
        for (int k = i; k < j; ++k) s += Ri[i][k] * R[k][j];
        Ri[i][j] = -s / R[j][j];
      }
    }
  } else {
    for (int i = 0; i < C; ++i)
      for (int j = 0; j < P; ++j) Qm[i][j] = 0.0;
  }
  uint8_t* tb = table + (size_t)tile * L::kTileBytes;
  for (int j = 0; j < P; ++j) {
    uint16_t part[3][C];
    for (int i = 0; i < C; ++i) {
      const double q = Qm[i][j];
      part[0][i] = bf16_bits((float)q);
      const double r1 = q - bf16_value(part[0][i]);
      part[1][i] = bf16_bits((float)r1);
      const double r2 = r1 - bf16_value(part[1][i]);
      part[2][i] = bf16_bits((float)r2);
    }
    uint8_t* col = tb + j * F::kQBytes;
    // K slot k (< kSlots) of the 32-wide operand holds part k / C, entry k % C
    // (hi, mid and, unless split, lo); the rest is zero.
    for (int qg = 0; qg < F::kALanes / 16; ++qg) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(col + (16 * qg + n) * 16);
      for (int u = 0; u < 8; ++u) {
        const int k = 8 * qg + u;
        dst[u] = k < F::kSlots ? part[k / C][k % C] : (uint16_t)0;
      }
    }
    if (F::kSplit) {  // lo part: K slots 0..C-1 of the 16-wide operand
      for (int qg = 0; qg < 3; ++qg) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(col + F::kALanes * 16 + (16 * qg + n) * 8);
        for (int u = 0; u < 4; ++u) {
          const int k = 4 * qg + u;
          dst[u] = k < C ? part[2][k] : (uint16_t)0;
        }
      }
    }
  }
  float* rd = reinterpret_cast<float*>(tb + L::kROff + n * L::kRBytes);
  int o = 0;
  for (int i = 0; i < P; ++i)
    for (int j = i; j < P; ++j, ++o) {
      rd[o] = (float)Ri[i][j];
      rd[NR + o] = (float)R[i][j];
    }
}

struct EncArgs {
  const uint8_t* table;
  const uint16_t* W;  // bf16 bits, [rows][cols]
  int64_t nblk;       // rows * nbr
  int64_t cols, nbr;  // columns, blocks per row (ceil(cols / C))
  void* seeds;  // uint16 for K <= 16, uint32 above
  int8_t* coeffs;
  int8_t* exps;
  float* err;  // may be null
};

// The block's weights as the B operand(s) of the MFMAs, and its squared norm.
// 32-wide operand: K slot k < kSlots holds w[k % C] (against Q's parts), lane
// group qg holding slots 8qg .. 8qg+7; 16-wide operand (split formats): slot
// k < C holds w[k] (against lo), lane group qg holding slots 4qg .. 4qg+3.
template <int C, int P, int K, int Q>
struct BlockOps {
  using F = EncFmt<C, P, K, Q>;
  bf16x8 b1;
  s16x4 b2;
  // Block b of a [rows][cols] matrix: row b / nbr, columns (b % nbr) * C ..;
  // a row's last block may be short (cols not a multiple of C), and its
  // missing weights are read as zeros.
  __device__ void load(const uint16_t* W, int64_t b, bool valid, int64_t cols, int64_t nbr,
                       int qg, float& wn) {
    uint16_t x[C];
    if (cols % C == 0) {
      if constexpr (C == 8) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (valid) v = *reinterpret_cast<const uint4*>(W + b * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
      } else {
#pragma unroll
        for (int i = 0; i < C; ++i) x[i] = valid ? W[b * C + i] : (uint16_t)0;
      }
    } else {
      const int64_t r = valid ? b / nbr : 0;
      const int64_t c0 = (b - r * nbr) * C;
      const int64_t n = valid ? cols - c0 : 0;  // weights present (may exceed C)
#pragma unroll
      for (int i = 0; i < C; ++i) x[i] = i < n ? W[r * cols + c0 + i] : (uint16_t)0;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const float xf = __uint_as_float((uint32_t)x[i] << 16);
      s = fmaf(xf, xf, s);
    }
    wn = s;
    auto pick = [&](int k, int nslots, int per, int u) -> uint32_t {
      // slot per*qg + u of this lane, the lane group known only at run time
      uint32_t val = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = per * q + u;
        const uint32_t c = kk < nslots ? (uint32_t)x[kk % C] : 0u;
        if (qg == q) val = c;
      }
      (void)k;
      return val;
    };
    uint32_t w1[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      w1[h] = pick(0, F::kSlots, 8, 2 * h) | (pick(0, F::kSlots, 8, 2 * h + 1) << 16);
    b1 = __builtin_bit_cast(bf16x8, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    if constexpr (F::kSplit) {
      const uint32_t lo0 = pick(0, C, 4, 0) | (pick(0, C, 4, 1) << 16);
      const uint32_t lo1 = pick(0, C, 4, 2) | (pick(0, C, 4, 3) << 16);
      b2 = __builtin_bit_cast(s16x4, make_uint2(lo0, lo1));
    } else {
      b2 = s16x4{0, 0, 0, 0};
    }
  }
};

// t_j as nibbles at bits 4j (P <= 7), e + 15 at bits 28..31.
template <int P>
__device__ inline uint32_t pack_record(const float (&t)[P], int e) {
  uint32_t r = (uint32_t)(e + 15) << 28;
#pragma unroll
  for (int j = 0; j < P; ++j) r |= ((uint32_t)(int)t[j] & 15u) << (4 * j);
  return r;
}

template <int C, int P, int K, int Q>
__global__ void __launch_bounds__(kEncThreads, 4) encode_kernel(const EncArgs a) {
  using L = EncLayout<C, P, K, Q>;
  using F = EncFmt<C, P, K, Q>;
  constexpr int NR = L::NR, NT = F::kTiles, G = F::kStage;
  // Two stage buffers as separate objects, so that the compiler can tell that
  // reads of one never wait for the copy into the other.
  __shared__ __attribute__((aligned(16))) uint8_t stage0[L::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[L::kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, qg = lane >> 4;
  const int64_t block0 = ((int64_t)blockIdx.x * (kEncThreads / 64) + wave) * L::kBlocksPerWave;

  BlockOps<C, P, K, Q> ops[NT];
  float nwn[NT], best[NT];
  int bseed[NT];
  uint32_t brec[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int64_t b = block0 + 16 * T + n;
    float wn;
    ops[T].load(a.W, b, b < a.nblk, a.cols, a.nbr, qg, wn);
    nwn[T] = -wn;
    best[T] = __builtin_inff();
    bseed[T] = 0;
    brec[T] = 0u;
  }

  // Stage st of the table (bytes st*kStageBytes ..) is copied straight into LDS
  // (global_load_lds, 16 bytes per lane: wave w's lanes fill 1 KiB pieces
  // r*kEncThreads + 64w .. +63), one stage ahead of its use; the barrier after
  // each stage waits for the copy.
  auto fetch = [&](int st, uint8_t* dst) {
    const uint8_t* src = a.table + (size_t)st * L::kStageBytes;
#pragma unroll
    for (int r = 0; r < L::kChunksPerThread; ++r) {
      const int c0 = r * kEncThreads + 64 * wave;  // wave-uniform
      if (c0 < L::kChunks)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(src + (size_t)(c0 + lane) * 16),
            (__attribute__((address_space(3))) void*)(dst + c0 * 16), 16, 0, 0);
    }
  };

  // lanes 48..63 re-read lanes 0..15 when lane group 3 is unused (their B is zero)
  const int alane = F::kALanes == 64 ? lane : lane % 48;
  auto run_stage = [&](const uint8_t* sb, int st) {
    for (int s = 0; s < G; ++s) {
      const uint8_t* tb = sb + s * L::kTileBytes;
      bf16x8 A1[P];
      s16x4 A2[P];
#pragma unroll
      for (int j = 0; j < P; ++j) {
        A1[j] = *reinterpret_cast<const bf16x8*>(tb + j * F::kQBytes + alane * 16);
        if constexpr (F::kSplit)
          A2[j] = *reinterpret_cast<const s16x4*>(tb + j * F::kQBytes + F::kALanes * 16 +
                                                  (lane % 48) * 8);
      }
      const int seed_base = (st * G + s) * 16 + 1 + 4 * qg;  // seed of this lane's row v = 0
      // c = Q^T w for this seed tile against block tile T.
      auto tile_acc = [&](int T, f32x4 (&acc)[P]) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[j], ops[T].b1, zero, 0, 0, 0);
          if constexpr (F::kSplit) {
            // The lo part gets an accumulator of its own: chaining this MFMA onto
            // the 16x16x32 result (a different opcode) read a stale accumulator
            // when the two were issued back to back, and the compiler does not
            // separate them.
            const f32x4 lo = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A2[j], ops[T].b2, zero, 0, 0, 0);
            acc[j] += lo;
          }
        }
      };
      // -(least-squares residual) = ||c||^2 - ||w||^2, as one fixed FMA chain.
      auto neg_residual = [&](int T, const f32x4 (&acc)[P], int v) {
        float s2 = fmaf(acc[0][v], acc[0][v], nwn[T]);
#pragma unroll
        for (int j = 1; j < P; ++j) s2 = fmaf(acc[j][v], acc[j][v], s2);
        return s2;
      };
      // Pass 1, the hot loop: one flag bit per block tile, set when some seed's
      // residual is below the block's best score.  No branch between tiles, so
      // one tile's MFMAs overlap the previous tile's arithmetic.
      uint32_t flags = 0;  // wave-uniform: bit T set when any lane of tile T has a candidate
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        f32x4 acc[P];
        tile_acc(T, acc);
        float m = neg_residual(T, acc, 0);
#pragma unroll
        for (int v = 1; v < 4; ++v) m = fmaxf(m, neg_residual(T, acc, v));
        if (__builtin_amdgcn_ballot_w64(m > -best[T])) flags |= 1u << T;
      }
      if (flags == 0) continue;
      // Pass 2 (rare): the flagged tiles again (same MFMAs, same values), each
      // candidate seed quantised and scored.
#pragma unroll
      for (int T = 0; T < NT; ++T) {
        if (!((flags >> T) & 1u)) continue;
        f32x4 acc[P];
        tile_acc(T, acc);
        bool improved = false;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float Lv = neg_residual(T, acc, v);
          const bool cand = Lv > -best[T];
          if (!__builtin_amdgcn_ballot_w64(cand)) continue;
          const int seed = seed_base + v;
          const float* rd =
              reinterpret_cast<const float*>(tb + P * F::kQBytes + (4 * qg + v) * L::kRBytes);
          float Ri[NR], Rm[NR];
#pragma unroll
          for (int o = 0; o < NR; ++o) {
            Ri[o] = rd[o];
            Rm[o] = rd[NR + o];
          }
          float c[P], ts[P];
#pragma unroll
          for (int j = 0; j < P; ++j) c[j] = acc[j][v];
          // t* = R^-1 c (upper triangular, row-major packed)
          {
            int o = 0;
#pragma unroll
            for (int i = 0; i < P; ++i) {
              float sum = Ri[o] * c[i];
              ++o;
#pragma unroll
              for (int k = i + 1; k < P; ++k, ++o) sum = fmaf(Ri[o], c[k], sum);
              ts[i] = sum;
            }
          }
          float hi = ts[0], lo = ts[0];
#pragma unroll
          for (int j = 1; j < P; ++j) {
            hi = fmaxf(hi, ts[j]);
            lo = fminf(lo, ts[j]);
          }
          // Smallest e with hi * 2^-e < H - 1/2 and lo * 2^-e >= -(H + 1/2),
          // H = 2^(Q-1) (the range that rounds half-to-even into [-H, H-1]):
          // with hi = f 2^k, f in [0.5, 1), e = k - (Q-1) when f < 1 - 2^-Q,
          // else k - Q + 2; with -lo = g 2^k, e = k - Q when g <= 1/2 + 2^-(Q+1),
          // else k - Q + 1.  (Q = 4: 15/16 and 17/32.)
          constexpr float kH = (float)(1 << (Q - 1));
          int e_hi = -64, e_lo = -64;
          if (hi > 0.f) {
            int k;
            const float f = frexpf(hi, &k);
            e_hi = k - (Q - 1) + (f >= 1.f - 0.5f / kH ? 1 : 0);
          }
          if (lo < 0.f) {
            int k;
            const float g = frexpf(-lo, &k);
            e_lo = k - Q + (g > 0.5f + 0.25f / kH ? 1 : 0);
          }
          const int e = min(max(max(e_hi, e_lo), -15), 0);
          float t[P], tau[P];
#pragma unroll
          for (int j = 0; j < P; ++j) {
            t[j] = fminf(fmaxf(rintf(ldexpf(ts[j], -e)), -kH), kH - 1.f);
            tau[j] = ldexpf(t[j], e);
          }
          // score = residual + ||c - R tau||^2
          float q2 = 0.f;
          {
            int o = 0;
#pragma unroll
            for (int i = 0; i < P; ++i) {
              float d = c[i];
#pragma unroll
              for (int k = i; k < P; ++k, ++o) d = fmaf(-Rm[o], tau[k], d);
              q2 = fmaf(d, d, q2);
            }
          }
          const float score = fmaxf(q2 - Lv, 0.f);
          if (cand && seed <= F::kLastSeed && score < best[T]) {
            best[T] = score;
            bseed[T] = seed;
            brec[T] = pack_record<P>(t, e);
            improved = true;
          }
        }
        // Merge the four lanes that share the block (lane groups qg = 0..3),
        // needed only when one of them found a better seed.
        if (!__builtin_amdgcn_ballot_w64(improved)) continue;
#pragma unroll
        for (int off = 16; off <= 32; off *= 2) {
          const float ob = __shfl_xor(best[T], off);
          const int os = __shfl_xor(bseed[T], off);
          const uint32_t orc = (uint32_t)__shfl_xor((int)brec[T], off);
          if (ob < best[T] || (ob == best[T] && os < bseed[T])) {
            best[T] = ob;
            bseed[T] = os;
            brec[T] = orc;
          }
        }
      }
    }
  };

  static_assert(L::kStages % 2 == 0, "stages alternate between two buffers");
  fetch(0, stage0);
  __syncthreads();
  for (int st = 0; st < L::kStages; st += 2) {
    fetch(st + 1, stage1);
    run_stage(stage0, st);
    __syncthreads();
    if (st + 2 < L::kStages) fetch(st + 2, stage0);
    run_stage(stage1, st + 1);
    __syncthreads();
  }

  if (qg == 0) {
#pragma unroll
    for (int T = 0; T < NT; ++T) {
      const int64_t b = block0 + 16 * T + n;
      if (b >= a.nblk) continue;
      if constexpr (K <= 16) static_cast<uint16_t*>(a.seeds)[b] = (uint16_t)bseed[T];
      else static_cast<uint32_t*>(a.seeds)[b] = (uint32_t)bseed[T];
      a.exps[b] = (int8_t)((int)(brec[T] >> 28) - 15);
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const int nib = (int)((brec[T] >> (4 * j)) & 15u);
        a.coeffs[b * P + j] = (int8_t)(nib - ((nib & 8) << 1));
      }
      if (a.err) a.err[b] = best[T];
    }
  }
}

}  // namespace

// Formats the encoder is built for (C, P, K, Q): the two packed ones, then the
// rest of the 4-bit frontier ((K + QP + 4) / C = 4 at K = 16, Q = 4: (6,1) ..
// (12,7)), the 3-bit frontier (largest P within 3 bits), two more points at
// C = 8, and the frontiers at other seed widths (K = 12, 20) and with 3-bit
// coefficients.
#define SEEDLM_ENC_FORMATS(X)                                                     \
  X(8, 3, 16, 4) X(12, 4, 16, 4)                                                  \
  X(6, 1, 16, 4) X(7, 2, 16, 4) X(9, 4, 16, 4) X(10, 5, 16, 4) X(11, 6, 16, 4)    \
  X(12, 7, 16, 4) X(8, 1, 16, 4) X(9, 1, 16, 4) X(10, 2, 16, 4) X(11, 3, 16, 4)   \
  X(8, 2, 16, 4) X(8, 4, 16, 4)                                                   \
  X(7, 3, 12, 4) X(9, 3, 20, 4) X(8, 2, 12, 4) X(12, 3, 20, 4)                    \
  X(8, 4, 16, 3) X(10, 3, 16, 3)

bool encoder_format_supported(int C, int P, int K, int Q) {
#define X(c, p, k, q) if (C == c && P == p && K == k && Q == q) return true;
  SEEDLM_ENC_FORMATS(X)
#undef X
  return false;
}

size_t encoder_table_bytes(int C, int P, int K, int Q) {
#define X(c, p, k, q)                                                                  \
  if (C == c && P == p && K == k && Q == q)                                            \
    return (size_t)EncFmt<c, p, k, q>::kSeedTiles * EncLayout<c, p, k, q>::kTileBytes;
  SEEDLM_ENC_FORMATS(X)
#undef X
  return 0;
}

int launch_seed_table(int C, int P, int K, int Q, void* table, hipStream_t s) {
#define X(c, p, k, q)                                                                   \
  if (C == c && P == p && K == k && Q == q) {                                           \
    const dim3 grid(16 * EncFmt<c, p, k, q>::kSeedTiles / 256), block(256);             \
    hipLaunchKernelGGL((seed_table_kernel<c, p, k, q>), grid, block, 0, s,              \
                       static_cast<uint8_t*>(table));                                   \
    SEEDLM_HIP_CHECK(hipGetLastError());                                                \
    return SEEDLM_OK;                                                                   \
  }
  SEEDLM_ENC_FORMATS(X)
#undef X
  return SEEDLM_E_UNSUPPORTED;
}

int launch_encode(int C, int P, int K, int Q, const void* table, const void* W, int64_t rows,
                  int64_t cols, void* seeds, int8_t* coeffs, int8_t* exps, float* err,
                  hipStream_t s) {
  const int64_t nbr = (cols + C - 1) / C;
  const int64_t nblk = rows * nbr;
  EncArgs a{static_cast<const uint8_t*>(table), static_cast<const uint16_t*>(W), nblk, cols, nbr,
            seeds, coeffs, exps, err};
#define X(c, p, k, q)                                                                   \
  if (C == c && P == p && K == k && Q == q) {                                           \
    const int64_t per = EncLayout<c, p, k, q>::kBlocksPerGroup;                         \
    const int64_t groups = (nblk + per - 1) / per;                                      \
    if (groups > 0x7FFFFFFF) return SEEDLM_E_UNSUPPORTED;                               \
    hipLaunchKernelGGL((encode_kernel<c, p, k, q>), dim3((unsigned)groups),             \
                       dim3(kEncThreads), 0, s, a);                                     \
    SEEDLM_HIP_CHECK(hipGetLastError());                                                \
    return SEEDLM_OK;                                                                   \
  }
  SEEDLM_ENC_FORMATS(X)
#undef X
  return SEEDLM_E_UNSUPPORTED;
}

}  // namespace seedlm
