// Prefill-size decode-GEMM on the matrix cores: Y[t][r] = sum_c W[r][c] X[t][c]
// for any number of token rows t, fp16 X and Y, fp32 accumulation; 4-bit format
// (gemm_c8_kernel) and 3-bit format (gemm_c12_kernel, at the end of the file).
//
// SeedLM rebuilds the weights from each block's seed and coefficients where they
// are used (paperhub.cn rebuttal text before Eq. (1); atlas.scime.ai
// "Approach").  With many activation rows the rebuild is amortised over all of
// them: a workgroup decodes a 128-row x 32-column tile of W exactly (the integer
// block sum, entering as fp16(w * 2^10)) into LDS once, and its four waves
// contract it against a 512-token slice of X with v_mfma_f32_32x32x16_f16.
//
// Tiles (one workgroup = 256 threads = 4 waves):
//   rows    r0 .. r0+127 of W (output features), tokens t0 .. t0+T-1 of X,
//           T = 512 (256 for inputs of at most 256 tokens);
//   K step  32 columns = 4 blocks = one 16-byte group of a packed row;
//   waves   1 x 4: wave w owns all 128 rows and tokens t0 + (T/4) w .. +T/4-1,
//           i.e. 4 x T/128 MFMA tiles of 32 x 32 (up to 256 fp32 accumulators
//           per lane), up to 32 MFMAs per K step.  (Against 2 x 2 waves of
//           64 rows x T/2 tokens this reads 16 instead of 20 KiB of operands
//           per wave and step.)
// Per K step each thread loads one 16-byte group (4 blocks) of one row, two
// steps ahead, and decodes the previous one into a W buffer in LDS, which all
// four waves read.  X is read by one wave only, so it does not pass through
// LDS: each lane loads its own B operands (16 bytes per 32-token tile and
// slice) straight into registers, one step ahead, in two register sets.  The
// decode of step k+1 and the MFMAs of step k use different W buffers, so the
// matrix cores run while the VALU decodes.
//
// Work units: a call is cut into whole tiles and, where the tiles would not
// fill the last round of workgroups on the GPU (or a small matrix would not
// fill one), tiles whose K steps are split over several workgroups.  The whole
// tiles run in one launch, the split units in a second, which writes fp32
// partial tiles into scratch, and gemm_fixup_kernel adds each tile's
// partials in a fixed order (deterministic) and writes it.  The 3-bit kernel
// is split the same way.
//
// MFMA operand layout (v_mfma_f32_32x32x16_f16, wave64): lane l supplies the 8
// K values 8*(l/32) .. 8*(l/32)+7 of A row l%32 and of B column l%32; the
// 32 x 32 fp32 result gives lane l column l%32, rows 8g + 4(l/32) + v in
// register 4g + v (g, v = 0..3).  A = W rows, B = X tokens, so the result is
// Y^T: lane l holds token l%32 and runs of four consecutive rows.
#include <hip/hip_fp16.h>

#include <algorithm>

#include "lfsr_device.h"
#include "mfma_decode.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmThreads = 256;
constexpr int kTileRows = 128;
constexpr int kStepCols = 32;                       // 4 blocks of 8 columns, one 16-byte group
constexpr int kSlices = kStepCols / 16;             // MFMAs of K = 16 per step
constexpr int kLdsStride = kStepCols * 2 + 16;      // bytes per W row in LDS (padded)
constexpr int kWBytes = kTileRows * kLdsStride;     // 10 KiB
constexpr int kRG = kTileRows / 32;                 // 32-row MFMA tiles per wave
static_assert(kSlices == 2, "operand sets");

// Token tile: 512 tokens (128 per wave), or 256 for short inputs.
template <int TOKS>
struct TokTile {
  static constexpr int kTileToks = TOKS;
  static constexpr int kNTiles = TOKS / 4 / 32;  // 32-token MFMA tiles per wave
};

struct GemmArgs {
  const uint32_t* words;
  const __half* x;
  __half* y;
  float* part;  // partial tiles of the split units (kTileRows x T floats each)
  int rows, cols, Mp, nb, ntok;
  uint32_t words_bytes, x_bytes;  // buffer sizes (< 2^31)
  int row_tiles;  // tile t covers rows (t % row_tiles) * 128.., tokens (t / row_tiles) * T..
  int full;       // units 0 .. full-1 are whole tiles 0 .. full-1
  int splits;     // later units: tile full + v / splits, K part v % splits
  int split_steps;  // K steps per part
};

template <int TOKS, bool kSplit>
__global__ void __launch_bounds__(kGemmThreads, 1) gemm_c8_kernel(const GemmArgs a) {
  constexpr int kTileToks = TokTile<TOKS>::kTileToks, kNTiles = TokTile<TOKS>::kNTiles;
  __shared__ uint32_t T0[256], T1[256];
  // Three W buffers, as separate objects indexed at compile time, so that the
  // compiler can tell that reads of one never wait for writes into another.
  __shared__ __attribute__((aligned(16))) uint8_t w0[kWBytes], w1[kWBytes], w2[kWBytes];
  uint8_t* const wbuf[3] = {w0, w1, w2};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // This workgroup's unit: whole tile blockIdx.x (the K range a compile-time
  // whole, which keeps the loop's address arithmetic as simple as before
  // splitting existed: 4-5% faster than a runtime range), or, in a launch of
  // the split units, K steps [kb, ke) of tile full + slot / splits.
  const int nsteps = (a.nb + 3) / 4;
  int tile = (int)blockIdx.x, kb = 0, ke = nsteps;
  const int slot = (int)blockIdx.x;
  if constexpr (kSplit) {
    tile = a.full + slot / a.splits;
    kb = (slot % a.splits) * a.split_steps;
    ke = min(nsteps, kb + a.split_steps);
  }
  const int r0 = (tile % a.row_tiles) * kTileRows, t0 = (tile / a.row_tiles) * kTileToks;

  for (int e = tid; e < 512; e += kGemmThreads) {
    const uint32_t v = (uint32_t)e & 255u;
    if (e < 256) T0[v] = c8_table_word(ext_bits<uint32_t>(v));
    else T1[v] = c8_table_word(ext_bits<uint32_t>(v << 8));
  }

  // This thread's share of a K step: row dr = tid / 2 of the tile, whose step
  // is one 16-byte group (4 blocks) of the packed row; the two threads of a
  // row decode its words 2h and 2h+1 (h = tid & 1).  Buffer loads: an
  // out-of-range offset reads zeros, so no load is conditional and steps past
  // the matrix's end simply load zeros (zero words decode to t = 0).  A split
  // unit's steps are a whole number of pairs (below), so it multiplies no step
  // past its own part; the loads it issues ahead past the part are not used.
  const int dr = tid >> 1, h = tid & 1;
  const int row = r0 + dr;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.words, 0, (int)a.words_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, (int)a.x_bytes, 0x00020000);
  auto load_w = [&](int ks) -> uint4 {
    const int b0 = ks * 4;  // first block of the group
    const int p = b0 / kPanelBlocks;
    const int Wps = (int)panel_stored_width(p, a.nb, kPanelBlocks);
    const int q0 = b0 - p * kPanelBlocks;
    const uint32_t off = (row < a.Mp && q0 < Wps)
                             ? (uint32_t)((p * a.Mp * kPanelBlocks + row * Wps + q0) * 4)
                             : 0x80000000u;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // Decode word p of a step's group into a W buffer: it holds block
  // (p + row) & 3 of the step (the packed rows rotate their groups).
  auto put_w1 = [&](uint8_t* dst, uint32_t w, uint32_t ext, int p) {
    const int slot4 = (p + row) & 3;
    *reinterpret_cast<half8*>(dst + dr * kLdsStride + slot4 * 16) = decode_c8_ext(w, ext);
  };
  auto mine = [&](uint4 wq, int j) -> uint32_t {  // word 2h + j of the group
    return h ? (j ? wq.w : wq.z) : (j ? wq.y : wq.x);
  };
  auto put_w = [&](uint8_t* dst, uint4 wq) {
#pragma unroll
    for (int j = 0; j < 2; ++j) put_w1(dst, mine(wq, j), ext_c8(mine(wq, j), T0, T1), 2 * h + j);
  };

  f32x16 acc[kRG][kNTiles];
#pragma unroll
  for (int g = 0; g < kRG; ++g)
#pragma unroll
    for (int n = 0; n < kNTiles; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[g][n][v] = 0.f;

  const int arow = lane & 31, kq = lane >> 5;
  // B operands straight from X (no LDS: only this wave uses its tokens).  Lane
  // l takes token l % 32 of each of the wave's 32-token tiles and the columns
  // 16 s + 8 (l / 32) .. +7 of slice s of a step: one 16-byte load per tile and
  // slice.  Tokens past the input and columns past the matrix read zeros; the
  // column test is needed only in a step that reaches the last column (cols is
  // a multiple of 8, so a load never straddles a token row's end).  Staging X
  // in LDS with buffer_load ... lds, as an earlier version did, was up to 22%
  // slower below 2048 tokens, and at 2048 up to 9% slower (8192 x 8192) and
  // within 1% on the largest shapes.
  uint32_t xo[kNTiles];
#pragma unroll
  for (int n = 0; n < kNTiles; ++n) {
    const int tok = t0 + kTileToks / 4 * wave + 32 * n + arow;
    xo[n] = tok < a.ntok ? (uint32_t)tok * (uint32_t)a.cols * 2u + 16u * kq : 0x80000000u;
  }
  half8 XB[2][2][kNTiles];  // [register set][slice][token tile]
  auto load_b = [&](int ks, int set) {
    const bool whole = (ks + 1) * kStepCols <= a.cols;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) {
        uint32_t off = xo[n] + (uint32_t)(ks * kStepCols * 2 + s * 32);
        if (!whole && ks * kStepCols + 16 * s + 8 * kq >= a.cols) off = 0x80000000u;
        XB[set][s][n] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
      }
  };

  // A operands of slices 0 and 1 (read from the W buffer).  Set 1 carries a
  // step's slice 1 across the step's closing barrier: a step first issues the
  // reads of its slice 0 and runs the MFMAs of the previous step's slice 1
  // while they are in flight, then reads its slice 1 (used after the barrier)
  // while the MFMAs of its slice 0 run, so no MFMA waits on a read issued right
  // before it.  The first step's "previous slice" multiplies zeros.
  half8 A[2][kRG];
#pragma unroll
  for (int g = 0; g < kRG; ++g) A[1][g] = half8{};
#pragma unroll
  for (int n = 0; n < kNTiles; ++n) XB[1][1][n] = half8{};
  auto mfmas = [&](int aset, int bset, int s) {
#pragma unroll
    for (int g = 0; g < kRG; ++g)
#pragma unroll
      for (int n = 0; n < kNTiles; ++n)
        acc[g][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[aset][g], XB[bset][s][n], acc[g][n], 0, 0, 0);
  };
  // The scheduler is told to alternate one MFMA with up to six VALU
  // instructions (the decode of one word of the next step), then the decode's
  // store, so that the decode issues while the matrix cores work.
  auto interleave = [&]() {
#pragma unroll
    for (int m = 0; m < kRG * kNTiles; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
  };
  // The MFMAs of step ks (W buffer wb, B register set c) with the previous
  // step's slice 1 first, the B loads of step ks + 1 into the other set once
  // those MFMAs have read it, and the decode of step ks + 1 into wnext.
  auto mma = [&](const uint8_t* wb, uint8_t* wnext, uint4 wq, int ks, int c) {
    uint32_t ext2[2];  // table lookups of both words
#pragma unroll
    for (int j = 0; j < 2; ++j) ext2[j] = ext_c8(mine(wq, j), T0, T1);
    const uint8_t* wl = wb + arow * kLdsStride + kq * 16;
    auto rd = [&](int s) {
#pragma unroll
      for (int g = 0; g < kRG; ++g)
        A[s][g] = *reinterpret_cast<const half8*>(wl + g * 32 * kLdsStride + s * 32);
    };
    rd(0);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(1, 1 - c, 1);
    load_b(ks + 1, 1 - c);
    put_w1(wnext, mine(wq, 0), ext2[0], 2 * h);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    rd(1);
    mfmas(0, c, 0);
    put_w1(wnext, mine(wq, 1), ext2[1], 2 * h + 1);
    __builtin_amdgcn_sched_group_barrier(0x100, kRG, 0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Prologue: step kb's words and B operands and step kb+1's words in flight,
  // step kb decoded.
  uint4 wr3[3];
  wr3[0] = load_w(kb);
  wr3[1] = load_w(kb + 1);
  load_b(kb, 0);
  __syncthreads();  // T0/T1 ready
  put_w(wbuf[0], wr3[0]);
  __syncthreads();

  // Step k (W buffers (k - kb) % 3, B set (k - kb) % 2): load the words of
  // step k + 2, run the MFMAs of step k, decode step k + 1, then wait for this
  // thread's LDS work only (the compiler waits for each load where its
  // registers are used) and meet at the barrier.
  auto step = [&](int k, int b, int c) {
    const int b1 = b == 2 ? 0 : b + 1, b2 = b == 0 ? 2 : b - 1;
    wr3[b2] = load_w(k + 2);
    mma(wbuf[b], wbuf[b1], wr3[b1], k, c);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's W writes are done
    __builtin_amdgcn_s_barrier();
  };
  // An even number of steps (a padded step multiplies zeros): rounds of six,
  // the loop unit of three W buffers and two B register sets, with buffers
  // indexed at compile time and one loop exit, so the accumulators keep their
  // registers; then two or four more.  (Parts rounded to six steps made the
  // 1024-row projections 4% slower: a part of 32 steps ran 36.)
  const int kend = kb + ((ke - kb + 1) & ~1);
  int ks = kb;
  for (; ks + 6 <= kend; ks += 6) {
    step(ks, 0, 0);
    step(ks + 1, 1, 1);
    step(ks + 2, 2, 0);
    step(ks + 3, 0, 1);
    step(ks + 4, 1, 0);
    step(ks + 5, 2, 1);
  }
  if (ks < kend) {
    step(ks, 0, 0);
    step(ks + 1, 1, 1);
    if (ks + 2 < kend) {
      step(ks + 2, 2, 0);
      step(ks + 3, 0, 1);
    }
  }
  mfmas(1, 1, 1);  // the last step's slice 1 (an even count: the last step used set 1)

  // Lane holds token 32n + l%32 of its wave's T/4 and rows 32g + 8j + 4(l/32) + v.
  if constexpr (kSplit) {
    // Partial tile, token-major: element (token i, row r) at i * 128 + r.
    float* const dst = a.part + (int64_t)slot * kTileRows * kTileToks;
#pragma unroll
    for (int g = 0; g < kRG; ++g)
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) {
        const int i = kTileToks / 4 * wave + 32 * n + arow;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 32 * g + 8 * j + 4 * kq;
          *reinterpret_cast<float4*>(dst + i * kTileRows + r) =
              make_float4(acc[g][n][4 * j], acc[g][n][4 * j + 1], acc[g][n][4 * j + 2],
                          acc[g][n][4 * j + 3]);
        }
      }
  } else {
#pragma unroll
    for (int g = 0; g < kRG; ++g)
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) {
        const int tok = t0 + kTileToks / 4 * wave + 32 * n + arow;
        if (tok >= a.ntok) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rb = r0 + 32 * g + 8 * j + 4 * kq;
          __half* dst = a.y + (int64_t)tok * a.rows + rb;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (rb + v < a.rows) dst[v] = __float2half_rn(acc[g][n][4 * j + v] * 0x1p-10f);
        }
      }
  }
}

// Y of the split tiles (either format): tile full + q adds its `splits`
// partial tiles (ROWS x TOKS floats, token-major) in part order and writes
// fp16(sum * 2^-10).  A thread owns four consecutive rows of one token (one
// 16-byte load per partial).
struct FixupArgs {
  const float* part;
  __half* y;
  int rows, ntok, row_tiles, full, splits;
};

template <int ROWS, int TOKS>
__global__ void __launch_bounds__(256) gemm_fixup_kernel(const FixupArgs a) {
  constexpr int kPer = ROWS * TOKS / 4 / 256;  // workgroups per tile
  const int q = (int)blockIdx.x / kPer;
  const int idx = ((int)blockIdx.x % kPer) * 256 + (int)threadIdx.x;
  const int i = idx / (ROWS / 4), r = (idx % (ROWS / 4)) * 4;
  const int tile = a.full + q;
  const int tok = (tile / a.row_tiles) * TOKS + i, row = (tile % a.row_tiles) * ROWS + r;
  if (tok >= a.ntok) return;
  const float* src = a.part + (int64_t)q * a.splits * ROWS * TOKS + i * ROWS + r;
  float4 s = *reinterpret_cast<const float4*>(src);
  for (int k = 1; k < a.splits; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)k * ROWS * TOKS);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  __half* dst = a.y + (int64_t)tok * a.rows + row;
  const float o[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (row + v < a.rows) dst[v] = __float2half_rn(o[v] * 0x1p-10f);
}

// The 3-bit format (C = 12, P = 4): the same scheme with a K step of 48 columns
// (one 16-byte group = 4 blocks of 12).  X and W rows of a step are 96 bytes =
// 6 chunks of 16 in LDS, logical chunk c of row t at position (c + rot(t)) mod 6
// with rot(t) = bit 2 ^ bit 3 of t: rows t and t+4 then put a chunk in opposite
// halves of a 32-byte bank pair and rows t and t+8 or t+12 land 8 chunks
// apart, so 16 consecutive rows read one chunk from 16 distinct 16-byte bank
// groups (and any aligned 8 from 8 distinct ones of 128 bytes).
//
// Tiles: ROWS x TOKS per workgroup, two threads per W row (2 ROWS threads),
// waves in a (ROWS / 64) x 2 grid of 64 rows x TOKS / 2 tokens each.  The X
// slice of a step costs 96 TOKS bytes of copying and the decode 4 ROWS blocks,
// for the same MFMA work when ROWS TOKS is fixed: copying X is the scarcer of
// the two here, so large grids take 256 x 256 tiles (eight waves, two per
// SIMD) and smaller grids 128 x 256 (four waves), which leaves more
// workgroups.  Tiles past the last full round split their K steps as in the
// 4-bit kernel (the 1024-row k and v projections of a Llama-3-8B layer: 64
// tiles of 128 x 256 at 2048 tokens, run as 256 quarters).
//
// Pipeline over three buffers of each kind: in step k the word loads and the
// X copy of step k+2 are issued, the MFMAs of step k run, and the decode of
// step k+1 (into the next W buffer) is spread over them four weights at a
// time; one wait for step k+1's X copy and one barrier end the step.
// Each block's exponent nibble comes from the format's separate nibble array
// (one u16 per group of four blocks, in the order of the group's words).
constexpr int kStep12 = 48;                    // columns per K step
constexpr int kSlices12 = kStep12 / 16;        // MFMAs of K = 16 per step
constexpr int kRow12 = 96;                     // LDS bytes per X token row / W row

__device__ inline int rot12(int t) { return ((t >> 2) ^ (t >> 3)) & 1; }

template <int ROWS, int TOKS>
struct Tile12 {
  static constexpr int kThreads = 2 * ROWS;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kNTiles = TOKS / 2 / 32;                // 32-token MFMA tiles per wave
  static constexpr int kWBytes = ROWS * kRow12;
  static constexpr int kXBytes = TOKS * kRow12;
  static constexpr int kXCopies = kXBytes / 1024 / kWaves;     // 1 KiB LDS copies per wave per step
  static_assert(kXCopies * 1024 * kWaves == kXBytes, "X tile layout");
  static_assert(3 * (kWBytes + kXBytes) + 4096 <= 160 * 1024, "LDS");
};

struct Gemm12Args {
  const uint32_t* words;
  const __half* x;
  __half* y;
  float* part;  // partial tiles of the split units (ROWS x TOKS floats each)
  int rows, cols, Mp, nb, ntok;
  uint32_t buf_bytes, exp_off, x_bytes;  // packed buffer size, exponent array offset, X size
  int row_tiles, full, splits, split_steps;  // work units, as for the 4-bit kernel
};

template <int ROWS, int TOKS, bool kSplit>
__global__ void __launch_bounds__(2 * ROWS, 1) gemm_c12_kernel(const Gemm12Args a) {
  using TL = Tile12<ROWS, TOKS>;
  constexpr int kNTiles = TL::kNTiles, kXBytes = TL::kXBytes, kWBytes = TL::kWBytes;
  constexpr int kXCopies = TL::kXCopies, kThreads = TL::kThreads;
  __shared__ uint64_t T0[256], T1[256];
  __shared__ __attribute__((aligned(16))) uint8_t w0[kWBytes], w1[kWBytes], w2[kWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t x0[kXBytes], x1[kXBytes], x2[kXBytes];
  uint8_t* const wbuf[3] = {w0, w1, w2};
  uint8_t* const xbuf[3] = {x0, x1, x2};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wt = wave & 1;
  // This workgroup's unit: whole tile blockIdx.x, or (split launch) K steps
  // [kb, ke) of tile full + slot / splits, as in the 4-bit kernel.
  const int nsteps = (a.nb + 3) / 4;
  int tile = (int)blockIdx.x, kb = 0, ke = nsteps;
  const int slot = (int)blockIdx.x;
  if constexpr (kSplit) {
    tile = a.full + slot / a.splits;
    kb = (slot % a.splits) * a.split_steps;
    ke = min(nsteps, kb + a.split_steps);
  }
  const int r0 = (tile % a.row_tiles) * ROWS, t0 = (tile / a.row_tiles) * TOKS;

  for (int e = tid; e < 512; e += kThreads) {
    const uint32_t u = (uint32_t)e & 255u;
    if (e < 256) T0[u] = ext_bits<uint64_t>(u);
    else T1[u] = ext_bits<uint64_t>(u << 8);
  }

  // Row dr = tid / 2 of the tile; the two threads of a row decode its words 2h
  // and 2h+1 of the step's group.  Out-of-range offsets read zeros (zero words
  // decode to t = 0).
  const int dr = tid >> 1, h = tid & 1;
  const int row = r0 + dr;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.words, 0, (int)a.buf_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, (int)a.x_bytes, 0x00020000);
  struct Group {
    uint4 w;
    uint32_t e;  // the group's exponent nibbles
  };
  auto load_w = [&](int ks) -> Group {
    constexpr int PB = panel_blocks(12);
    const int b0 = ks * 4;
    const int p = b0 / PB;
    const int Wps = (int)panel_stored_width(p, a.nb, PB);
    const int q0 = b0 - p * PB;
    const bool ok = row < a.Mp && q0 < Wps;
    const uint32_t off = ok ? (uint32_t)((p * a.Mp * PB + row * Wps + q0) * 4) : 0x80000000u;
    const uint32_t eoff =
        ok ? a.exp_off + (uint32_t)((p * a.Mp * (PB / 4) + row * (Wps / 4) + q0 / 4) * 2)
           : 0x80000000u;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
    Group g;
    g.w = make_uint4(v[0], v[1], v[2], v[3]);
    g.e = __builtin_amdgcn_raw_buffer_load_b16(wrs, eoff, 0, 0);
    return g;
  };
  // X of a step straight into LDS: copy i of this wave fills the 16-byte pieces
  // P = (kXCopies wave + i) * 64 + lane, i.e. position P % 6 of token P / 6,
  // which holds chunk (P % 6 - rot(token)) mod 6.  The X offsets of the pieces
  // move by 96 bytes per step, so they are worked out once; xc = 8 * chunk is
  // the column inside the step (INT_MAX for tokens past the end).
  uint32_t xo[kXCopies];
  int xc[kXCopies];
#pragma unroll
  for (int i = 0; i < kXCopies; ++i) {
    const int P = (kXCopies * wave + i) * 64 + lane;
    const int tok = P / 6, pos = P - 6 * tok;
    const int c = pos >= rot12(tok) ? pos - rot12(tok) : pos + 5;
    const bool ok = t0 + tok < a.ntok;
    xo[i] = ok ? (uint32_t)((t0 + tok) * a.cols + 8 * c) * 2u : 0u;
    xc[i] = ok ? 8 * c : 0x7FFFFFFF;
  }
  const int xwave = __builtin_amdgcn_readfirstlane(kXCopies * wave);
  auto copy_x = [&](int ks, uint8_t* dst) {
    const int lim = a.cols - ks * kStep12;
#pragma unroll
    for (int i = 0; i < kXCopies; ++i) {
      const uint32_t off = xc[i] < lim ? xo[i] + (uint32_t)(ks * kStep12 * 2) : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void*)(dst + (xwave + i) * 1024), 16, off, 0, 0,
          0);
    }
  };
  // Word 2h + j of a group holds block (2h + j + row) & 3 of the step (rotated
  // groups); weights 4q .. 4q+3 of that block are logical bytes 24 slot + 8q of
  // the W row, stored as one 8-byte write at their rotated chunk.
  const int rd = rot12(dr);
  auto w_addr = [&](uint8_t* dst, int j, int q) -> uint64_t* {
    const int slot = (2 * h + j + dr) & 3;
    const int b = 24 * slot + 8 * q;
    int c = (b >> 4) + rd;
    c = c >= 6 ? c - 6 : c;
    return reinterpret_cast<uint64_t*>(dst + dr * kRow12 + c * 16 + (b & 15));
  };
  auto mine = [&](const Group& q, int j) -> uint32_t {  // word 2h + j of the group
    return h ? (j ? q.w.w : q.w.z) : (j ? q.w.y : q.w.x);
  };
  auto setup = [&](const Group& q, int j) {
    return dec12_setup(mine(q, j), q.e >> (8 * h + 4 * j) & 15u, T0, T1);
  };

  f32x16 acc[2][kNTiles];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int n = 0; n < kNTiles; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[g][n][v] = 0.f;

  // Operand reads: lane l takes A row / B token l % 32 and the 8 columns of
  // chunk 2s + l / 32 of slice s, at that row's rotated position.
  const int arow = lane & 31, kq = lane >> 5;
  int po[kSlices12];
#pragma unroll
  for (int s = 0; s < kSlices12; ++s) {
    const int c = 2 * s + kq + rot12(arow);
    po[s] = (c >= 6 ? c - 6 : c) * 16;
  }
  // MFMAs of one step, with the decode of the next step's two blocks spread
  // over the three slices (quads 0, 1 of block 0; quad 2 of block 0 and quad 0
  // of block 1; quads 1, 2 of block 1), alternating one MFMA with a few VALU
  // instructions.
  auto mma = [&](const uint8_t* wb, const uint8_t* xb, uint8_t* wnext, const Group& qn) {
    Dec12 d0 = setup(qn, 0);
    Dec12 d1 = setup(qn, 1);
    const uint8_t* wl = wb + (64 * wr + arow) * kRow12;
    const uint8_t* xl = xb + (TOKS / 2 * wt + arow) * kRow12;
    half8 A[2][2], B[2][kNTiles];
    auto rd_ops = [&](int s) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
        A[s & 1][g] = *reinterpret_cast<const half8*>(wl + g * 32 * kRow12 + po[s]);
#pragma unroll
      for (int n = 0; n < kNTiles; ++n)
        B[s & 1][n] = *reinterpret_cast<const half8*>(xl + n * 32 * kRow12 + po[s]);
    };
    rd_ops(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kSlices12; ++s) {
      if (s + 1 < kSlices12) rd_ops(s + 1);
      if (s < 2) dec12_pin(d0);
      if (s > 0) dec12_pin(d1);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int n = 0; n < kNTiles; ++n)
          acc[g][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[s & 1][g], B[s & 1][n], acc[g][n],
                                                             0, 0, 0);
      if (s == 0) {
        *w_addr(wnext, 0, 0) = dec12_quad<0>(d0);
        *w_addr(wnext, 0, 1) = dec12_quad<4>(d0);
      } else if (s == 1) {
        *w_addr(wnext, 0, 2) = dec12_quad<8>(d0);
        *w_addr(wnext, 1, 0) = dec12_quad<0>(d1);
      } else {
        *w_addr(wnext, 1, 1) = dec12_quad<4>(d1);
        *w_addr(wnext, 1, 2) = dec12_quad<8>(d1);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + kNTiles, 0);
#pragma unroll
      for (int m = 0; m < 2 * kNTiles; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 96 / (2 * kNTiles), 0);  // then VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
      __builtin_amdgcn_sched_barrier(0);  // slices stay in order
    }
  };

  // Prologue: the words and X of steps kb and kb+1 in flight; step kb decoded.
  Group gq[3];
  gq[0] = load_w(kb);
  gq[1] = load_w(kb + 1);
  copy_x(kb, xbuf[0]);
  copy_x(kb + 1, xbuf[1]);
  __syncthreads();  // T0/T1 ready (waits for all loads too)
  {
    const Dec12 d0 = setup(gq[0], 0);
    const Dec12 d1 = setup(gq[0], 1);
    *w_addr(wbuf[0], 0, 0) = dec12_quad<0>(d0);
    *w_addr(wbuf[0], 0, 1) = dec12_quad<4>(d0);
    *w_addr(wbuf[0], 0, 2) = dec12_quad<8>(d0);
    *w_addr(wbuf[0], 1, 0) = dec12_quad<0>(d1);
    *w_addr(wbuf[0], 1, 1) = dec12_quad<4>(d1);
    *w_addr(wbuf[0], 1, 2) = dec12_quad<8>(d1);
  }
  __syncthreads();

  // Step k (buffers b = k % 3, b1 = (k+1) % 3, b2 = (k+2) % 3): the word
  // loads of step k+2 into gq[b2] (whose words were decoded in step k-1) and
  // the X copy of step k+2 into xbuf[b2] (read in step k-1, before the last
  // barrier); MFMAs of step k with step k+1 decoded into wbuf[b1]; then wait
  // until step k+1's X copy has landed and meet at the barrier.  vmcnt counts
  // in issue order: the word loads go before the copy, so that the compiler's
  // own wait for the words decoded in step k+1 does not also wait for step
  // k+2's copy, and the final wait leaves only step k+2's loads in flight.
  auto step = [&](int k, int b) {
    const int b1 = b == 2 ? 0 : b + 1, b2 = b == 0 ? 2 : b - 1;
    gq[b2] = load_w(k + 2);
    __builtin_amdgcn_sched_barrier(0);
    copy_x(k + 2, xbuf[b2]);
    mma(wbuf[b], xbuf[b], wbuf[b1], gq[b1]);
    __builtin_amdgcn_s_waitcnt(0x0070 | (kXCopies + 2));  // vmcnt(kXCopies + 2) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  };
  // Whole rounds of three steps (one loop exit); steps past the matrix's end
  // multiply zeros, and a split unit's steps are whole rounds of its part.
  for (int ks = kb; ks < ke; ks += 3) {
    step(ks, 0);
    step(ks + 1, 1);
    step(ks + 2, 2);
  }

  // Lane holds token 32n + l%32 of its wave's half and rows 32g + 8j + 4(l/32) + v
  // of its wave's 64.
  if constexpr (kSplit) {
    // Partial tile, token-major: element (token i, row r) at i * ROWS + r.
    float* const dst = a.part + (int64_t)slot * ROWS * TOKS;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) {
        const int i = TOKS / 2 * wt + 32 * n + arow;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 64 * wr + 32 * g + 8 * j + 4 * kq;
          *reinterpret_cast<float4*>(dst + i * ROWS + r) =
              make_float4(acc[g][n][4 * j], acc[g][n][4 * j + 1], acc[g][n][4 * j + 2],
                          acc[g][n][4 * j + 3]);
        }
      }
  } else {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int n = 0; n < kNTiles; ++n) {
        const int tok = t0 + TOKS / 2 * wt + 32 * n + arow;
        if (tok >= a.ntok) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rb = r0 + 64 * wr + 32 * g + 8 * j + 4 * kq;
          __half* dst = a.y + (int64_t)tok * a.rows + rb;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (rb + v < a.rows) dst[v] = __float2half_rn(acc[g][n][4 * j + v] * 0x1p-10f);
        }
      }
  }
}

// How a launch is cut into work units.  Tiles past the last whole round of
// workgroups on the GPU (every tile, when a small matrix has fewer tiles than
// compute units) run as `splits` units each, over consecutive ranges of K
// steps, when they would otherwise leave at least half of the compute units
// idle in that round: 896 tiles of the 4-bit 28672 x 8192 matrix at 2048
// tokens run as 768 whole tiles and 256 half tiles (3.5 rounds of work instead
// of 4), the 32 tiles of a 1024 x 8192 matrix as 256 eighths.
constexpr int64_t kMaxSplits = 8;
constexpr int64_t kMinSplitSteps = 8;  // K steps per part, at least
struct Plan {
  int rows_tile, toks;  // tile: 128 x 512 or 128 x 256 (4-bit), 256 or 128 x 256 (3-bit)
  int64_t row_tiles, tiles, full, tail, splits, split_steps;
  int64_t units() const { return full + tail * splits; }
  size_t part_bytes() const {
    return (size_t)(tail * splits) * rows_tile * toks * sizeof(float);
  }
};
void split_tail(Plan& p, int64_t nsteps, int64_t unit) {
  p.full = p.tiles;
  p.tail = 0;
  p.splits = 1;
  p.split_steps = nsteps;
  const int64_t cus = device_cu_count();
  const int64_t rem = p.tiles % cus;
  if (rem > 0 && 2 * rem <= cus) {
    const int64_t sp = std::min(std::min(cus / rem, kMaxSplits), nsteps / kMinSplitSteps);
    if (sp >= 2) {
      // whole loop units per part: pairs of steps (4-bit), rounds of three (3-bit)
      p.split_steps = ((nsteps + sp - 1) / sp + unit - 1) / unit * unit;
      p.splits = (nsteps + p.split_steps - 1) / p.split_steps;  // no empty part
      p.tail = rem;
      p.full = p.tiles - rem;
    }
  }
}
Plan plan_for(const seedlm_matrix* h, int64_t ntok) {
  Plan p{};
  if (h->C == 8) {
    p.rows_tile = kTileRows;
    p.toks = ntok > 256 ? 512 : 256;
  } else {
    // 256 x 256 tiles where they give every compute unit a workgroup
    p.toks = 256;
    p.rows_tile = ((h->rows + 255) / 256) * ((ntok + 255) / 256) >= device_cu_count() ? 256 : 128;
  }
  p.row_tiles = (h->rows + p.rows_tile - 1) / p.rows_tile;
  p.tiles = p.row_tiles * ((ntok + p.toks - 1) / p.toks);
  split_tail(p, (h->nb + 3) / 4, h->C == 8 ? 2 : 3);
  return p;
}

FixupArgs fixup_args(const Plan& p, const float* part, void* y, const seedlm_matrix* h,
                     int64_t ntok) {
  return FixupArgs{part, static_cast<__half*>(y), (int)h->rows, (int)ntok, (int)p.row_tiles,
                   (int)p.full, (int)p.splits};
}

// Whole tiles, then the split units, then the additions of their partials.
template <int TOKS>
void launch_c8(const GemmArgs& a, const Plan& p, const FixupArgs& f, hipStream_t s) {
  if (p.full > 0)
    hipLaunchKernelGGL((gemm_c8_kernel<TOKS, false>), dim3((unsigned)p.full), dim3(kGemmThreads),
                       0, s, a);
  if (p.tail > 0) {
    hipLaunchKernelGGL((gemm_c8_kernel<TOKS, true>), dim3((unsigned)(p.tail * p.splits)),
                       dim3(kGemmThreads), 0, s, a);
    hipLaunchKernelGGL((gemm_fixup_kernel<kTileRows, TOKS>),
                       dim3((unsigned)(p.tail * (kTileRows * TOKS / 4 / 256))), dim3(256), 0, s, f);
  }
}
template <int ROWS, int TOKS>
void launch_c12(const Gemm12Args& a, const Plan& p, const FixupArgs& f, hipStream_t s) {
  if (p.full > 0)
    hipLaunchKernelGGL((gemm_c12_kernel<ROWS, TOKS, false>), dim3((unsigned)p.full),
                       dim3(2 * ROWS), 0, s, a);
  if (p.tail > 0) {
    hipLaunchKernelGGL((gemm_c12_kernel<ROWS, TOKS, true>), dim3((unsigned)(p.tail * p.splits)),
                       dim3(2 * ROWS), 0, s, a);
    hipLaunchKernelGGL((gemm_fixup_kernel<ROWS, TOKS>),
                       dim3((unsigned)(p.tail * (ROWS * TOKS / 4 / 256))), dim3(256), 0, s, f);
  }
}

}  // namespace

int check_gemm(const seedlm_matrix* h, const void* x, int64_t ntok, int xdt, int ydt) {
  if (xdt != SEEDLM_F16 || ydt != SEEDLM_F16) return SEEDLM_E_UNSUPPORTED;
  // the token limit of the earlier 2-D grids (65535 token tiles of 256), kept
  if ((ntok + 255) / 256 > 65535) return SEEDLM_E_UNSUPPORTED;
  if (!h->is_4bit() && !h->is_3bit()) return SEEDLM_E_UNSUPPORTED;
  if (h->cols % 8 != 0 || (uintptr_t)x % 16 != 0) return SEEDLM_E_UNSUPPORTED;
  // 32-bit buffer offsets: the packed buffer and X must each stay below 2 GiB.
  const int64_t packed = h->C == 12 ? (int64_t)h->bytes : h->nwords * 4;
  if (packed >= (1LL << 31) || ntok * h->cols * 2 >= (1LL << 31)) return SEEDLM_E_UNSUPPORTED;
  if (plan_for(h, ntok).units() >= (1LL << 31)) return SEEDLM_E_UNSUPPORTED;
  return SEEDLM_OK;
}

size_t gemm_scratch_bytes(const seedlm_matrix* h, int64_t ntok) {
  return plan_for(h, ntok).part_bytes();
}

int launch_gemm(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, float* part,
                hipStream_t s) {
  const Plan p = plan_for(h, ntok);
  if (p.part_bytes() > 0 && !part) return SEEDLM_E_INVALID;
  const FixupArgs f = fixup_args(p, part, y, h, ntok);
  if (h->C == 12) {
    const Gemm12Args a{static_cast<const uint32_t*>(h->d_buf), static_cast<const __half*>(x),
                       static_cast<__half*>(y), part, (int)h->rows, (int)h->cols, (int)h->Mp,
                       (int)h->nb, (int)ntok, (uint32_t)h->bytes, (uint32_t)h->exp_off,
                       (uint32_t)(ntok * h->cols * 2), (int)p.row_tiles, (int)p.full,
                       (int)p.splits, (int)p.split_steps};
    if (p.rows_tile == 256) launch_c12<256, 256>(a, p, f, s);
    else launch_c12<128, 256>(a, p, f, s);
  } else {
    const GemmArgs a{static_cast<const uint32_t*>(h->d_buf), static_cast<const __half*>(x),
                     static_cast<__half*>(y), part, (int)h->rows, (int)h->cols, (int)h->Mp,
                     (int)h->nb, (int)ntok, (uint32_t)(h->nwords * 4),
                     (uint32_t)(ntok * h->cols * 2), (int)p.row_tiles, (int)p.full,
                     (int)p.splits, (int)p.split_steps};
    if (p.toks == 512) launch_c8<512>(a, p, f, s);
    else launch_c8<256>(a, p, f, s);
  }
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
