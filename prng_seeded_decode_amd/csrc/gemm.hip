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
//           T = 512 (or 256 when 512-token tiles would leave over half the CUs
//           idle);
//   K step  32 columns = 4 blocks = one 16-byte group of a packed row;
//   waves   2 x 2: wave (wr, wt) owns rows r0 + 64 wr .. +63 and tokens
//           t0 + (T/2) wt .. +T/2-1, i.e. 2 x T/64 MFMA tiles of 32 x 32 (up to
//           256 fp32 accumulators per lane), up to 32 MFMAs per K step.
// Per K step each thread loads one 16-byte group (4 blocks) of one row into
// registers and copies 8 x 16 bytes of X straight into LDS, two steps ahead;
// the decode of step k+1 and the MFMAs of step k use different LDS buffers, so
// the matrix cores run while the VALU decodes.
//
// MFMA operand layout (v_mfma_f32_32x32x16_f16, wave64): lane l supplies the 8
// K values 8*(l/32) .. 8*(l/32)+7 of A row l%32 and of B column l%32; the
// 32 x 32 fp32 result gives lane l column l%32, rows 8g + 4(l/32) + v in
// register 4g + v (g, v = 0..3).  A = W rows, B = X tokens, so the result is
// Y^T: lane l holds token l%32 and runs of four consecutive rows.
#include <hip/hip_fp16.h>

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
constexpr int kXRow = kStepCols * 2;                // bytes per token row of an X tile
constexpr int kXChunks = kXRow / 16;                // 16-byte chunks per token row
constexpr int kLdsStride = kStepCols * 2 + 16;      // bytes per W row in LDS (padded)
constexpr int kWBytes = kTileRows * kLdsStride;     // 10 KiB
static_assert(kXChunks == 4, "X tile layout");

// Token tile: 512 (256 per wave, 256 accumulator registers) for long inputs,
// 256 when 512-token tiles would leave more than half the compute units idle.
template <int TOKS>
struct TokTile {
  static constexpr int kTileToks = TOKS;
  static constexpr int kNTiles = TOKS / 2 / 32;     // 32-token MFMA tiles per wave
  static constexpr int kXBytes = TOKS * kXRow;      // swizzled, no padding
  static constexpr int kXCopies = kXBytes / 1024 / 4;  // 1 KiB LDS copies per wave per step
};

struct GemmArgs {
  const uint32_t* words;
  const __half* x;
  __half* y;
  int rows, cols, Mp, nb, ntok;
  uint32_t words_bytes, x_bytes;  // buffer sizes (< 2^31)
};

// Chunk swizzle of the X tiles (see copy_x); depends on token bits 1..3 only.
__device__ inline int xswz(int t) { return (((t >> 1) ^ (t >> 3)) & 1) | (((t >> 2) & 1) << 1); }

template <int TOKS>
__global__ void __launch_bounds__(kGemmThreads, 1) gemm_c8_kernel(const GemmArgs a) {
  constexpr int kTileToks = TokTile<TOKS>::kTileToks, kNTiles = TokTile<TOKS>::kNTiles;
  constexpr int kXBytes = TokTile<TOKS>::kXBytes, kXCopies = TokTile<TOKS>::kXCopies;
  // Three buffers of each kind, as separate objects indexed at compile time, so
  // that the compiler can tell that reads of one never wait for copies into
  // another.
  __shared__ uint32_t T0[256], T1[256];
  __shared__ __attribute__((aligned(16))) uint8_t w0[kWBytes], w1[kWBytes], w2[kWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t x0[kXBytes], x1[kXBytes], x2[kXBytes];
  uint8_t* const wbuf[3] = {w0, w1, w2};
  uint8_t* const xbuf[3] = {x0, x1, x2};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wt = wave & 1;
  const int r0 = blockIdx.x * kTileRows, t0 = blockIdx.y * kTileToks;

  for (int e = tid; e < 512; e += kGemmThreads) {
    const uint32_t u = (uint32_t)e & 255u;
    if (e < 256) T0[u] = ext_bits<uint32_t>(u);
    else T1[u] = ext_bits<uint32_t>(u << 8);
  }

  // This thread's share of a K step: row dr = tid / 2 of the tile, whose step
  // is one 16-byte group (4 blocks) of the packed row; the two threads of a
  // row decode its words 2h and 2h+1 (h = tid & 1).  Buffer loads: an
  // out-of-range offset reads zeros, so no load is conditional and steps past
  // the end simply load zeros.
  const int dr = tid >> 1, h = tid & 1;
  const int row = r0 + dr;
  const int nsteps = (a.nb + 3) / 4;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.words, 0, (int)a.words_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, (int)a.x_bytes, 0x00020000);
  auto load_w = [&](int ks) -> uint4 {
    const int b0 = ks * 4;  // first block of the group
    const int p = b0 / kPanelBlocks;
    const int Wps = (int)panel_stored_width(p, a.nb);
    const int q0 = b0 - p * kPanelBlocks;
    // zero words decode to t = 0
    const uint32_t off = (row < a.Mp && q0 < Wps)
                             ? (uint32_t)((p * a.Mp * kPanelBlocks + row * Wps + q0) * 4)
                             : 0x80000000u;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // X of a step goes straight into LDS (buffer_load ... lds, 16 bytes per
  // lane): the tile is T tokens x 64 bytes, and 16-byte chunk c of token t sits
  // at t*64 + ((c ^ f(t)) * 16) with f(t) = ((t>>1 ^ t>>3) & 1) | (t>>2 & 1) << 1.
  // Tokens with equal t mod 4 (equal bank offset t*64 within 256 bytes) get
  // distinct chunk positions over any 16 consecutive tokens, and tokens with
  // equal t mod 2 over any 8, so operand reads are free of bank conflicts
  // whether 16 lanes share 64 banks or 8 lanes share 32.  Wave w, copy i fills
  // LDS pieces P = (kXCopies w + i) * 64 + lane.
  auto copy_x = [&](int ks, uint8_t* dst) {
#pragma unroll
    for (int i = 0; i < kXCopies; ++i) {
      const int P = (kXCopies * wave + i) * 64 + lane;
      const int tok = P >> 2, c = (P & 3) ^ xswz(tok);
      const int col = ks * kStepCols + 8 * c;
      const uint32_t off = (t0 + tok < a.ntok && col < a.cols)
                               ? (uint32_t)((t0 + tok) * a.cols + col) * 2u
                               : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (__attribute__((address_space(3))) void*)(dst + (kXCopies * wave + i) * 1024), 16,
          off, 0, 0, 0);
    }
  };
  // Decode word p of a step's group into a W buffer: it holds block
  // (p + row) & 3 of the step (the packed rows rotate their groups).
  auto put_w1 = [&](uint8_t* dst, uint32_t w, uint32_t ext, int p) {
    const int slot = (p + row) & 3;
    *reinterpret_cast<half8*>(dst + dr * kLdsStride + slot * 16) = decode_c8_ext(w, ext);
  };
  auto mine = [&](uint4 wq, int j) -> uint32_t {  // word 2h + j of the group
    return h ? (j ? wq.w : wq.z) : (j ? wq.y : wq.x);
  };
  auto put_w = [&](uint8_t* dst, uint4 wq) {
#pragma unroll
    for (int j = 0; j < 2; ++j) put_w1(dst, mine(wq, j), ext_c8(mine(wq, j), T0, T1), 2 * h + j);
  };

  f32x16 acc[2][kNTiles];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int n = 0; n < kNTiles; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[g][n][v] = 0.f;

  const int arow = lane & 31, kq = lane >> 5, swz = xswz(arow);
  // MFMAs of one step: operands of slice s (16 columns) read one slice ahead;
  // after slice s's MFMAs, this thread's word s of the next step's group is
  // decoded, and the scheduler is told to alternate one MFMA with a few VALU
  // instructions, so that the decode issues while the matrix cores work.
  auto mma = [&](const uint8_t* wb, const uint8_t* xb, uint8_t* wnext, uint4 wq) {
    uint32_t ext2[2];  // table lookups of both words, issued with slice 0's reads
#pragma unroll
    for (int j = 0; j < 2; ++j) ext2[j] = ext_c8(mine(wq, j), T0, T1);
    const uint8_t* wl = wb + (64 * wr + arow) * kLdsStride + kq * 16;
    const uint8_t* xl = xb + (kTileToks / 2 * wt + arow) * kXRow;
    half8 A[2][2], B[2][kNTiles];
    auto rd = [&](int s) {
      const int xo = ((2 * s + kq) ^ swz) * 16;
#pragma unroll
      for (int g = 0; g < 2; ++g)
        A[s & 1][g] = *reinterpret_cast<const half8*>(wl + g * 32 * kLdsStride + s * 32);
#pragma unroll
      for (int n = 0; n < kNTiles; ++n)
        B[s & 1][n] = *reinterpret_cast<const half8*>(xl + n * 32 * kXRow + xo);
    };
    rd(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
      if (s + 1 < kSlices) rd(s + 1);
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int n = 0; n < kNTiles; ++n)
          acc[g][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[s & 1][g], B[s & 1][n], acc[g][n],
                                                             0, 0, 0);
      put_w1(wnext, mine(wq, s), ext2[s], 2 * h + s);
      // LDS reads first (the next slice's operands), then MFMAs alternating
      // with VALU, then the decode's store.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + kNTiles, 0);
#pragma unroll
      for (int m = 0; m < 2 * kNTiles; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then up to six VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      __builtin_amdgcn_sched_barrier(0);  // slices stay in order
    }
  };

  // Prologue: steps 0 and 1 in flight, step 0 decoded.
  uint4 wr3[3];
  copy_x(0, xbuf[0]);
  wr3[0] = load_w(0);
  copy_x(1, xbuf[1]);
  wr3[1] = load_w(1);
  __syncthreads();  // T0/T1 ready (waits for all loads too)
  put_w(wbuf[0], wr3[0]);
  __syncthreads();

  // Step k (buffers k % 3): start the copies of step k + 2, run the MFMAs of
  // step k, decode step k + 1, then wait until only step k + 2's nine loads are
  // in flight (vmcnt counts in issue order) and meet at the barrier.
  auto step = [&](int k, int b) {
    const int b1 = b == 2 ? 0 : b + 1, b2 = b == 0 ? 2 : b - 1;
    copy_x(k + 2, xbuf[b2]);
    wr3[b2] = load_w(k + 2);
    mma(wbuf[b], xbuf[b], wbuf[b1], wr3[b1]);
    __builtin_amdgcn_s_waitcnt(0x0079);  // vmcnt(9) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  };
  // Whole rounds of three steps (one loop exit, so the accumulators keep their
  // registers); the at most two steps past the end multiply zeros.
  for (int ks = 0; ks < nsteps; ks += 3) {
    step(ks, 0);
    step(ks + 1, 1);
    step(ks + 2, 2);
  }

  // Y[t][r]: lane holds token 32n + l%32 and rows 32g + 8j + 4(l/32) + v.
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int n = 0; n < kNTiles; ++n) {
      const int tok = t0 + kTileToks / 2 * wt + 32 * n + arow;
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
// workgroups.
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
  int rows, cols, Mp, nb, ntok;
  uint32_t buf_bytes, exp_off, x_bytes;  // packed buffer size, exponent array offset, X size
};

template <int ROWS, int TOKS>
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
  const int r0 = blockIdx.x * ROWS, t0 = blockIdx.y * TOKS;

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
  const int nsteps = (a.nb + 3) / 4;
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.words, 0, (int)a.buf_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, (int)a.x_bytes, 0x00020000);
  struct Group {
    uint4 w;
    uint32_t e;  // the group's exponent nibbles
  };
  auto load_w = [&](int ks) -> Group {
    const int b0 = ks * 4;
    const int p = b0 / kPanelBlocks;
    const int Wps = (int)panel_stored_width(p, a.nb);
    const int q0 = b0 - p * kPanelBlocks;
    const bool ok = row < a.Mp && q0 < Wps;
    const uint32_t off = ok ? (uint32_t)((p * a.Mp * kPanelBlocks + row * Wps + q0) * 4)
                            : 0x80000000u;
    const uint32_t eoff =
        ok ? a.exp_off + (uint32_t)((p * a.Mp * (kPanelBlocks / 4) + row * (Wps / 4) + q0 / 4) * 2)
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

  // Prologue: the words and X of steps 0 and 1 in flight; step 0 decoded.
  Group gq[3];
  gq[0] = load_w(0);
  gq[1] = load_w(1);
  copy_x(0, xbuf[0]);
  copy_x(1, xbuf[1]);
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
  // Whole rounds of three steps (one loop exit); steps past the end multiply
  // zeros.
  for (int ks = 0; ks < nsteps; ks += 3) {
    step(ks, 0);
    step(ks + 1, 1);
    step(ks + 2, 2);
  }

  // Y[t][r]: lane holds token 32n + l%32 and rows 32g + 8j + 4(l/32) + v.
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

template <int ROWS, int TOKS>
void launch_c12(const Gemm12Args& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.rows + ROWS - 1) / ROWS), (unsigned)((a.ntok + TOKS - 1) / TOKS));
  hipLaunchKernelGGL((gemm_c12_kernel<ROWS, TOKS>), grid, dim3(2 * ROWS), 0, s, a);
}

}  // namespace

int launch_gemm(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, int xdt, int ydt,
                hipStream_t s) {
  if (xdt != SEEDLM_F16 || ydt != SEEDLM_F16) return SEEDLM_E_UNSUPPORTED;
  // token tiles go on grid.y, which holds at most 65535 workgroups
  if ((ntok + 255) / 256 > 65535) return SEEDLM_E_UNSUPPORTED;
  if (h->C == 12) {
    if (h->cols % 8 != 0 || (uintptr_t)x % 16 != 0) return SEEDLM_E_UNSUPPORTED;
    if (h->bytes >= (1ULL << 31) || ntok * h->cols * 2 >= (1LL << 31)) return SEEDLM_E_UNSUPPORTED;
    Gemm12Args a{static_cast<const uint32_t*>(h->d_buf), static_cast<const __half*>(x),
                 static_cast<__half*>(y), (int)h->rows, (int)h->cols, (int)h->Mp, (int)h->nb,
                 (int)ntok, (uint32_t)h->bytes, (uint32_t)h->exp_off, (uint32_t)(ntok * h->cols * 2)};
    // 256 x 256 tiles where they give every compute unit a workgroup
    const int64_t big = ((h->rows + 255) / 256) * ((ntok + 255) / 256);
    if (big >= device_cu_count()) launch_c12<256, 256>(a, s);
    else launch_c12<128, 256>(a, s);
    SEEDLM_HIP_CHECK(hipGetLastError());
    return SEEDLM_OK;
  }
  if (h->C != 8) return SEEDLM_E_UNSUPPORTED;
  if (h->cols % 8 != 0 || (uintptr_t)x % 16 != 0) return SEEDLM_E_UNSUPPORTED;
  // 32-bit buffer offsets: the packed words and X must each stay below 2 GiB.
  if (h->nwords * 4 >= (1LL << 31) || ntok * h->cols * 2 >= (1LL << 31))
    return SEEDLM_E_UNSUPPORTED;
  GemmArgs a{static_cast<const uint32_t*>(h->d_buf), static_cast<const __half*>(x),
             static_cast<__half*>(y), (int)h->rows, (int)h->cols, (int)h->Mp, (int)h->nb,
             (int)ntok, (uint32_t)(h->nwords * 4), (uint32_t)(ntok * h->cols * 2)};
  const int64_t row_tiles = (h->rows + kTileRows - 1) / kTileRows;
  // 512-token tiles once they fill at least half of the compute units (each
  // does twice the MFMA work per decoded weight); 256-token tiles below that.
  if (2 * row_tiles * ((ntok + 511) / 512) >= device_cu_count()) {
    const dim3 grid((unsigned)row_tiles, (unsigned)((ntok + 511) / 512));
    hipLaunchKernelGGL(gemm_c8_kernel<512>, grid, dim3(kGemmThreads), 0, s, a);
  } else {
    const dim3 grid((unsigned)row_tiles, (unsigned)((ntok + 255) / 256));
    hipLaunchKernelGGL(gemm_c8_kernel<256>, grid, dim3(kGemmThreads), 0, s, a);
  }
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
