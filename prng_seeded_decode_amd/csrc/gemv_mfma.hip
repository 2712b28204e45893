// Skinny decode-GEMM on the matrix cores: y[b][r] = sum_c W[r][c] x[b][c] for
// batch 2..16 (any batch works), both packed formats, fp16 x and fp16 y.
//
// SeedLM rebuilds each block's weights from its seed and coefficients right
// where they are used (paperhub.cn rebuttal text before Eq. (1); atlas.scime.ai
// "Approach").  With several activation vectors the rebuilt block is shared by
// all of them, so here every block is decoded exactly once, straight into the
// operand registers of v_mfma_f32_16x16x32_f16, and the batch dimension (padded
// to 16) is the MFMA's N.  The decode itself is the exact integer one of
// seedlm_decode: I_i = sum_j t_j (z_{jC+i} - 2^15), w_i = I_i 2^(e-15); it then
// enters the MFMA as fp16(w_i * 2^10) (|w * 2^10| <= 32767, so no overflow),
// and the result is scaled back by 2^-10.  fp16 weights bound this path to the
// fp16-output tolerance; fp32-output calls use the exact kernels.
//
// Operand layout of v_mfma_f32_16x16x32_f16 (wave64): lane l supplies 8
// consecutive k values of A row (l % 16) and of B column (l % 16), the k group
// being l / 16; the 16x16 fp32 result gives lane l rows 4*(l/16)+v, column l%16.
// A 4-bit block is 8 columns, so one lane decodes one block per MFMA; a 3-bit
// lane decodes the four blocks of its 16-byte load (48 weights) and feeds them
// to six MFMAs, 8 weights each.  Any assignment of blocks to k groups is a
// valid MFMA as long as A and B agree; B (x) is read from LDS to match.
//
// Rows: a row group is 16 rows {row0 + rho + 4i}; the packed layout rotates
// each 4-slot group by (row mod 4) = rho, which is the same for all 16 rows,
// so a k group holds the same block for every row and the shared B operand is
// right.  Two tilings: a wave runs four row groups over its own 64 rows
// (256-row tiles), or one row group, the four waves covering 64 rows
// (64-row tiles, four times the workgroups for matrices too small to fill
// the GPU otherwise).
//
// Work split: a workgroup (4 waves, 256 or 64 rows) takes a contiguous chunk
// of panels; chunks write fp32 partials and
// reduce_chunks_kernel adds them in a fixed order (deterministic).  With a
// single chunk the kernel writes y directly.  The partials live in scratch
// that the caller passes per matrix (chunks * batch * Mp floats).
#include <hip/hip_fp16.h>

#include "lfsr_device.h"
#include "mfma_decode.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerTile = kRowsPerWave * kWaves;
constexpr int kBatchPad = 16;

template <int C>
struct Fmt;
template <>
struct Fmt<8> {
  static constexpr int P = 3;
  static constexpr int kCols = 8 * kPanelBlocks;  // columns of a panel
  static constexpr int kStride = kCols + 8;       // LDS row stride of x (halves)
  using Ext = uint32_t;                           // stream bits 16..47
};
template <>
struct Fmt<12> {
  static constexpr int P = 4;
  static constexpr int kCols = 12 * kPanelBlocks;
  static constexpr int kStride = kCols + 8;
  using Ext = uint64_t;  // stream bits 16..79 (63 needed)
};

struct MfmaArgs {
  const uint32_t* words;
  const __half* x;
  float* partial;
  __half* y;
  uint32_t buf_bytes;  // whole packed buffer (words, then exponents)
  uint32_t exp_off;    // byte offset of the 3-bit exponent nibbles
  int rows, cols, Mp, nb, np, batch;
  int tiles, chunk_panels, chunks;
  int wg_begin;   // first workgroup of this matrix in its main launch
  int red_begin;  // first reduce workgroup (64 rows) of this matrix
};

// Up to kMaxMfmaGroup matrices share a launch: workgroups are numbered matrix
// after matrix (a matrix's own split is unchanged), so small matrices run
// beside large ones and the per-launch cost is paid once.
constexpr int kMaxMfmaGroup = 8;
struct MfmaGroup {
  MfmaArgs m[kMaxMfmaGroup];
  int n;
};

template <int C, int RW>
__global__ void __launch_bounds__(kThreads, 4)
gemv_mfma_kernel(const MfmaGroup grp) {
  static_assert(RW == 1 || RW == 4, "row groups per wave");
  using F = Fmt<C>;
  constexpr int kUnits = 2 * RW;             // units per panel and wave
  constexpr int kPU = RW == 1 ? 2 : 1;       // panels per unrolled loop body
  using Ext = typename F::Ext;
  __shared__ Ext T0[256], T1[256];
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][kBatchPad * F::kStride];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, q = lane >> 4;
  int mi = 0;
  while (mi + 1 < grp.n && (int)blockIdx.x >= grp.m[mi + 1].wg_begin) ++mi;
  const MfmaArgs& a = grp.m[mi];
  const int local = (int)blockIdx.x - a.wg_begin;
  const int tile = local % a.tiles;
  const int chunk = local / a.tiles;
  const int pa = chunk * a.chunk_panels;
  const int pb = min(a.np, pa + a.chunk_panels);
  // Row group rr of this wave: rows row0 + rho + 4 i, i = 0..15, with rho =
  // rr (four groups over 64 rows per wave) or the wave (one group per wave,
  // 64-row tiles); row0 is a multiple of 64, so rho = row mod 4.
  const int row0 = RW == 4 ? tile * 4 * kRowsPerWave + wave * kRowsPerWave : tile * 64;
  auto rho_of = [&](int rr) { return RW == 4 ? rr : wave; };
  const int64_t Mp = a.Mp;

  for (int e = tid; e < 512; e += kThreads) {
    const uint32_t u = (uint32_t)e & 255u;
    if (e < 256) T0[u] = c8_table_word(ext_bits<Ext>(u));
    else T1[u] = c8_table_word(ext_bits<Ext>(u << 8));
  }

  // x staging: thread t holds batch row t / 16 and the kPer consecutive panel
  // columns (t % 16) kPer ..; buffer loads read zeros for padding rows (an
  // out-of-range offset) and columns past the row's end are set to zero.
  // With cols a multiple of 8 the run is read with 16-byte loads, otherwise
  // two bytes at a time; pairs sit in 32-bit registers and go to LDS as
  // 16-byte writes.
  constexpr int kPer = F::kCols / 16;  // halves per thread
  static_assert(kThreads == 16 * kBatchPad && kPer % 8 == 0, "x staging layout");
  const int xb = tid >> 4, xc0 = (tid & 15) * kPer;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.x, 0, (int)((uint32_t)a.batch * (uint32_t)a.cols * 2u), 0x00020000);
  uint32_t xr[kPer / 2];
  const bool x16 = a.cols % 8 == 0;  // 16-byte aligned runs of 8 columns
  auto fetch_x = [&](int p) {
    const int col0 = p * F::kCols + xc0;
    const int lim = a.cols - col0;  // columns k < lim of this run lie inside the row
    const uint32_t base = xb < a.batch ? (uint32_t)(xb * a.cols + col0) * 2u : 0x80000000u;
    if (x16) {  // lim is then a multiple of 8: a run of 8 is wholly in or out
#pragma unroll
      for (int k = 0; k < kPer; k += 8) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(
            xrsrc, k < lim ? base + 2u * k : 0x80000000u, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[k / 2 + j] = v[j];
      }
      return;
    }
#pragma unroll
    for (int k = 0; k < kPer; k += 2) {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(
          xrsrc, k < lim ? base + 2u * k : 0x80000000u, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(
          xrsrc, k + 1 < lim ? base + 2u * (k + 1) : 0x80000000u, 0, 0);
      xr[k / 2] = (lo & 0xFFFFu) | (hi << 16);
    }
  };
  auto store_x = [&](int buf) {
    uint4* dst = reinterpret_cast<uint4*>(&xs[buf][xb * F::kStride + xc0]);
#pragma unroll
    for (int k = 0; k < kPer / 8; ++k)
      dst[k] = make_uint4(xr[4 * k], xr[4 * k + 1], xr[4 * k + 2], xr[4 * k + 3]);
  };
  fetch_x(pa);
  store_x(pa & 1);
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.words, 0, (int)a.buf_bytes, 0x00020000);
  floatx4 acc[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) acc[rr] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Load unit k = 2*rr + h of the 32-block step p: the 16-byte record group
  // (slots 4g .. 4g+3 of the step, g = 4h + q) of row row0 + rho + 4*i16, and
  // its exponent nibbles (3-bit).  A 4-bit step is one packed panel; a 3-bit
  // step is two packed 16-block panels, 2p and 2p + 1, and unit h reads group
  // q of panel 2p + h.  Units are loaded two ahead into a 4-slot ring; the
  // ring crosses step boundaries, and loads past the last step read zeros.
  auto unit_load = [&](int p, int k, v4u& wd, uint32_t& ev) {
    const int rho = rho_of(k >> 1), h = k & 1;
    const int r = row0 + rho + 4 * i16;
    if constexpr (C == 8) {
      const int g = 4 * h + q;
      const int Wp = (int)panel_stored_width(p, a.nb, kPanelBlocks);
      const bool ok = p < pb && r < a.Mp && 4 * g < Wp;
      const uint32_t off =
          ok ? (uint32_t)(((int64_t)p * Mp * kPanelBlocks + (int64_t)r * Wp + 4 * g) * 4)
             : 0x80000000u;
      wd = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      ev = 0u;
    } else {
      constexpr int PB = panel_blocks(12);
      const int pp = 2 * p + h;  // packed panel; past the last one Wp <= 0
      const int Wp = (int)panel_stored_width(pp, a.nb, PB);
      const bool ok = p < pb && r < a.Mp && 4 * q < Wp;
      const uint32_t off =
          ok ? (uint32_t)(((int64_t)pp * Mp * PB + (int64_t)r * Wp + 4 * q) * 4) : 0x80000000u;
      const uint32_t eoff =
          ok ? a.exp_off +
                   (uint32_t)(((int64_t)pp * Mp * (PB / 4) + (int64_t)r * (Wp / 4) + q) * 2)
             : 0x80000000u;
      wd = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      ev = __builtin_amdgcn_raw_buffer_load_b16(rsrc, eoff, 0, 0);
    }
  };
  auto unit_compute = [&](const _Float16* xp, int k, const v4u wd, uint32_t ev) {
    const int rr = k >> 1, rho = rho_of(rr), h = k & 1;
    const int g = 4 * h + q;  // slot group of this lane: slots 4g .. 4g+3
    if constexpr (C == 8) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        // word n of the group holds slot 4g + ((n + row) & 3), row = rho mod 4
        const int slot = 4 * g + ((n + rho) & 3);
        const half8 A = decode_c8(wd[n], T0, T1);
        const half8 B = *reinterpret_cast<const half8*>(xp + 8 * slot);
        acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[rr], 0, 0, 0);
      }
    } else {
      // The 48 weights of the four blocks in twelve quads of four; MFMA m takes
      // quads 2m and 2m+1 (quad qd = weights 4 (qd % 3) .. +3 of block qd / 3)
      // and the x columns of the same weights.  A block is set up when its
      // first quad is needed, so at most two block states are live.
      Dec12 d[2];
#pragma unroll
      for (int m = 0; m < 6; ++m) {
        u64x2 aq;
        half4 bq[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int qd = 2 * m + hh, n = qd / 3, qq = qd % 3;
          if (qq == 0) d[n & 1] = dec12_setup(wd[n], (ev >> (4 * n)) & 0xFu, T0, T1);
          aq[hh] = qq == 0 ? dec12_quad<0>(d[n & 1])
                           : (qq == 1 ? dec12_quad<4>(d[n & 1]) : dec12_quad<8>(d[n & 1]));
          // word n of the group holds slot 4g + ((n + row) & 3), row = rho mod 4
          const int slot = 4 * g + ((n + rho) & 3);
          bq[hh] = *reinterpret_cast<const half4*>(xp + 12 * slot + 4 * qq);
        }
        const half8 A = __builtin_bit_cast(half8, aq);
        const half8 B = __builtin_shufflevector(bq[0], bq[1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[rr], 0, 0, 0);
      }
    }
  };

  v4u ring[4];
  uint32_t eRing[4];
  unit_load(pa, 0, ring[0], eRing[0]);
  unit_load(pa, 1, ring[1], eRing[1]);
  // kPU panels per loop body, so that the ring slot of every unit is known at
  // compile time; a body's second panel is skipped when it lies past the chunk.
  for (int p0 = pa; p0 < pb; p0 += kPU) {
#pragma unroll
    for (int pu = 0; pu < kPU; ++pu) {
      const int p = p0 + pu;
      if (pu == 0 || p < pb) {
        if (p + 1 < pb) fetch_x(p + 1);  // lands while this panel computes
        const _Float16* xp = xs[p & 1] + i16 * F::kStride;
#pragma unroll
        for (int k = 0; k < kUnits; ++k) {
          const int kk = pu * kUnits + k, kn = k + 2;  // kk: unit index in the body
          unit_load(p + kn / kUnits, kn % kUnits, ring[(kk + 2) & 3], eRing[(kk + 2) & 3]);
          unit_compute(xp, k, ring[kk & 3], eRing[kk & 3]);
        }
        if (p + 1 < pb) {
          store_x((p + 1) & 1);
          __syncthreads();
        }
      }
    }
  }

  // Result: lane holds rows 4*q + v of each row group, batch column i16.
  const int b = i16;
  if (b < a.batch) {
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = row0 + rho_of(rr) + 4 * (4 * q + v);
        if (r < a.rows) {
          const float val = acc[rr][v] * 0x1p-10f;
          if (a.chunks == 1)
            a.y[(int64_t)b * a.rows + r] = __float2half_rn(val);
          else
            a.partial[((int64_t)chunk * a.batch + b) * Mp + r] = val;
        }
      }
    }
  }
}

// y[b][r] = sum over chunks c of partial[c][b][r] for the group's matrices
// that were split into chunks.  A workgroup owns 64 rows of one matrix and
// every batch column (lane = row, wave w takes columns w, w+4, ...) and adds a
// column's chunks in chunk order, up to 32 loads in flight: fixed order, so
// repeated calls give the same bits.  One workgroup per 64 rows instead of one
// per 64 rows and batch column (with the chunks split over the four waves) made
// the Llama-3-70B batch-8 step 1.9% shorter and the Llama-3-8B batch-16 step 7%.
__global__ void __launch_bounds__(256) reduce_chunks_kernel(const MfmaGroup grp) {
  int mi = 0;
  while (mi + 1 < grp.n && (int)blockIdx.x >= grp.m[mi + 1].red_begin) ++mi;
  const MfmaArgs& a = grp.m[mi];
  const int rows = a.rows, Mp = a.Mp, batch = a.batch, chunks = a.chunks;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = ((int)blockIdx.x - a.red_begin) * 64 + lane;
  const int rr = r < rows ? r : rows - 1;  // in-bounds load; no store below
  const int64_t cstride = (int64_t)batch * Mp;
  for (int b = wv; b < batch; b += 4) {
    const float* __restrict__ src = a.partial + (int64_t)b * Mp + rr;
    float s = 0.f;
    for (int c0 = 0; c0 < chunks; c0 += 32) {
      float v[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) v[k] = c0 + k < chunks ? src[(c0 + k) * cstride] : 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) s += v[k];
    }
    if (r < rows) a.y[(int64_t)b * rows + r] = __float2half_rn(s);
  }
}

}  // namespace

namespace {

// The split of one matrix: tiling (256-row tiles where they give about four
// workgroups per CU over the panels, 64-row tiles for smaller matrices) and
// panel chunks to reach that many workgroups.
int plan_mfma(const seedlm_matrix* h, const void* x, void* y, float* partial, int batch,
              MfmaArgs& a, bool& wide) {
  if (h->bytes >= 0x80000000ull || h->Mp >= (1 << 30) ||
      (int64_t)batch * h->cols * 2 >= (1LL << 31))
    return SEEDLM_E_UNSUPPORTED;
  a = MfmaArgs{};
  a.words = static_cast<const uint32_t*>(h->d_buf);
  a.x = static_cast<const __half*>(x);
  a.partial = partial;
  a.y = static_cast<__half*>(y);
  a.buf_bytes = (uint32_t)h->bytes;
  a.exp_off = (uint32_t)h->exp_off;
  a.rows = (int)h->rows;
  a.cols = (int)h->cols;
  a.Mp = (int)h->Mp;
  a.nb = (int)h->nb;
  a.np = (int)((h->nb + kPanelBlocks - 1) / kPanelBlocks);  // 32-block steps
  a.batch = batch;
  // Four workgroups per CU per matrix: on the Llama-3-70B layer at batch 8 one
  // or two per CU (fewer chunks and partials, longer workgroups) made the step
  // 5-12% slower and eight or sixteen 1% slower.
  const int64_t want = 4LL * device_cu_count();
  wide = ((h->Mp + kRowsPerTile - 1) / kRowsPerTile) * a.np >= want;
  const int tile_rows = wide ? kRowsPerTile : 64;
  a.tiles = (int)((h->Mp + tile_rows - 1) / tile_rows);
  int64_t chunks = (want + a.tiles - 1) / a.tiles;
  if (chunks < 1) chunks = 1;
  if (chunks > a.np) chunks = a.np;
  a.chunk_panels = (int)((a.np + chunks - 1) / chunks);
  a.chunks = (a.np + a.chunk_panels - 1) / a.chunk_panels;
  if ((int64_t)a.tiles * a.chunks >= (1LL << 30)) return SEEDLM_E_UNSUPPORTED;
  return SEEDLM_OK;
}

template <int C, int RW>
void launch_main(const MfmaGroup& g, int grid, hipStream_t s) {
  hipEvent_t e0, e1;
  main_launch_events(&e0, &e1);
  hipExtLaunchKernelGGL((gemv_mfma_kernel<C, RW>), dim3((unsigned)grid), dim3(kThreads), 0, s, e0,
                        e1, 0, g);
}

}  // namespace

int64_t mfma_partial_floats(const seedlm_matrix* h, int batch) {
  MfmaArgs a;
  bool wide;
  if (plan_mfma(h, nullptr, nullptr, nullptr, batch, a, wide) != SEEDLM_OK) return 0;
  return a.chunks == 1 ? 0 : (int64_t)a.chunks * batch * h->Mp;
}

int launch_gemv_mfma_group(const seedlm_matrix* const* hs, const void* const* xs,
                           void* const* ys, float* const* partials, int n, int batch, int xdt,
                           int ydt, hipStream_t s, int phases) {
  if (xdt != SEEDLM_F16 || ydt != SEEDLM_F16) return SEEDLM_E_UNSUPPORTED;
  if (batch < 1 || batch > kBatchPad) return SEEDLM_E_INVALID;
  if (n < 1 || n > kMaxMfmaGroup) return SEEDLM_E_INVALID;
  MfmaArgs args[kMaxMfmaGroup];
  bool wide[kMaxMfmaGroup];
  for (int i = 0; i < n; ++i) {
    if (!hs[i]->is_4bit() && !hs[i]->is_3bit()) return SEEDLM_E_UNSUPPORTED;
    const int st = plan_mfma(hs[i], xs[i], ys[i], partials[i], batch, args[i], wide[i]);
    if (st != SEEDLM_OK) return st;
    if (args[i].chunks > 1 && !partials[i]) return SEEDLM_E_INVALID;
  }
  if (phases & 1) {
    // One launch per (format, tiling) present.
    for (int C : {8, 12}) {
      for (bool w : {true, false}) {
        MfmaGroup g{};
        int64_t grid = 0;
        for (int i = 0; i < n; ++i) {
          if (hs[i]->C != C || wide[i] != w) continue;
          g.m[g.n] = args[i];
          g.m[g.n].wg_begin = (int)grid;
          grid += (int64_t)args[i].tiles * args[i].chunks;
          ++g.n;
        }
        if (g.n == 0) continue;
        if (grid >= (1LL << 31)) return SEEDLM_E_UNSUPPORTED;
        if (C == 8) {
          if (w) launch_main<8, 4>(g, (int)grid, s);
          else launch_main<8, 1>(g, (int)grid, s);
        } else {
          if (w) launch_main<12, 4>(g, (int)grid, s);
          else launch_main<12, 1>(g, (int)grid, s);
        }
        SEEDLM_HIP_CHECK(hipGetLastError());
      }
    }
  }
  if (phases & 2) {
    // One reduce launch over the matrices that were split into chunks (the
    // others wrote y directly).
    MfmaGroup g{};
    int64_t red = 0;
    for (int i = 0; i < n; ++i) {
      if (args[i].chunks == 1) continue;
      g.m[g.n] = args[i];
      g.m[g.n].red_begin = (int)red;
      red += (args[i].rows + 63) / 64;
      ++g.n;
    }
    if (g.n > 0) {
      hipLaunchKernelGGL(reduce_chunks_kernel, dim3((unsigned)red), dim3(256), 0,
                         s, g);
      SEEDLM_HIP_CHECK(hipGetLastError());
    }
  }
  return SEEDLM_OK;
}

}  // namespace seedlm
