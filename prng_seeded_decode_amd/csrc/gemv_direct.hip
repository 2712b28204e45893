// Direct fused decode-GEMV: every lane rebuilds one block exactly and
// multiplies it with x at once (SeedLM's inference step: fetch s and t,
// rebuild the weights on the fly and use them to compute the activations;
// paperhub.cn rebuttal text before Eq. (1); blocks w = 2^e U(s) t,
// atlas.scime.ai "Approach").
//
// The batch-1 table-lookup kernels price each block through per-panel tables of
// x; building those tables and adding panel partials in a second launch costs
// a fixed ~15 us, which dominates matrices of a few million weights.  This
// kernel has neither: a workgroup owns R rows over the whole reduction axis,
// its waves split those rows into four row groups and the panels among up to
// four panel lanes, and the panel lanes' sums combine in LDS in a fixed order
// (deterministic).  It serves small matrices in the pages' formats and every
// matrix in the other packed formats.
//
// Per block (exact, as seedlm_decode): I_i = sum_j t_j (z_{jC+i} - 2^(K-1)),
// w_i = I_i 2^(e-(K-1)) in fp32, then acc[b] += w_i x[b][col] in fp32 for each
// batch row.  The stream bits past the seed come from GF(2) byte tables in LDS
// (ext(s) = T0[s & 255] ^ T1[(s >> 8) & 255] ^ T2[s >> 16]).
//
// Lane mapping: a wave reads 64 consecutive words of a panel, i.e. RPW = 64/PB
// whole panel rows (PB = 32 blocks for C = 8, 16 for C = 12); lane l holds the
// word at position l % PB of row l / PB, which is the row's slot
// q = (s & ~3) | ((s + row) & 3) (the layout rotates groups of four by the
// row).  Its x columns come straight from global memory (L1/L2 resident: x is
// read by every row), so x's size is not limited.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "lfsr_device.h"
#include "mfma_decode.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

constexpr int kRowGroups = 4;    // waves per panel lane, each on its own rows
constexpr int kMaxLanesP = 4;    // panel lanes per workgroup
constexpr int kMaxWaves = kRowGroups * kMaxLanesP;
constexpr int kMaxDirect = 8;    // matrices per launch

struct DirectMatrix {
  const uint32_t* words;
  const void* x;
  void* y;
  uint32_t buf_bytes;  // whole packed buffer (words, then exponents)
  uint32_t exp_off;    // C = 12: byte offset of the exponent nibbles
  uint32_t x_bytes;    // batch * cols * sizeof(x element)
  int rows, cols, nb, Mp, np;
  int lanes_p;   // panel lanes of this matrix's workgroups (1, 2 or 4)
  int wg_begin;  // first workgroup of this matrix
};
struct DirectGroup {
  DirectMatrix m[kMaxDirect];
  int n, batch;
  int waves;  // waves per workgroup: 4 x the largest panel-lane count
};

template <typename YT>
__device__ inline void y_store(YT* p, float v);
template <>
__device__ inline void y_store<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void y_store<__half>(__half* p, float v) { *p = __float2half_rn(v); }

// x[col0 .. col0 + C - 1] of one batch row as fp32 (byte offset off into the
// x buffer).  A row's last block may reach past the row (and, in the last
// batch row, past the buffer, where a wide buffer load would return zeros for
// all of it): `whole` is false for such a block, which then loads one element
// at a time (elements past the buffer read zero; its weights past the row's
// end are zero).
template <int C, typename XT>
__device__ inline void load_x(__amdgpu_buffer_rsrc_t xr, uint32_t off, bool whole,
                              float (&xv)[C]) {
  if (!whole) {
#pragma unroll
    for (int e = 0; e < C; ++e) {
      const uint32_t o = off + (uint32_t)(e * sizeof(XT));
      if constexpr (sizeof(XT) == 4) {
        xv[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, o, 0, 0));
      } else {
        const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(xr, o, 0, 0);
        xv[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
      }
    }
    return;
  }
  if constexpr (sizeof(XT) == 4) {
#pragma unroll
    for (int k = 0; k < C / 4; ++k) {  // 16-byte aligned: C*4 is a multiple of 16
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16u * k, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) xv[4 * k + e] = __uint_as_float(v[e]);
    }
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    uint32_t d[C / 2];
    if constexpr (C == 8) {  // 16-byte aligned
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = v[e];
    } else {  // 24 bytes per block: 8-byte aligned
#pragma unroll
      for (int k = 0; k < C / 4; ++k) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(xr, off + 8u * k, 0, 0);
        d[2 * k] = v[0];
        d[2 * k + 1] = v[1];
      }
    }
#pragma unroll
    for (int e = 0; e < C / 2; ++e) {
      const h2 h = __builtin_bit_cast(h2, d[e]);
      xv[2 * e] = (float)h[0];
      xv[2 * e + 1] = (float)h[1];
    }
  }
}

template <int C, int P, int K>
using DirectExt = typename std::conditional<(C * P - 1 <= 32), uint32_t, uint64_t>::type;

template <int C, int P, int K, int Q, int BMAX, typename XT, typename YT>
__global__ void __launch_bounds__(64 * kMaxWaves) gemv_direct_kernel(const DirectGroup grp) {
  using Ext = DirectExt<C, P, K>;
  constexpr int PB = panel_blocks(C);
  constexpr int RPW = 64 / PB;             // panel rows per wave
  constexpr int R = kRowGroups * RPW;      // rows per workgroup
  constexpr uint32_t kSeedMask = (1u << K) - 1u;
  // K = 16 sums fit 22 bits, so they can start from the float 1.5 * 2^23
  // (kMagic) and convert with the scale in one FMA; K = 20 sums do not.
  constexpr bool kMagicSum = K == 16;
  __shared__ Ext T[3][256];
  __shared__ float wsum[kMaxLanesP][BMAX][R];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = 64 * grp.waves;
  int mi = 0;
  while (mi + 1 < grp.n && (int)blockIdx.x >= grp.m[mi + 1].wg_begin) ++mi;
  const DirectMatrix& M = grp.m[mi];
  const int batch = grp.batch;
  // The matrix's own panel-lane count (from its panel count alone) fixes which
  // wave takes which panel and the summation order, so a matrix gives the
  // same bits alone or in a group; spare waves take no panels.
  const int L = M.lanes_p;
  const int rg = wave % kRowGroups, pl = wave / kRowGroups;
  const int rr = rg * RPW + lane / PB;  // row inside the workgroup
  const int r = ((int)blockIdx.x - M.wg_begin) * R + rr;
  const int spos = lane % PB;           // word position inside the panel row

  for (int e = tid; e < 768; e += nthreads) {
    const uint32_t u = (uint32_t)e & 255u, k = (uint32_t)e >> 8;
    T[k][u] = (k == 2 && K <= 16) ? Ext(0) : ext_bits_k<K, Ext>(u << (8 * k));
  }
  __syncthreads();

  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)M.words, 0, (int)M.buf_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)M.x, 0, (int)M.x_bytes, 0x00020000);
  float acc[BMAX];
#pragma unroll
  for (int b = 0; b < BMAX; ++b) acc[b] = 0.f;
  const int64_t Mp = M.Mp;
  // one block of panel p; rows past Mp, positions past the stored width and
  // panels past the last read zero words (t = 0: no contribution)
  auto load = [&](int p, uint32_t& w, uint32_t& ev) {
    const int Wp = (int)panel_stored_width(p, M.nb, PB);
    const bool ok = pl < L && p < M.np && r < M.Mp && spos < Wp;
    const int64_t k = (int64_t)p * Mp * PB + (int64_t)r * Wp + spos;
    w = __builtin_amdgcn_raw_buffer_load_b32(rsrc, ok ? (uint32_t)(k * 4) : 0x80000000u, 0, 0);
    ev = 0u;
    if constexpr (C == 12) {
      const uint32_t eoff =
          ok ? M.exp_off +
                   (uint32_t)(((int64_t)p * Mp * (PB / 4) + (int64_t)r * (Wp / 4) + spos / 4) * 2)
             : 0x80000000u;
      ev = __builtin_amdgcn_raw_buffer_load_b16(rsrc, eoff, 0, 0);
    }
  };
  auto compute = [&](int p, uint32_t w, uint32_t ev) {
    const int q = (spos & ~3) | ((spos + r) & 3);  // the block's slot in the panel
    const int col0 = (p * PB + q) * C;
    // x of the block's columns (zeros past the buffer; weights past the row's
    // end are zeroed below): batch row 0 is requested before the decode, the
    // others after it, one row at a time
    auto x_off = [&](int b) {
      return (uint32_t)((int64_t)b * M.cols + col0) * (uint32_t)sizeof(XT);
    };
    const bool whole = col0 + C <= M.cols;
    float x0[C];
    load_x<C, XT>(xr, x_off(0), whole, x0);
    const uint32_t gexp = C == 8 ? (w >> 28) : ((ev >> (4 * (spos & 3))) & 0xFu);
    Ext ext = T[0][w & 0xFFu] ^ T[1][(w >> 8) & 0xFFu];
    if constexpr (K > 16) ext ^= T[2][(w >> 16) & 0xFu];
    const uint64_t S = (uint64_t)(w & kSeedMask) | ((uint64_t)ext << K);
    int t[P], tsum = 0;
#pragma unroll
    for (int jj = 0; jj < P; ++jj) {
      t[jj] = ((int)(w << (32 - K - Q * (jj + 1)))) >> (32 - Q);
      tsum += t[jj];
    }
    // 2^(e - (K-1)) with e = g - 15
    const float sc = __uint_as_float((gexp + (uint32_t)(127 - 14 - K)) << 23);
    const int base = (kMagicSum ? kMagic : 0) - (1 << (K - 1)) * tsum;
    const float moff = -kMagicF * sc;
    float wv[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      int I = base;
#pragma unroll
      for (int jj = 0; jj < P; ++jj) {
        const int n = jj * C + i;  // window at stream bit n
        int z;
        if constexpr (K == 16) {
          z = (int)(n <= 16 ? ubfe((uint32_t)S, n, 16)
                            : (n <= 32 ? ubfe((uint32_t)(S >> 16), n - 16, 16)
                                       : ubfe((uint32_t)(S >> 32), n - 32, 16)));
        } else {
          z = (int)((uint32_t)(S >> n) & kSeedMask);
        }
        I = mad24(t[jj], z, I);
      }
      const float v = kMagicSum ? __builtin_fmaf(__int_as_float(I), sc, moff) : (float)I * sc;
      wv[i] = col0 + i < M.cols ? v : 0.f;
      acc[0] = __builtin_fmaf(wv[i], x0[i], acc[0]);
    }
#pragma unroll
    for (int b = 1; b < BMAX; ++b) {
      if (b < batch) {
        float xv[C];
        load_x<C, XT>(xr, x_off(b), whole, xv);
#pragma unroll
        for (int i = 0; i < C; ++i) acc[b] = __builtin_fmaf(wv[i], xv[i], acc[b]);
      }
    }
  };
  // panels pl, pl + L, ...: two words in flight per lane
  const int p0 = pl < L ? pl : M.np;
  uint32_t wa, ea, wb, eb;
  load(p0, wa, ea);
  load(p0 + L, wb, eb);
  for (int p = p0; p < M.np; p += 2 * L) {
    compute(p, wa, ea);
    load(p + 2 * L, wa, ea);
    if (p + L < M.np) compute(p + L, wb, eb);
    load(p + 3 * L, wb, eb);
  }

  // Row sums: over the PB lanes of a row (butterfly), then over the panel
  // lanes in a fixed order.
#pragma unroll
  for (int b = 0; b < BMAX; ++b) {
    if (b < batch) {
#pragma unroll
      for (int m = 1; m < PB; m <<= 1) acc[b] += __shfl_xor(acc[b], m, 64);
      if (spos == 0) wsum[pl][b][rr] = acc[b];
    }
  }
  __syncthreads();
  for (int k = tid; k < batch * R; k += nthreads) {
    const int b = k / R, row = k - b * R;
    const int rowg = ((int)blockIdx.x - M.wg_begin) * R + row;
    if (rowg < M.rows) {
      float v = wsum[0][b][row];
      if (L > 1) v += wsum[1][b][row];
      if (L > 2) v = v + (wsum[2][b][row] + wsum[3][b][row]);
      y_store(static_cast<YT*>(M.y) + (int64_t)b * M.rows + rowg, v);
    }
  }
}

template <int C, int P, int K, int Q, typename XT, typename YT>
void launch_typed(const DirectGroup& grp, int grid, hipStream_t s) {
  hipEvent_t e0, e1;
  main_launch_events(&e0, &e1);
  const dim3 block(64 * grp.waves);
  if (grp.batch == 1)
    hipExtLaunchKernelGGL((gemv_direct_kernel<C, P, K, Q, 1, XT, YT>), dim3((unsigned)grid),
                          block, 0, s, e0, e1, 0, grp);
  else
    hipExtLaunchKernelGGL((gemv_direct_kernel<C, P, K, Q, SEEDLM_MAX_BATCH, XT, YT>),
                          dim3((unsigned)grid), block, 0, s, e0, e1, 0, grp);
}

template <int C, int P, int K, int Q>
void launch_fmt(const DirectGroup& grp, int grid, int xdt, int ydt, hipStream_t s) {
  if (xdt == SEEDLM_F32 && ydt == SEEDLM_F32) launch_typed<C, P, K, Q, float, float>(grp, grid, s);
  else if (xdt == SEEDLM_F32) launch_typed<C, P, K, Q, float, __half>(grp, grid, s);
  else if (ydt == SEEDLM_F32) launch_typed<C, P, K, Q, __half, float>(grp, grid, s);
  else launch_typed<C, P, K, Q, __half, __half>(grp, grid, s);
}

}  // namespace

bool direct_fits(const seedlm_matrix* h, int batch) {
  const int64_t xb = batch * h->cols * 4;  // fp32 x at most
  return h->bytes < 0x80000000ull && h->Mp < (1 << 28) && xb < (1LL << 31) &&
         (h->nb + 1) * h->C * 4 < (1LL << 31);
}

int launch_gemv_direct_group(const seedlm_matrix* const* hs, const void* const* xs,
                             void* const* ys, int n, int batch, int xdt, int ydt, hipStream_t s) {
  if (n < 1 || n > kMaxDirect || batch < 1 || batch > SEEDLM_MAX_BATCH) return SEEDLM_E_INVALID;
  DirectGroup grp{};
  grp.n = n;
  grp.batch = batch;
  int64_t grid = 0;
  int lanes_max = 1;
  const int xsize = xdt == SEEDLM_F32 ? 4 : 2;
  for (int i = 0; i < n; ++i) {
    const seedlm_matrix* h = hs[i];
    if (h->C != hs[0]->C || h->P != hs[0]->P || h->K != hs[0]->K) return SEEDLM_E_INVALID;
    if (!direct_fits(h, batch)) return SEEDLM_E_UNSUPPORTED;
    DirectMatrix& M = grp.m[i];
    M.words = static_cast<const uint32_t*>(h->d_buf);
    M.x = xs[i];
    M.y = ys[i];
    M.buf_bytes = (uint32_t)h->bytes;
    M.exp_off = (uint32_t)h->exp_off;
    M.x_bytes = (uint32_t)(batch * h->cols * xsize);
    M.rows = (int)h->rows;
    M.cols = (int)h->cols;
    M.nb = (int)h->nb;
    M.Mp = (int)h->Mp;
    M.np = (int)h->np;
    // about two panels per wave, at most kMaxLanesP panel lanes
    M.lanes_p = 1;
    while (M.lanes_p < kMaxLanesP && 2 * M.lanes_p < M.np) M.lanes_p *= 2;
    lanes_max = std::max(lanes_max, M.lanes_p);
    M.wg_begin = (int)grid;
    const int rows_per_wg = kRowGroups * (64 / h->pb);
    grid += (h->Mp + rows_per_wg - 1) / rows_per_wg;
  }
  if (grid >= (1LL << 31)) return SEEDLM_E_UNSUPPORTED;
  grp.waves = kRowGroups * lanes_max;
  const seedlm_matrix* h = hs[0];
  if (h->is_4bit()) launch_fmt<8, 3, 16, 4>(grp, (int)grid, xdt, ydt, s);
  else if (h->is_3bit()) launch_fmt<12, 4, 16, 4>(grp, (int)grid, xdt, ydt, s);
  else if (h->C == 8) launch_fmt<8, 4, 16, 3>(grp, (int)grid, xdt, ydt, s);
  else launch_fmt<12, 3, 20, 4>(grp, (int)grid, xdt, ydt, s);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
