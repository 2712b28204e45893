// Batch-1 fused decode-GEMV for the 4-bit format (C=8, P=3, K=16).
//
// SeedLM's inference step fetches each block's seed s and coefficients t, rebuilds
// the block's weights from the LFSR output and uses them at once (paperhub.cn
// rebuttal text before Eq. (1); blocks of C weights = 2^e U(s) t, atlas.scime.ai
// "Approach").  This kernel never forms the weights.  It uses the sliding-window
// structure of the 16-bit Fibonacci LFSR instead:
//
//   state z_n = sum_k b[n+k] 2^k for one bit stream b (b[0..15] = seed bits),
//   column j of U holds states z_{8j} .. z_{8j+7}, so for one block
//   D_j = sum_i x_i (z_{8j+i} - 2^15) = sum_{m<23} b[8j+m] c_m - 2^15 sum_i x_i,
//   c_m = sum_{i+k=m, i<8, k<16} x_i 2^k.
//   With stream bytes B_0..B_4 (B_0, B_1 = seed bytes):
//   D_j = L0[B_j] + 2 c_7 B_{j+1} + L2[B_{j+2}],
//   L0[v] = sum_{k<8} bit_k(v) c_k - 2^15 sum_i x_i,  L2[v] = sum_{k<7} bit_k(v) c_{16+k}
//   (bits 8..15 of the window have c_m = 2^(m-7) c_7, so the middle byte enters
//   linearly).  The block adds 2^(e-15) sum_j t_j D_j to its row.
//
// Per panel (32 blocks = 256 columns) the workgroup builds L0 and L2 for the
// panel's 32 column blocks in LDS, component-major so that lanes working on
// different slots read different banks.  Stream bytes B_2..B_4 come from GF(2)
// tables (ext(s) = T0[s & 255] ^ T1[s >> 8]; the LFSR is linear over GF(2)),
// replicated per slot for the same reason, or -- TABLE variant -- from a
// 2^16-entry table of extension bits in global memory (L2/MALL resident).
//
// LDS: region A row v = [L0[v] for slots 0..31 | T1[v] x32], region B row v =
// [T0[v] x32 | L2[v] for slots 0..31]; 256 B per row, so one v_perm_b32 turns a
// stream byte and a per-lane constant into a row/column address, and
// L0[B1] + T1[B1] come back from a single ds_read2_b32.
//
// Lane mapping: lane = 8*rho + g; the lane owns row r0+rho and slot group g
// (slots 4g..4g+3) and reads the group's four words with one 16-byte load.  The
// packed layout rotates each group by the row index, so the four rows of a
// half-wave touch 32 different slots at every step.  Each block's work is
// issued in three stages (GF(2) reads, table reads, arithmetic) over the four
// words of a lane, so the LDS latency of one block hides behind the others.  A
// row's partial sum is reduced over its 8 lanes with DPP and written per panel;
// reduce_panels_kernel adds the panels in a fixed order (deterministic).
#include <hip/hip_fp16.h>

#include "lfsr_device.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

constexpr int kThreads = 1024;  // 16 waves: 4 per SIMD
constexpr int kWaves = kThreads / 64;
constexpr int kPrefetch = 2;    // 16-byte loads in flight per lane

struct Smem {
  uint32_t A[256][64];  // [L0 (32 slots) | T1 (32 copies)]
  uint32_t B[256][64];  // [T0 (32 copies) | L2 (32 slots)]
  float xs[256];
  float c7x2[32];
};
constexpr uint32_t kRegionB = 65536;  // byte offset of B inside Smem

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <typename XT>
__device__ inline float ldx(const XT* p);
template <>
__device__ inline float ldx<float>(const float* p) { return *p; }
template <>
__device__ inline float ldx<__half>(const __half* p) { return __half2float(*p); }

// LDS byte address [lanec.b0, src.byte K, lanec.b2, 0]: row = stream byte,
// column = this lane's slot (lanec.b0 = 4*slot), region = lanec.b2.
template <int K>
__device__ inline uint32_t lut_addr(uint32_t src, uint32_t lanec) {
  return __builtin_amdgcn_perm(src, lanec, 0x0C020000u | ((4u + K) << 8));
}

template <typename T>
__device__ inline T lds_at(const uint8_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(base + byte_off);
}

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <typename XT>
__device__ void build_panel_lut(Smem& sm, const XT* __restrict__ x, int64_t cols, int64_t p) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    const int64_t c = p * 256 + tid;
    sm.xs[tid] = c < cols ? ldx(x + c) : 0.f;
  }
  __syncthreads();
  // Thread -> (slot, value group): kNV consecutive table rows per thread; the
  // low kLB bits of the row index come from small tables built by doubling,
  // the high bits are fixed per thread.
  constexpr int kNV = 256 / (kThreads / 32);
  constexpr int kLB = kNV == 16 ? 4 : (kNV == 8 ? 3 : 2);
  static_assert((1 << kLB) == kNV, "threads must give 4, 8 or 16 rows per thread");
  const int slot = tid & 31, vg = tid >> 5;
  float xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = sm.xs[slot * 8 + i];
  // c_m = sum_{i+k=m, i<8, k<16} x_i 2^k: doubling for m <= 7 (only c_0..c_7
  // are needed there), halving downwards for m = 22..16.
  float c[23];
  c[0] = xv[0];
#pragma unroll
  for (int m = 1; m < 8; ++m) c[m] = fmaf(2.f, c[m - 1], xv[m]);
  c[22] = 32768.f * xv[7];
#pragma unroll
  for (int m = 21; m >= 16; --m) c[m] = fmaf(0.5f, c[m + 1], 32768.f * xv[m - 15]);
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) S += xv[i];
  float B0 = -32768.f * S, B2 = 0.f;
#pragma unroll
  for (int k = kLB; k < 8; ++k) {
    if ((vg >> (k - kLB)) & 1) {
      B0 += c[k];
      if (k < 7) B2 += c[16 + k];
    }
  }
  float A0[kNV], A2[kNV];
  A0[0] = A2[0] = 0.f;
#pragma unroll
  for (int n = 1; n < kNV; ++n) {
    const int low = __builtin_ctz(n), rest = n & (n - 1);
    A0[n] = A0[rest] + c[low];
    A2[n] = A2[rest] + c[16 + low];
  }
#pragma unroll
  for (int n = 0; n < kNV; ++n) {
    const int v = vg * kNV + n;
    sm.A[v][slot] = __float_as_uint(A0[n] + B0);
    sm.B[v][32 + slot] = __float_as_uint(A2[n] + B2);
  }
  if (vg == 0) sm.c7x2[slot] = 2.f * c[7];
}

template <typename XT, bool kGlobalTable>
__global__ void __launch_bounds__(kThreads, 1)
    gemv_lut_kernel(const uint32_t* __restrict__ words, uint32_t words_bytes,
                    const XT* __restrict__ x, float* __restrict__ partial,
                    const uint32_t* __restrict__ ext_table, int64_t Mp, int64_t cols,
                    int64_t nb, int64_t np) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rho = lane >> 3, g = lane & 7;
  const uint8_t* lds = reinterpret_cast<const uint8_t*>(&sm);

  // Per-slot copies of the GF(2) tables (built once per launch).
  if (!kGlobalTable && tid < 512) {
    const uint32_t u = tid & 255;
    const uint32_t val = tid < 256 ? ext_bits<uint32_t>(u) : ext_bits<uint32_t>(u << 8);
    uint4* dst = reinterpret_cast<uint4*>(tid < 256 ? &sm.B[u][0] : &sm.A[u][32]);
#pragma unroll
    for (int k = 0; k < 8; ++k) dst[k] = make_uint4(val, val, val, val);
  }

  // Slots of this lane's four words: slot_j = 4g + ((j + row) & 3); slabs start
  // at multiples of 8 rows, so row & 3 == rho & 3.
  uint32_t lcA[4], lcB[4];
  int slotj[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    slotj[j] = 4 * g + ((j + rho) & 3);
    lcA[j] = (uint32_t)slotj[j] * 4u;
    lcB[j] = lcA[j] | kRegionB;
  }

  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)words, 0, (int)words_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t prsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)partial, 0, (int)(np * Mp * 4), 0x00020000);

  // Work items: (panel, 8-row slab), panel-major; each workgroup takes one
  // contiguous range.
  const int slabs = (int)(Mp / 8);
  const int64_t total = np * slabs;
  const int64_t G = gridDim.x;
  const int64_t begin = (int64_t)blockIdx.x * total / G;
  const int64_t end = ((int64_t)blockIdx.x + 1) * total / G;

  for (int64_t it = begin; it < end;) {
    const int64_t p = it / slabs;
    const int sa = (int)(it - p * slabs);
    const int64_t seg_end = (p + 1) * slabs < end ? (p + 1) * slabs : end;
    const int sb = (int)(seg_end - p * slabs);
    const int Wp = (int)panel_stored_width(p, nb);
    __syncthreads();  // previous panel's tables no longer in use
    build_panel_lut<XT>(sm, x, cols, p);
    __syncthreads();
    float c7j[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c7j[j] = sm.c7x2[slotj[j]];

    // Lanes outside the panel's width get an out-of-range base: their loads
    // return zero words (t = 0, no contribution).  Offsets grow by one slab
    // stride per step, so no per-load bounds logic is needed.
    const uint32_t lane_base =
        4 * g < Wp ? (uint32_t)(p * Mp * kPanelBlocks + rho * Wp + 4 * g) * 4u : 0x80000000u;
    const uint32_t slab_stride = 8u * (uint32_t)Wp * 4u;
    const uint32_t pstore = g == 0 ? (uint32_t)(p * Mp + rho) * 4u : 0x80000000u;

    v4u buf[kPrefetch];
    const int s_first = sa + wave;
#pragma unroll
    for (int d = 0; d < kPrefetch; ++d)
      buf[d] = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc, lane_base + (uint32_t)(s_first + d * kWaves) * slab_stride, 0, 0);

    for (int s0 = s_first; s0 < sb; s0 += kWaves * kPrefetch) {
#pragma unroll
      for (int d = 0; d < kPrefetch; ++d) {
        const int sl = s0 + d * kWaves;
        const v4u q = buf[d];
        buf[d] = __builtin_amdgcn_raw_buffer_load_b128(
            rsrc, lane_base + (uint32_t)(sl + kWaves * kPrefetch) * slab_stride, 0, 0);

        // Stage 1: GF(2) halves and the seed-byte L0 values of all four blocks.
        float l0b0[4], l0b1[4];
        uint32_t ext[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t a0 = lut_addr<0>(q[j], lcA[j]);
          const uint32_t a1 = lut_addr<1>(q[j], lcA[j]);
          l0b0[j] = lds_at<float>(lds, a0);
          l0b1[j] = lds_at<float>(lds, a1);
          if (kGlobalTable) {
            ext[j] = ext_table[q[j] & 0xFFFFu];
          } else {
            ext[j] = lds_at<uint32_t>(lds, a0 + kRegionB) ^ lds_at<uint32_t>(lds, a1 + 128);
          }
        }
        // Stage 2: table values of the extension bytes B_2..B_4.
        float l0b2[4], l2b2[4], l2b3[4], l2b4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          l0b2[j] = lds_at<float>(lds, lut_addr<0>(ext[j], lcA[j]));
          l2b2[j] = lds_at<float>(lds, lut_addr<0>(ext[j], lcB[j]) + 128);
          l2b3[j] = lds_at<float>(lds, lut_addr<1>(ext[j], lcB[j]) + 128);
          l2b4[j] = lds_at<float>(lds, lut_addr<2>(ext[j], lcB[j]) + 128);
        }
        // Stage 3: arithmetic.
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = q[j];
          const float E0 = fmaf(c7j[j], (float)((w >> 8) & 0xFFu), l0b0[j] + l2b2[j]);
          const float E1 = fmaf(c7j[j], (float)(ext[j] & 0xFFu), l0b1[j] + l2b3[j]);
          const float E2 = fmaf(c7j[j], (float)((ext[j] >> 8) & 0xFFu), l0b2[j] + l2b4[j]);
          const float t0 = (float)(((int)(w << 12)) >> 28);
          const float t1 = (float)(((int)(w << 8)) >> 28);
          const float t2 = (float)(((int)(w << 4)) >> 28);
          const float V = fmaf(t2, E2, fmaf(t1, E1, t0 * E0));
          const float part = ldexpf(V, (int)(w >> 28));
          acc = j == 0 ? part : acc + part;
        }
        // Sum the row over its 8 lanes (xor 1, xor 2, then mirror within 8).
        acc += dpp<0xB1>(acc);
        acc += dpp<0x4E>(acc);
        acc += dpp<0x141>(acc);
        const uint32_t so = sl < sb ? pstore + (uint32_t)sl * 32u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc * 0x1p-30f), prsrc, so, 0, 0);
      }
    }
    it = seg_end;
  }
}

template <typename YT>
__device__ inline void store_y(YT* p, float v);
template <>
__device__ inline void store_y<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void store_y<__half>(__half* p, float v) { *p = __float2half_rn(v); }

// y[r] = sum over panels of partial[p][r]: four lanes per row each add the
// panels p = part, part+4, part+8, ... (four loads issued at once), then the
// four sums combine as (0+1) + (2+3) with two DPP steps.  Fixed order for a
// given panel count, so repeated calls give identical results.
template <typename YT>
__global__ void __launch_bounds__(256) reduce_panels_kernel(const float* __restrict__ partial,
                                                            YT* __restrict__ y, int64_t rows,
                                                            int64_t Mp, int64_t np) {
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2;
  const int part = threadIdx.x & 3;
  const bool ok = r < rows;
  float s = 0.f;
  int64_t p = part;
  for (; p + 12 < np; p += 16) {
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ok ? partial[(p + 4 * k) * Mp + r] : 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += v[k];
  }
  for (; p < np; p += 4) s += ok ? partial[p * Mp + r] : 0.f;
  s += dpp<0xB1>(s);  // lanes (0,1), (2,3)
  s += dpp<0x4E>(s);  // (0+1) + (2+3)
  if (ok && part == 0) store_y(y + r, s);
}

template <typename XT, bool kGT>
void launch_main(const seedlm_matrix* h, const void* x, const uint32_t* table, hipStream_t s) {
  const int64_t total = h->np * (h->Mp / 8);
  int64_t G = device_cu_count();
  if (G > total) G = total;
  hipLaunchKernelGGL((gemv_lut_kernel<XT, kGT>), dim3((unsigned)G), dim3(kThreads), 0, s,
                     static_cast<const uint32_t*>(h->d_buf), (uint32_t)h->bytes,
                     static_cast<const XT*>(x), h->d_work, table, h->Mp, h->cols, h->nb, h->np);
}

}  // namespace

int launch_gemv_lut(const seedlm_matrix* h, const void* x, void* y, int xdt, int ydt,
                    bool global_table, hipStream_t s) {
  if (h->C != 8 || h->P != 3) return SEEDLM_E_UNSUPPORTED;
  if (h->bytes >= 0x80000000ull) return SEEDLM_E_UNSUPPORTED;  // 32-bit buffer offsets
  const uint32_t* table = nullptr;
  if (global_table) {
    if (!h->d_ext_table) return SEEDLM_E_INVALID;
    table = h->d_ext_table;
  }
  if (xdt == SEEDLM_F32) {
    if (global_table) launch_main<float, true>(h, x, table, s);
    else launch_main<float, false>(h, x, table, s);
  } else {
    if (global_table) launch_main<__half, true>(h, x, table, s);
    else launch_main<__half, false>(h, x, table, s);
  }
  SEEDLM_HIP_CHECK(hipGetLastError());
  const int64_t grid = (h->rows * 4 + 255) / 256;
  if (ydt == SEEDLM_F32)
    hipLaunchKernelGGL((reduce_panels_kernel<float>), dim3((unsigned)grid), dim3(256), 0, s,
                       h->d_work, static_cast<float*>(y), h->rows, h->Mp, h->np);
  else
    hipLaunchKernelGGL((reduce_panels_kernel<__half>), dim3((unsigned)grid), dim3(256), 0, s,
                       h->d_work, static_cast<__half*>(y), h->rows, h->Mp, h->np);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace seedlm
