// Pieces shared by the batch-1 table-lookup GEMV kernels (gemv_lut.hip for the
// 4-bit format, gemv_lut12.hip for the 3-bit one): the launch descriptor of a
// group of matrices, the host-side work split, the deterministic panel
// reduction and a few device helpers.
//
// Both kernels cut every matrix into column units (a packed panel: 32 blocks
// for C = 8, 16 blocks for C = 12), build per-unit lookup tables of x in LDS and
// stream the unit's rows past them, writing one fp32 partial per (unit, row).
// reduce_panels_kernel then adds the partials of each row in a fixed order.
#pragma once

#include <hip/hip_fp16.h>

#include <algorithm>

#include "seedlm_internal.h"

namespace seedlm {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Up to kMaxGroup matrices share one launch; their work items are numbered one
// after another (matrix-major, then column unit, then row slab).
constexpr int kMaxGroup = 8;
struct LutMatrix {
  const uint32_t* words;
  const void* x;
  float* partial;
  void* y;
  uint32_t words_bytes;  // C = 8: the packed words; C = 12: words and exponents
  uint32_t exp_off;      // C = 12: byte offset of the exponent nibbles
  int Mp, rows, cols, nb;
  int np;                // column units (= partials per row)
  int slabs;             // row slabs per unit
  int64_t item_begin;    // first global work item of this matrix
  int red_begin;         // first reduce workgroup of this matrix (64 rows each)
};
constexpr int kMaxWorkgroups = 512;
struct LutGroup {
  LutMatrix m[kMaxGroup];
  int n;
  int red_blocks;  // reduce workgroups over all matrices
  float scale;     // power of two applied to each row's sum of partials
  int grid;
  // Workgroup w processes global work items [bounds[w], bounds[w+1]).
  int32_t bounds[kMaxWorkgroups + 1];
};

// Numbers the items and reduce workgroups of grp.m[0..n-1] (np, slabs, Mp and
// rows set) and splits the items into one range per workgroup, of about equal
// cost: one unit per slab, plus build_cost per column unit a range starts or
// enters (its table build).  Returns false if a count overflows the launch.
inline bool split_group(LutGroup& grp, int64_t build_cost) {
  int64_t items = 0, red = 0, total_cost = 0;
  for (int i = 0; i < grp.n; ++i) {
    LutMatrix& M = grp.m[i];
    M.item_begin = items;
    M.red_begin = (int)red;
    items += (int64_t)M.np * M.slabs;
    red += (M.rows + 63) / 64;
    total_cost += (int64_t)M.np * (M.slabs + build_cost);
  }
  if (red >= (1LL << 30) || items >= (1LL << 31)) return false;
  grp.red_blocks = (int)red;
  int64_t G = device_cu_count();
  if (G > kMaxWorkgroups) G = kMaxWorkgroups;
  if (G > items) G = items;
  // Costs accumulate unit by unit: a range that enters a unit pays the build
  // once, then one per slab.  One sweep places every boundary.
  grp.bounds[0] = 0;
  int64_t w = 1, acc = 0;
  for (int i = 0; i < grp.n && w < G; ++i) {
    const int64_t slabs = grp.m[i].slabs;
    for (int64_t p = 0; p < grp.m[i].np && w < G; ++p) {
      const int64_t start = grp.m[i].item_begin + p * slabs;
      const int64_t next = acc + build_cost + slabs;  // cost before the next unit
      for (; w < G && w * total_cost / G <= next; ++w) {
        const int64_t t = w * total_cost / G;
        const int64_t j = t <= acc ? 0 : std::max<int64_t>(1, t - acc - build_cost);
        grp.bounds[w] = (int32_t)(start + j);
      }
      acc = next;
    }
  }
  for (; w < G; ++w) grp.bounds[w] = (int32_t)items;
  grp.bounds[G] = (int32_t)items;
  grp.grid = (int)G;
  return true;
}

// LDS byte address [lanec.b0, src.byte K, lanec.b2, 0]: row = stream byte,
// column = this lane's slot (lanec.b0 = 4*column), region = lanec.b2.
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

template <typename YT>
__device__ inline void store_y(YT* p, float v);
template <>
__device__ inline void store_y<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void store_y<__half>(__half* p, float v) { *p = __float2half_rn(v); }

// Panel reduction: y[r] = scale * sum over units p of partial[p][r] (scale is a
// power of two, so applying it to the sum instead of to every partial gives the
// same bits and saves the main kernels a multiply per row sum).  A workgroup owns
// 64 consecutive rows of one matrix (lane = row, so every load reads 256
// contiguous bytes); wave w adds units w, w+4, w+8, ... with up to 32 loads in
// flight, and the four wave sums combine through LDS as (w0+w1)+(w2+w3).  The
// order is fixed for a given unit count, so repeated calls give identical
// results.
template <typename YT>
__global__ void __launch_bounds__(256) reduce_panels_kernel(const LutGroup grp) {
  __shared__ float wsum[4][64];
  int mi = 0;
  while (mi + 1 < grp.n && (int)blockIdx.x >= grp.m[mi + 1].red_begin) ++mi;
  const LutMatrix& M = grp.m[mi];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int r = ((int)blockIdx.x - M.red_begin) * 64 + lane;
  const int rr = r < M.rows ? r : M.rows - 1;  // in-bounds load; no store below
  const float* __restrict__ partial = M.partial + rr;
  const int np = M.np;
  const int64_t Mp = M.Mp;
  float s = 0.f;
  for (int p0 = wv; p0 < np; p0 += 4 * 32) {
    float v[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int p = p0 + 4 * k;
      v[k] = p < np ? partial[p * Mp] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) s += v[k];
  }
  wsum[wv][lane] = s;
  __syncthreads();
  if (wv == 0 && r < M.rows)
    store_y(static_cast<YT*>(M.y) + r,
            ((wsum[0][lane] + wsum[1][lane]) + (wsum[2][lane] + wsum[3][lane])) * grp.scale);
}

inline int launch_reduce(const LutGroup& grp, int ydt, hipStream_t s) {
  if (ydt == SEEDLM_F32)
    hipLaunchKernelGGL((reduce_panels_kernel<float>), dim3((unsigned)grp.red_blocks), dim3(256), 0,
                       s, grp);
  else
    hipLaunchKernelGGL((reduce_panels_kernel<__half>), dim3((unsigned)grp.red_blocks), dim3(256),
                       0, s, grp);
  SEEDLM_HIP_CHECK(hipGetLastError());
  return SEEDLM_OK;
}

}  // namespace
}  // namespace seedlm
