// Prefill product through a decoded copy of W (Y = X W^T for many activation
// rows).  With hundreds of rows or more the product is compute-bound, and a
// library GEMM on the matrix cores outruns a kernel that rebuilds each weight
// tile inside its K loop.  So this path decodes the whole matrix once into a
// caller-provided fp16 workspace -- fp16(w * 2^10), the same exact block
// rebuild and the same values the matrix-core kernels feed their MFMAs
// (SeedLM: weights rebuilt from seed and coefficients, paperhub.cn rebuttal
// text before Eq. (1); blocks 2^e U(s) t, atlas.scime.ai "Approach") -- and
// multiplies it with rocBLAS's gemm_ex (fp16 operands, fp32 accumulation,
// alpha = 2^-10).  The decoded copy is transient: it lives in the caller's
// workspace only for the call.
#include <hip/hip_fp16.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "lfsr_device.h"
#include "mfma_decode.h"
#include "seedlm_internal.h"

namespace seedlm {
namespace {

constexpr int kDecThreads = 256;

// Workgroups on grid.y = panel p, threads over the panel's stored words in
// storage order, grid-stride along grid.x: consecutive lanes read consecutive
// words and write their blocks' fp16 runs next to each other (a row's group
// of four lands in one 64-byte span), so loads and stores both coalesce.
// Word j of the panel is row j / Wps, position s = j % Wps of the row's stored
// width, and holds block q = (s & ~3) | ((s + r) & 3) of the panel (the
// layout rotates each group of four by the row).  Padding rows and slots past
// the last block are skipped; cols is a multiple of 8, so every 16-byte
// (4-bit) or 8-byte (3-bit quad) store lies inside the row.  (One 16-byte
// group per thread, with four stores 64 bytes apart per lane, measured 1.5x
// slower.)
template <int C>
__global__ void __launch_bounds__(kDecThreads) decode_f16_kernel(
    const uint32_t* __restrict__ buf, uint32_t exp_off, _Float16* __restrict__ Wd, int rows,
    int cols, int Mp, int nb) {
  using Ext = typename std::conditional<C == 8, uint32_t, uint64_t>::type;
  __shared__ Ext T0[256], T1[256];
  for (int e = threadIdx.x; e < 512; e += kDecThreads) {
    const uint32_t u = (uint32_t)e & 255u;
    if (e < 256) T0[u] = ext_bits<Ext>(u);
    else T1[u] = ext_bits<Ext>(u << 8);
  }
  __syncthreads();
  const int p = blockIdx.y;
  const int Wps = (int)panel_stored_width(p, nb);
  const uint32_t* pw = buf + (int64_t)p * Mp * kPanelBlocks;
  const uint16_t* ex = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(buf) +
                                                         exp_off) +
                       (int64_t)p * Mp * (kPanelBlocks / 4);
  const int n = Mp * Wps;
  const int stride = gridDim.x * kDecThreads;
  auto one = [&](int j, uint32_t w, uint32_t e) {
    const int r = Wps == kPanelBlocks ? j >> 5 : j / Wps;
    const int s = j - r * Wps;
    const int q = (s & ~3) | ((s + r) & 3);
    const int b = p * kPanelBlocks + q;
    if (j >= n || r >= rows || b >= nb) return;
    _Float16* dst = Wd + (int64_t)r * cols + (int64_t)b * C;
    if constexpr (C == 8) {
      *reinterpret_cast<half8*>(dst) = decode_c8(w, T0, T1);
    } else {
      const Dec12 d = dec12_setup(w, (e >> (4 * (s & 3))) & 15u, T0, T1);
      uint64_t* o = reinterpret_cast<uint64_t*>(dst);
      const int left = cols - b * 12;  // columns of this block inside the row (multiple of 4)
      o[0] = dec12_quad<0>(d);
      if (left > 4) o[1] = dec12_quad<4>(d);
      if (left > 8) o[2] = dec12_quad<8>(d);
    }
  };
  // Four words per lane in flight: their loads go out before any decode.
  for (int j0 = blockIdx.x * kDecThreads + threadIdx.x; j0 < n; j0 += 4 * stride) {
    uint32_t w[4], e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * stride;
      w[u] = j < n ? pw[j] : 0u;
      e[u] = 0u;
      if constexpr (C == 12) {
        const int r = Wps == kPanelBlocks ? j >> 5 : j / Wps;
        e[u] = j < n ? ex[r * (Wps / 4) + ((j - r * Wps) >> 2)] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) one(j0 + u * stride, w[u], e[u]);
  }
}

// One rocBLAS handle per device, created on first use; calls serialise on a
// mutex around the stream binding and the launch.
struct Blas {
  std::mutex mu;
  rocblas_handle h[64] = {};
};
Blas& blas() {
  static Blas b;
  return b;
}

}  // namespace

size_t decoded_bytes(const seedlm_matrix* h) { return (size_t)h->rows * (size_t)h->cols * 2; }

int launch_gemm_decoded(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, int xdt,
                        int ydt, void* ws, size_t ws_bytes, hipStream_t s) {
  if (xdt != SEEDLM_F16 || ydt != SEEDLM_F16) return SEEDLM_E_UNSUPPORTED;
  if (h->cols % 8 != 0 || (uintptr_t)x % 16 != 0 || (uintptr_t)ws % 16 != 0)
    return SEEDLM_E_UNSUPPORTED;
  if (ws_bytes < decoded_bytes(h)) return SEEDLM_E_INVALID;
  if (h->rows >= (1LL << 31) || h->cols >= (1LL << 31) || ntok >= (1LL << 31))
    return SEEDLM_E_UNSUPPORTED;
  if (h->Mp * kPanelBlocks >= (1LL << 31) || h->np >= 65536) return SEEDLM_E_UNSUPPORTED;
  // about eight workgroups per CU over all panels
  const int64_t per_panel = (h->Mp * kPanelBlocks + kDecThreads - 1) / kDecThreads;
  const int64_t gx = std::max<int64_t>(
      1, std::min<int64_t>(per_panel, (8LL * device_cu_count() + h->np - 1) / h->np));
  const dim3 grid((unsigned)gx, (unsigned)h->np);
  if (h->C == 8)
    hipLaunchKernelGGL(decode_f16_kernel<8>, grid, dim3(kDecThreads), 0, s,
                       static_cast<const uint32_t*>(h->d_buf), 0u, static_cast<_Float16*>(ws),
                       (int)h->rows, (int)h->cols, (int)h->Mp, (int)h->nb);
  else
    hipLaunchKernelGGL(decode_f16_kernel<12>, grid, dim3(kDecThreads), 0, s,
                       static_cast<const uint32_t*>(h->d_buf), (uint32_t)h->exp_off,
                       static_cast<_Float16*>(ws), (int)h->rows, (int)h->cols, (int)h->Mp,
                       (int)h->nb);
  SEEDLM_HIP_CHECK(hipGetLastError());

  // Y[ntok][rows] (row-major) = column-major Y^T (rows x ntok, ld rows)
  //   = op(A) op(B) with A = the decoded W stored column-major as cols x rows
  //   (ld cols, transposed) and B = X stored column-major as cols x ntok.
  Blas& B = blas();
  std::lock_guard<std::mutex> lock(B.mu);
  if (h->device < 0 || h->device >= 64) return SEEDLM_E_DEVICE;
  rocblas_handle& bh = B.h[h->device];
  if (!bh && rocblas_create_handle(&bh) != rocblas_status_success) {
    bh = nullptr;
    return SEEDLM_E_DEVICE;
  }
  if (rocblas_set_stream(bh, s) != rocblas_status_success) return SEEDLM_E_DEVICE;
  const float alpha = 0x1p-10f, beta = 0.f;
  const rocblas_status st = rocblas_gemm_ex(
      bh, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)h->rows,
      (rocblas_int)ntok, (rocblas_int)h->cols, &alpha, ws, rocblas_datatype_f16_r,
      (rocblas_int)h->cols, x, rocblas_datatype_f16_r, (rocblas_int)h->cols, &beta, y,
      rocblas_datatype_f16_r, (rocblas_int)h->rows, y, rocblas_datatype_f16_r,
      (rocblas_int)h->rows, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? SEEDLM_OK : SEEDLM_E_DEVICE;
}

}  // namespace seedlm
