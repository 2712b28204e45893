// C-ABI entry points that launch kernels: argument checks and kernel choice.
#include <mutex>
#include <new>

#include "lfsr_device.h"
#include "seedlm_internal.h"

namespace seedlm {

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

__global__ void ext_table_kernel(uint32_t* __restrict__ table) {
  const uint32_t s = blockIdx.x * blockDim.x + threadIdx.x;
  // extension bits 16..39 in the low three bytes, the seed's high byte on top
  if (s < 65536u) table[s] = (ext_bits<uint32_t>(s) & 0x00FFFFFFu) | ((s >> 8) << 24);
}

bool dtype_ok(int d) { return d == SEEDLM_F32 || d == SEEDLM_F16; }

int check_common(seedlm_handle h, const void* x, void* y, int batch, int xdt, int ydt) {
  if (!h || !x || !y) return SEEDLM_E_INVALID;
  if (batch < 1 || batch > SEEDLM_MAX_BATCH) return SEEDLM_E_INVALID;
  if (!dtype_ok(xdt) || !dtype_ok(ydt)) return SEEDLM_E_UNSUPPORTED;
  return SEEDLM_OK;
}

}  // namespace

// The 2^16-entry table of extension bits b[16..47] (the TABLE variant keeps it
// resident in L2 / the MALL instead of rebuilding the bits per block).
int build_ext_table(seedlm_matrix* h) {
  if (h->d_ext_table) return SEEDLM_OK;
  SEEDLM_HIP_CHECK(hipMalloc((void**)&h->d_ext_table, 65536 * sizeof(uint32_t)));
  hipLaunchKernelGGL(ext_table_kernel, dim3(256), dim3(256), 0, 0, h->d_ext_table);
  SEEDLM_HIP_CHECK(hipGetLastError());
  SEEDLM_HIP_CHECK(hipDeviceSynchronize());
  return SEEDLM_OK;
}

}  // namespace seedlm

using namespace seedlm;

extern "C" {

int seedlm_gemv_variant(seedlm_handle h, const void* x, void* y, int batch, int x_dtype,
                        int y_dtype, int variant, void* stream) {
  int st = check_common(h, x, y, batch, x_dtype, y_dtype);
  if (st != SEEDLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant) {
    case SEEDLM_VARIANT_AUTO:
      if (batch == 1 && h->C == 8) return launch_gemv_lut(h, x, y, x_dtype, y_dtype, false, s);
      if (batch == 1 && h->C == 12)
        return launch_gemv_lut12_group(&h, &x, &y, 1, x_dtype, y_dtype, s, 3);
      if (x_dtype == SEEDLM_F16 && y_dtype == SEEDLM_F16)
        return launch_gemv_mfma(h, x, y, batch, x_dtype, y_dtype, s);
      return launch_gemv_simple(h, x, y, batch, x_dtype, y_dtype, s);
    case SEEDLM_VARIANT_LUT:
      if (batch != 1) return SEEDLM_E_UNSUPPORTED;
      if (h->C == 12) return launch_gemv_lut12_group(&h, &x, &y, 1, x_dtype, y_dtype, s, 3);
      return launch_gemv_lut(h, x, y, x_dtype, y_dtype, false, s);
    case SEEDLM_VARIANT_TABLE: {
      if (batch != 1 || h->C != 8) return SEEDLM_E_UNSUPPORTED;
      st = build_ext_table(h);
      if (st != SEEDLM_OK) return st;
      return launch_gemv_lut(h, x, y, x_dtype, y_dtype, true, s);
    }
    case SEEDLM_VARIANT_SIMPLE:
      return launch_gemv_simple(h, x, y, batch, x_dtype, y_dtype, s);
    case SEEDLM_VARIANT_MFMA:
      return launch_gemv_mfma(h, x, y, batch, x_dtype, y_dtype, s);
    default:
      return SEEDLM_E_UNSUPPORTED;
  }
}

int seedlm_gemv(seedlm_handle h, const void* x, void* y, int batch, int x_dtype, int y_dtype,
                void* stream) {
  return seedlm_gemv_variant(h, x, y, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, stream);
}

namespace {

// Shared body of seedlm_gemv_many{,_begin,_end}: phases & 1 runs the main
// kernels, phases & 2 the panel reductions.  Matrices outside the grouped
// batch-1 paths run their whole seedlm_gemv in phase 1.
int gemv_many_phases(const seedlm_handle* handles, const void* const* x, void* const* y, int n,
                     int batch, int x_dtype, int y_dtype, void* stream, int phases) {
  if (!handles || !x || !y || n < 0) return SEEDLM_E_INVALID;
  for (int i = 0; i < n; ++i) {
    const int st = check_common(handles[i], x[i], y[i], batch, x_dtype, y_dtype);
    if (st != SEEDLM_OK) return st;
    for (int j = 0; j < i; ++j)
      if (handles[j] == handles[i]) return SEEDLM_E_INVALID;  // shared workspace
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  int i = 0;
  const bool mfma = batch > 1 && x_dtype == SEEDLM_F16 && y_dtype == SEEDLM_F16;
  while (i < n) {
    // Group up to 8 consecutive matrices: at batch 1 those of one format (the
    // table-lookup kernels), at batch > 1 with fp16 x and y any of them (the
    // matrix-core kernel, which launches per format itself).
    const int C = handles[i]->C;
    int k = 0;
    while (batch == 1 && i + k < n && k < 8 && handles[i + k]->C == C &&
           handles[i + k]->bytes < 0x80000000ull)
      ++k;
    while (mfma && i + k < n && k < 8) ++k;
    if (k >= 1) {
      const seedlm_matrix* hs[8];
      for (int j = 0; j < k; ++j) hs[j] = handles[i + j];
      int st;
      if (mfma)
        st = launch_gemv_mfma_group(hs, x + i, y + i, k, batch, x_dtype, y_dtype, s, phases);
      else if (C == 8)
        st = launch_gemv_lut_group(hs, x + i, y + i, k, x_dtype, y_dtype, false, s, phases);
      else
        st = launch_gemv_lut12_group(hs, x + i, y + i, k, x_dtype, y_dtype, s, phases);
      if (st != SEEDLM_OK) return st;
      i += k;
    } else {
      if (phases & 1) {
        const int st = seedlm_gemv_variant(handles[i], x[i], y[i], batch, x_dtype, y_dtype,
                                           SEEDLM_VARIANT_AUTO, stream);
        if (st != SEEDLM_OK) return st;
      }
      ++i;
    }
  }
  return SEEDLM_OK;
}

}  // namespace

int seedlm_gemv_many(const seedlm_handle* handles, const void* const* x, void* const* y, int n,
                     int batch, int x_dtype, int y_dtype, void* stream) {
  return gemv_many_phases(handles, x, y, n, batch, x_dtype, y_dtype, stream, 3);
}

int seedlm_gemv_many_begin(const seedlm_handle* handles, const void* const* x, void* const* y,
                           int n, int batch, int x_dtype, int y_dtype, void* stream) {
  return gemv_many_phases(handles, x, y, n, batch, x_dtype, y_dtype, stream, 1);
}

int seedlm_gemv_many_end(const seedlm_handle* handles, const void* const* x, void* const* y,
                         int n, int batch, int x_dtype, int y_dtype, void* stream) {
  return gemv_many_phases(handles, x, y, n, batch, x_dtype, y_dtype, stream, 2);
}

int seedlm_decode(seedlm_handle h, float* W_out, void* stream) {
  if (!h || !W_out) return SEEDLM_E_INVALID;
  return launch_decode(h, W_out, static_cast<hipStream_t>(stream));
}

int seedlm_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0)
    return SEEDLM_E_INVALID;
  return launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
}

int seedlm_fp16_gemv(const void* W, const void* x, void* y, int64_t rows, int64_t cols,
                     int batch, void* stream) {
  if (!W || !x || !y || rows <= 0 || cols <= 0 || cols % 8 != 0) return SEEDLM_E_INVALID;
  if (batch < 1 || batch > SEEDLM_MAX_BATCH) return SEEDLM_E_INVALID;
  return launch_fp16_gemv(W, x, y, rows, cols, batch, static_cast<hipStream_t>(stream));
}

int seedlm_gemm(seedlm_handle h, const void* X, void* Y, int64_t ntok, int x_dtype, int y_dtype,
                void* stream) {
  if (!h || !X || !Y || ntok < 1) return SEEDLM_E_INVALID;
  return launch_gemm(h, X, Y, ntok, x_dtype, y_dtype, static_cast<hipStream_t>(stream));
}

int seedlm_gemm_decoded_bytes(seedlm_handle h, size_t* bytes) {
  if (!h || !bytes) return SEEDLM_E_INVALID;
  *bytes = decoded_workspace_bytes(h);
  return SEEDLM_OK;
}

int seedlm_gemm_decoded(seedlm_handle h, const void* X, void* Y, int64_t ntok, int x_dtype,
                        int y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || !X || !Y || !workspace || ntok < 1) return SEEDLM_E_INVALID;
  return launch_gemm_decoded(h, X, Y, ntok, x_dtype, y_dtype, workspace, workspace_bytes,
                             static_cast<hipStream_t>(stream));
}

int seedlm_encoder_create(int C, int P, int K, int Q, seedlm_encoder_handle* out) {
  if (!out) return SEEDLM_E_INVALID;
  *out = nullptr;
  if (!encoder_format_supported(C, P, K, Q)) return SEEDLM_E_UNSUPPORTED;
  seedlm_encoder* e = new (std::nothrow) seedlm_encoder;
  if (!e) return SEEDLM_E_NOMEM;
  e->C = C;
  e->P = P;
  e->K = K;
  e->Q = Q;
  e->table_bytes = encoder_table_bytes(C, P, K, Q);
  int rc = SEEDLM_OK;
  if (hipGetDevice(&e->device) != hipSuccess) rc = SEEDLM_E_DEVICE;
  if (rc == SEEDLM_OK && hipMalloc(&e->d_table, e->table_bytes) != hipSuccess) {
    e->d_table = nullptr;
    rc = SEEDLM_E_NOMEM;
  }
  if (rc == SEEDLM_OK) rc = launch_seed_table(C, P, K, Q, e->d_table, nullptr);
  if (rc == SEEDLM_OK && hipStreamSynchronize(nullptr) != hipSuccess) rc = SEEDLM_E_DEVICE;
  if (rc != SEEDLM_OK) {
    if (e->d_table) (void)hipFree(e->d_table);
    delete e;
    return rc;
  }
  *out = e;
  return SEEDLM_OK;
}

int seedlm_encoder_destroy(seedlm_encoder_handle e) {
  if (!e) return SEEDLM_OK;
  int rc = SEEDLM_OK;
  if (e->d_table && hipFree(e->d_table) != hipSuccess) rc = SEEDLM_E_DEVICE;
  delete e;
  return rc;
}

int seedlm_encode(seedlm_encoder_handle e, const void* W, int64_t rows, int64_t cols, void* seeds,
                  int8_t* coeffs, int8_t* exps, float* err, void* stream) {
  if (!e || !W || !seeds || !coeffs || !exps) return SEEDLM_E_INVALID;
  if (rows <= 0 || cols <= 0) return SEEDLM_E_INVALID;
  const uintptr_t align = e->C == 8 && cols % 8 == 0 ? 16 : 2;
  if ((uintptr_t)W % align != 0) return SEEDLM_E_INVALID;
  if (rows > INT64_MAX / (cols + e->C)) return SEEDLM_E_INVALID;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SEEDLM_E_DEVICE;
  if (dev != e->device) return SEEDLM_E_INVALID;
  return launch_encode(e->C, e->P, e->K, e->Q, e->d_table, W, rows, cols, seeds, coeffs, exps, err,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"
