// Prefill product through a decoded copy of W (Y = X W^T for many activation
// rows).  With hundreds of rows or more the product is compute-bound, and a
// library GEMM on the matrix cores outruns a kernel that rebuilds each weight
// tile inside its K loop.  So this path decodes the whole matrix once into a
// caller-provided fp16 workspace -- fp16(w * 2^10), the same exact block
// rebuild and the same values the matrix-core kernels feed their MFMAs
// (SeedLM: weights rebuilt from seed and coefficients, paperhub.cn rebuttal
// text before Eq. (1); blocks 2^e U(s) t, atlas.scime.ai "Approach") -- and
// multiplies it with a hipBLASLt matmul (fp16 operands, fp32 accumulation,
// alpha = 2^-10).  The decoded copy is transient: it lives in the caller's
// workspace only for the call.
#include <hip/hip_fp16.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
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
    if (e < 256) T0[u] = c8_table_word(ext_bits<Ext>(u));
    else T1[u] = c8_table_word(ext_bits<Ext>(u << 8));
  }
  __syncthreads();
  constexpr int PB = panel_blocks(C);
  constexpr int kLogPB = PB == 32 ? 5 : 4;
  const int p = blockIdx.y;
  const int Wps = (int)panel_stored_width(p, nb, PB);
  const uint32_t* pw = buf + (int64_t)p * Mp * PB;
  const uint16_t* ex = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(buf) +
                                                         exp_off) +
                       (int64_t)p * Mp * (PB / 4);
  const int n = Mp * Wps;
  const int stride = gridDim.x * kDecThreads;
  auto one = [&](int j, uint32_t w, uint32_t e) {
    const int r = Wps == PB ? j >> kLogPB : j / Wps;
    const int s = j - r * Wps;
    const int q = (s & ~3) | ((s + r) & 3);
    const int b = p * PB + q;
    if (j >= n || r >= rows || b >= nb) return;
    _Float16* dst = Wd + (int64_t)r * cols + (int64_t)b * C;
    if constexpr (C == 8) {
      // Nontemporal: the copy bypasses L2 and MALL, so the GEMM that reads it
      // next does not compete with its write-back (70B layer at 256 tokens:
      // the step 10% faster; even at 2048).  A wave writes whole lines here;
      // the 3-bit stores below (8 bytes at a 24-byte stride per lane) measured
      // 1.2-1.6x slower as nontemporal stores and stay ordinary.
      __builtin_nontemporal_store(decode_c8(w, T0, T1), reinterpret_cast<half8*>(dst));
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
        const int r = Wps == PB ? j >> kLogPB : j / Wps;
        e[u] = j < n ? ex[r * (Wps / 4) + ((j - r * Wps) >> 2)] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) one(j0 + u * stride, w[u], e[u]);
  }
}

// One hipBLASLt handle per device, created on first use, and one matmul plan
// (descriptors and the heuristic's first algorithm) per device, shape and
// scratch size.  The heuristic query costs far more host time than a launch,
// so it runs once per shape.  Plans and handles live until the process ends;
// the cache is emptied when it reaches kMaxPlans entries.  Calls serialise on
// a mutex while they look up a plan and enqueue.
constexpr size_t kMaxPlans = 64;

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t scratch = 0;  // bytes the algorithm needs
};

void destroy(Plan& p) {
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
  if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
  if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
  p = Plan{};
}

struct Blas {
  std::mutex mu;
  hipblasLtHandle_t h[64] = {};
  std::map<std::tuple<int, int64_t, int64_t, int64_t, size_t>, Plan> plans;
};
Blas& blas() {
  static Blas b;
  return b;
}

// Y[ntok][rows] (row-major) is column-major Y^T (rows x ntok, ld rows)
//   = op(A) B with A = the decoded W stored column-major as cols x rows (ld
//   cols, op = transpose) and B = X stored column-major as cols x ntok.
bool make_plan(hipblasLtHandle_t lt, int64_t rows, int64_t cols, int64_t ntok, size_t scratch_max,
               Plan& p) {
  const hipblasOperation_t opA = HIPBLAS_OP_T, opB = HIPBLAS_OP_N;
  bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opA,
                                            sizeof(opA)) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opB,
                                            sizeof(opB)) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16F, cols, rows, cols) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16F, cols, ntok, cols) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatrixLayoutCreate(&p.d, HIP_R_16F, rows, ntok, rows) ==
                HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  const uint64_t max_ws = scratch_max;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                             &max_ws, sizeof(max_ws)) == HIPBLAS_STATUS_SUCCESS;
  // The heuristic's first candidate can ask for more scratch than is offered
  // (8192 x 28672 at 512 and 1024 tokens did, despite the preference), so the
  // plan takes the first of its candidates that runs within it.
  constexpr int kCandidates = 16;
  hipblasLtMatmulHeuristicResult_t res[kCandidates];
  int found = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(lt, p.desc, p.a, p.b, p.d, p.d, pref, kCandidates,
                                             res, &found) == HIPBLAS_STATUS_SUCCESS;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  int pick = -1;
  for (int i = 0; ok && i < found && i < kCandidates && pick < 0; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= scratch_max) pick = i;
  if (pick < 0) {
    destroy(p);
    return false;
  }
  p.algo = res[pick].algo;
  p.scratch = res[pick].workspaceSize;
  return true;
}

}  // namespace

size_t decoded_bytes(const seedlm_matrix* h) { return (size_t)h->rows * (size_t)h->cols * 2; }

// Where the GEMM's scratch starts in the workspace: past the decoded matrix,
// rounded up to 256 bytes.
size_t scratch_offset(const seedlm_matrix* h) { return (decoded_bytes(h) + 255) & ~(size_t)255; }

size_t decoded_workspace_bytes(const seedlm_matrix* h) {
  return scratch_offset(h) + kDecodedScratchBytes;
}

int launch_gemm_decoded(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, int xdt,
                        int ydt, void* ws, size_t ws_bytes, hipStream_t s) {
  if (xdt != SEEDLM_F16 || ydt != SEEDLM_F16) return SEEDLM_E_UNSUPPORTED;
  if (h->cols % 8 != 0 || (uintptr_t)x % 16 != 0 || (uintptr_t)ws % 16 != 0)
    return SEEDLM_E_UNSUPPORTED;
  if (ws_bytes < decoded_bytes(h)) return SEEDLM_E_INVALID;
  if (h->rows >= (1LL << 31) || h->cols >= (1LL << 31) || ntok >= (1LL << 31))
    return SEEDLM_E_UNSUPPORTED;
  if (!h->is_4bit() && !h->is_3bit()) return SEEDLM_E_UNSUPPORTED;
  if (h->Mp * h->pb >= (1LL << 31) || h->np >= 65536) return SEEDLM_E_UNSUPPORTED;
  // The GEMM handle is per device and binds to the current one when created.
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SEEDLM_E_DEVICE;
  if (cur != h->device) return SEEDLM_E_INVALID;
  // The workspace past the decoded matrix, up to kDecodedScratchBytes, is
  // offered to the GEMM as scratch.
  const size_t off = scratch_offset(h);
  const size_t scratch_max =
      ws_bytes > off ? std::min(ws_bytes - off, kDecodedScratchBytes) & ~(size_t)255 : 0;
  void* scratch = scratch_max ? static_cast<char*>(ws) + off : nullptr;
  // The plan comes first, so that a shape the library cannot run fails before
  // anything is enqueued.
  Blas& B = blas();
  std::lock_guard<std::mutex> lock(B.mu);
  if (h->device < 0 || h->device >= 64) return SEEDLM_E_DEVICE;
  hipblasLtHandle_t& lt = B.h[h->device];
  if (!lt && hipblasLtCreate(&lt) != HIPBLAS_STATUS_SUCCESS) {
    lt = nullptr;
    return SEEDLM_E_DEVICE;
  }
  const auto key = std::make_tuple(h->device, h->rows, h->cols, ntok, scratch_max);
  auto found = B.plans.find(key);
  if (found == B.plans.end()) {
    if (B.plans.size() >= kMaxPlans) {
      for (auto& kv : B.plans) destroy(kv.second);
      B.plans.clear();
    }
    Plan p;
    if (!make_plan(lt, h->rows, h->cols, ntok, scratch_max, p)) return SEEDLM_E_DEVICE;
    found = B.plans.emplace(key, p).first;
  }
  // about eight workgroups per CU over all panels
  const int64_t per_panel = (h->Mp * h->pb + kDecThreads - 1) / kDecThreads;
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

  const Plan& p = found->second;
  const float alpha = 0x1p-10f, beta = 0.f;
  const hipblasStatus_t st =
      hipblasLtMatmul(lt, p.desc, &alpha, ws, p.a, x, p.b, &beta, y, p.d, y, p.d, &p.algo,
                      p.scratch ? scratch : nullptr, p.scratch, s);
  return st == HIPBLAS_STATUS_SUCCESS ? SEEDLM_OK : SEEDLM_E_DEVICE;
}

}  // namespace seedlm
