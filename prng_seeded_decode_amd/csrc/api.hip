// C-ABI entry points that launch kernels: argument checks and kernel choice.
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

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

constexpr int kMaxDevices = 64;
std::mutex g_table_mu;
uint32_t* g_ext_table[kMaxDevices] = {nullptr};

bool dtype_ok(int d) { return d == SEEDLM_F32 || d == SEEDLM_F16; }

// Calls launch on the current device, which must be the one h was packed on.
bool on_handle_device(const seedlm_matrix* h) {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == h->device;
}

// ---- per-stream scratch for the split reductions ----
//
// A call's partials live in a buffer of the library keyed by (device, stream),
// never in a handle: calls on one stream run one after another on the GPU, so
// they can share it, and calls on different streams get different buffers.  A
// buffer that is too small is replaced by one at least twice its size; the old
// one stays allocated (retired) until seedlm_scratch_release, so launches still
// in flight, and graphs captured from earlier calls, keep valid memory.
struct StreamScratch {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
std::mutex g_scratch_mu;
std::vector<StreamScratch> g_scratch;
std::vector<StreamScratch> g_retired;

int stream_scratch(int dev, hipStream_t s, size_t bytes, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  StreamScratch* e = nullptr;
  for (StreamScratch& c : g_scratch)
    if (c.device == dev && c.stream == s) e = &c;
  if (e && e->bytes >= bytes) {
    *out = e->ptr;
    return SEEDLM_OK;
  }
  size_t want = (bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
  if (e && want < 2 * e->bytes) want = 2 * e->bytes;
  void* p = nullptr;
  if (hipMalloc(&p, want) != hipSuccess) return SEEDLM_E_NOMEM;
  if (e) {
    g_retired.push_back(*e);
    e->ptr = p;
    e->bytes = want;
  } else {
    g_scratch.push_back(StreamScratch{dev, s, p, want});
  }
  *out = p;
  return SEEDLM_OK;
}

// ---- timing events of the main kernels (measurement only) ----
struct TimingEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local TimingEvents t_pending;  // set for the next call
thread_local TimingEvents t_active;   // handed out during a call's main launches

// ---- kernel choice and grouping ----

enum Kind { kLut8, kLut12, kMfma, kSimple, kTable, kDirect };

// Batch-1 calls in the pages' formats whose launch group holds at most this
// many blocks, in matrices of at most kDirectMaxPanels panels per row, run the
// direct kernel: there the table builds and the second (reduction) launch of
// the table-lookup kernels cost more than the direct kernel's exact per-lane
// decode.  GPU time per call (events around it): 4-bit 2048x2048 7.0 us direct
// against 11.2 us, 2048x4096 9.1 against 12.2, 4096x4096 12.9 against 12.6,
// 1024x8192 (32 panels) 13.0 against 12.3; 3-bit 4096x4096 13.7 against 16.2,
// 4096x8192 22.2 against 18.7 (the 3-bit table-lookup kernel does about twice
// the work per weight).
constexpr int64_t kDirectMaxBlocks4 = 5 << 18;  // 1.25M blocks
constexpr int64_t kDirectMaxBlocks3 = 1 << 21;  // 2M blocks
constexpr int64_t kDirectMaxPanels = 24;

struct Group {
  int begin, count;
  Kind kind;
};

// Matrices of one call are cut into launch groups: at batch 1 up to 8
// consecutive matrices of one format (the table-lookup kernels), at batch > 1
// with fp16 x and y up to 8 of any format (the matrix-core kernel, which
// launches per format itself), otherwise one matrix at a time through the
// exact per-lane kernel.  A variant other than AUTO applies to a single matrix.
// next_group gives the group that starts at matrix i (no heap allocation, so
// the no-alloc entry point can use it too).
int next_group(const seedlm_handle* hs, int n, int batch, int xdt, int ydt, int variant, int i,
               Group* g) {
  const bool f16 = xdt == SEEDLM_F16 && ydt == SEEDLM_F16;
  // The table-lookup and matrix-core kernels take the pages' two formats.
  auto fast = [&](int m) { return hs[m]->is_4bit() || hs[m]->is_3bit(); };
  if (variant != SEEDLM_VARIANT_AUTO) {
    if (n != 1) return SEEDLM_E_INVALID;
    switch (variant) {
      case SEEDLM_VARIANT_LUT:
        if (batch != 1 || !fast(0)) return SEEDLM_E_UNSUPPORTED;
        *g = {0, 1, hs[0]->is_4bit() ? kLut8 : kLut12};
        return SEEDLM_OK;
      case SEEDLM_VARIANT_TABLE:
        if (batch != 1 || !hs[0]->is_4bit()) return SEEDLM_E_UNSUPPORTED;
        *g = {0, 1, kTable};
        return SEEDLM_OK;
      case SEEDLM_VARIANT_SIMPLE:
        *g = {0, 1, kSimple};
        return SEEDLM_OK;
      case SEEDLM_VARIANT_MFMA:
        if (!f16 || !fast(0)) return SEEDLM_E_UNSUPPORTED;
        *g = {0, 1, kMfma};
        return SEEDLM_OK;
      case SEEDLM_VARIANT_DIRECT:
        if (!direct_fits(hs[0], batch)) return SEEDLM_E_UNSUPPORTED;
        *g = {0, 1, kDirect};
        return SEEDLM_OK;
      default:
        return SEEDLM_E_UNSUPPORTED;
    }
  }
  auto same_format = [&](int a, int b) {
    return hs[a]->C == hs[b]->C && hs[a]->P == hs[b]->P && hs[a]->K == hs[b]->K;
  };
  // Up to 8 consecutive matrices of i's format that the direct kernel takes.
  auto direct_run = [&]() {
    int k = 0;
    while (i + k < n && k < 8 && same_format(i, i + k) && direct_fits(hs[i + k], batch)) ++k;
    return k;
  };
  int k = 0;
  Kind kind = kSimple;
  if (!fast(i) || (batch > 1 && !f16)) {
    // the exact kernels: direct for every shape it takes, else one wave per row
    k = direct_run();
    if (k > 0) kind = kDirect;
    else k = 1;
  } else if (batch == 1) {
    while (i + k < n && k < 8 && same_format(i, i + k)) ++k;
    kind = hs[i]->is_4bit() ? kLut8 : kLut12;
    int64_t blocks = 0, np_max = 0;
    bool fits = true;
    for (int j = i; j < i + k; ++j) {
      blocks += hs[j]->rows * hs[j]->nb;
      np_max = std::max<int64_t>(np_max, hs[j]->np);
      fits = fits && direct_fits(hs[j], batch);
    }
    if (fits && blocks <= (hs[i]->is_4bit() ? kDirectMaxBlocks4 : kDirectMaxBlocks3) &&
        np_max <= kDirectMaxPanels)
      kind = kDirect;
  } else {
    kind = kMfma;
    while (i + k < n && k < 8 && fast(i + k)) ++k;
  }
  *g = {i, k, kind};
  return SEEDLM_OK;
}

constexpr int64_t kScratchAlign = 64;  // floats (256 bytes) between matrices

int64_t partial_floats(Kind kind, const seedlm_matrix* h, int batch) {
  int64_t f = 0;
  switch (kind) {
    case kLut8:
    case kTable: f = lut_partial_floats(h); break;
    case kLut12: f = lut12_partial_floats(h); break;
    case kMfma: f = mfma_partial_floats(h, batch); break;
    default: f = 0;
  }
  return (f + kScratchAlign - 1) / kScratchAlign * kScratchAlign;
}

// Scratch floats of a whole call (the matrices' ranges one after another).
int total_partial_floats(const seedlm_handle* hs, int n, int batch, int xdt, int ydt,
                         int variant, int64_t* total) {
  *total = 0;
  Group g;
  for (int i = 0; i < n; i += g.count) {
    const int st = next_group(hs, n, batch, xdt, ydt, variant, i, &g);
    if (st != SEEDLM_OK) return st;
    for (int j = 0; j < g.count; ++j) *total += partial_floats(g.kind, hs[g.begin + j], batch);
  }
  return SEEDLM_OK;
}

int check_call(const seedlm_handle* hs, const void* const* x, void* const* y, int n, int batch,
               int xdt, int ydt) {
  if (!hs || !x || !y || n < 0) return SEEDLM_E_INVALID;
  if (batch < 1 || batch > SEEDLM_MAX_BATCH) return SEEDLM_E_INVALID;
  if (!dtype_ok(xdt) || !dtype_ok(ydt)) return SEEDLM_E_UNSUPPORTED;
  for (int i = 0; i < n; ++i)
    if (!hs[i] || !x[i] || !y[i]) return SEEDLM_E_INVALID;
  int dev = -1;
  if (n > 0 && hipGetDevice(&dev) != hipSuccess) return SEEDLM_E_DEVICE;
  for (int i = 0; i < n; ++i)
    if (hs[i]->device != dev) return SEEDLM_E_INVALID;  // packed on another device
  return SEEDLM_OK;
}

// Where a call's partials go: the library's per-stream scratch (allocated on
// demand), or the static scratch of the no-alloc entry point.
enum ScratchSource { kStreamScratch, kStaticScratch };

// ---- static scratch of seedlm_gemv_many_noalloc ----
//
// A file-scope device array: every device the library runs on holds its own
// copy (kStaticScratchBytes) until the process ends.  In host code `scratch` is
// only a stand-in for the symbol, never a device address: its address on a
// device comes from hipGetSymbolAddress, taken once per device with that device
// current and kept in g_static_ptr; kernels get that pointer.  The main kernels
// write every partial the reductions read, so nothing needs clearing between
// calls; calls that overlap on one device share the array and race.
constexpr size_t kStaticScratchBytes = SEEDLM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {nullptr};

int static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return SEEDLM_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SEEDLM_E_DEVICE;
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return SEEDLM_OK;
}

// The body of every gemv entry point: phases & 1 runs the main kernels, phases
// & 2 the reductions of the split ones.  The exact per-lane kernel has no
// reduction and runs whole in phase 1.
int run_gemv(const seedlm_handle* hs, const void* const* x, void* const* y, int n, int batch,
             int xdt, int ydt, int variant, void* stream, int phases, ScratchSource src) {
  // Timing events asked for apply to this call's main kernels only.
  struct ActiveEvents {
    explicit ActiveEvents(bool main) {
      if (main) {
        t_active = t_pending;
        t_pending = TimingEvents{};
      }
    }
    ~ActiveEvents() { t_active = TimingEvents{}; }
  } active_events(phases & 1);
  int st = check_call(hs, x, y, n, batch, xdt, ydt);
  if (st != SEEDLM_OK || n == 0) return st;
  int64_t total = 0;
  st = total_partial_floats(hs, n, batch, xdt, ydt, variant, &total);
  if (st != SEEDLM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* base = nullptr;
  if (total > 0) {
    void* p = nullptr;
    if (src == kStreamScratch) {
      st = stream_scratch(hs[0]->device, s, (size_t)total * sizeof(float), &p);
    } else {
      if ((size_t)total * sizeof(float) > kStaticScratchBytes) return SEEDLM_E_SCRATCH_LIMIT;
      st = static_scratch(hs[0]->device, &p);
    }
    if (st != SEEDLM_OK) return st;
    base = static_cast<float*>(p);
  }
  int64_t off = 0;
  Group g;
  for (int i = 0; i < n; i += g.count) {
    st = next_group(hs, n, batch, xdt, ydt, variant, i, &g);
    if (st != SEEDLM_OK) return st;
    const seedlm_matrix* gh[8];
    float* parts[8];
    for (int j = 0; j < g.count; ++j) {
      gh[j] = hs[g.begin + j];
      const int64_t f = partial_floats(g.kind, gh[j], batch);
      parts[j] = f > 0 ? base + off : nullptr;
      off += f;
    }
    const void* const* gx = x + g.begin;
    void* const* gy = y + g.begin;
    switch (g.kind) {
      case kLut8:
      case kTable: {
        const uint32_t* table = nullptr;
        if (g.kind == kTable) {
          table = ext_table(gh[0]->device);
          if (!table) return SEEDLM_E_DEVICE;
        }
        st = launch_gemv_lut_group(gh, gx, gy, parts, g.count, xdt, ydt, table, s, phases);
        break;
      }
      case kLut12:
        st = launch_gemv_lut12_group(gh, gx, gy, parts, g.count, xdt, ydt, s, phases);
        break;
      case kMfma:
        st = launch_gemv_mfma_group(gh, gx, gy, parts, g.count, batch, xdt, ydt, s, phases);
        break;
      case kSimple:
        st = (phases & 1) ? launch_gemv_simple(gh[0], gx[0], gy[0], batch, xdt, ydt, s)
                          : SEEDLM_OK;
        break;
      case kDirect:
        st = (phases & 1) ? launch_gemv_direct_group(gh, gx, gy, g.count, batch, xdt, ydt, s)
                          : SEEDLM_OK;
        break;
    }
    if (st != SEEDLM_OK) return st;
  }
  return SEEDLM_OK;
}

}  // namespace

// The 2^16-entry table of extension bits b[16..47] (the TABLE variant keeps it
// resident in L2 / the MALL instead of rebuilding the bits per block), one per
// device, built synchronously by the first seedlm_pack there.
int ensure_ext_table(int device) {
  if (device < 0 || device >= kMaxDevices) return SEEDLM_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_table_mu);
  if (g_ext_table[device]) return SEEDLM_OK;
  uint32_t* t = nullptr;
  if (hipMalloc((void**)&t, 65536 * sizeof(uint32_t)) != hipSuccess) return SEEDLM_E_NOMEM;
  hipLaunchKernelGGL(ext_table_kernel, dim3(256), dim3(256), 0, 0, t);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(nullptr) != hipSuccess) {
    (void)hipFree(t);
    return SEEDLM_E_DEVICE;
  }
  g_ext_table[device] = t;
  return SEEDLM_OK;
}

void main_launch_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = t_active.start;
  *stop = t_active.stop;
  t_active.start = nullptr;  // only the first main launch records the start
}

const uint32_t* ext_table(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_table_mu);
  return g_ext_table[device];
}

}  // namespace seedlm

using namespace seedlm;

extern "C" {

int seedlm_gemv_variant(seedlm_handle h, const void* x, void* y, int batch, int x_dtype,
                        int y_dtype, int variant, void* stream) {
  return run_gemv(&h, &x, &y, 1, batch, x_dtype, y_dtype, variant, stream, 3, kStreamScratch);
}

int seedlm_gemv(seedlm_handle h, const void* x, void* y, int batch, int x_dtype, int y_dtype,
                void* stream) {
  return run_gemv(&h, &x, &y, 1, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, stream, 3,
                  kStreamScratch);
}

int seedlm_gemv_many(const seedlm_handle* handles, const void* const* x, void* const* y, int n,
                     int batch, int x_dtype, int y_dtype, void* stream) {
  return run_gemv(handles, x, y, n, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, stream, 3,
                  kStreamScratch);
}

int seedlm_gemv_many_noalloc(const seedlm_handle* handles, const void* const* x, void* const* y,
                             int n, int batch, int x_dtype, int y_dtype, void* stream) {
  return run_gemv(handles, x, y, n, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, stream, 3,
                  kStaticScratch);
}

int seedlm_gemv_many_begin(const seedlm_handle* handles, const void* const* x, void* const* y,
                           int n, int batch, int x_dtype, int y_dtype, void* stream) {
  return run_gemv(handles, x, y, n, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, stream, 1,
                  kStreamScratch);
}

int seedlm_gemv_many_end(const seedlm_handle* handles, const void* const* x, void* const* y,
                         int n, int batch, int x_dtype, int y_dtype, void* stream) {
  return run_gemv(handles, x, y, n, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, stream, 2,
                  kStreamScratch);
}

int seedlm_gemv_scratch_bytes(const seedlm_handle* handles, int n, int batch, int x_dtype,
                              int y_dtype, size_t* bytes) {
  if (!handles || n < 0 || !bytes) return SEEDLM_E_INVALID;
  if (batch < 1 || batch > SEEDLM_MAX_BATCH) return SEEDLM_E_INVALID;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return SEEDLM_E_UNSUPPORTED;
  for (int i = 0; i < n; ++i)
    if (!handles[i]) return SEEDLM_E_INVALID;
  int64_t total = 0;
  const int st =
      total_partial_floats(handles, n, batch, x_dtype, y_dtype, SEEDLM_VARIANT_AUTO, &total);
  if (st != SEEDLM_OK) return st;
  *bytes = (size_t)total * sizeof(float);
  return SEEDLM_OK;
}

int seedlm_bench_time_next_call(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return SEEDLM_E_INVALID;
  t_pending.start = static_cast<hipEvent_t>(start_event);
  t_pending.stop = static_cast<hipEvent_t>(stop_event);
  return SEEDLM_OK;
}

int seedlm_scratch_release(void) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SEEDLM_E_DEVICE;
  int rc = SEEDLM_OK;
  for (std::vector<StreamScratch>* list : {&g_scratch, &g_retired}) {
    for (StreamScratch& e : *list) {
      if (!e.ptr) continue;
      if (hipSetDevice(e.device) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
          hipFree(e.ptr) != hipSuccess)
        rc = SEEDLM_E_DEVICE;
    }
    list->clear();
  }
  if (hipSetDevice(cur) != hipSuccess) rc = SEEDLM_E_DEVICE;
  return rc;
}

int seedlm_decode(seedlm_handle h, float* W_out, void* stream) {
  if (!h || !W_out) return SEEDLM_E_INVALID;
  if (!on_handle_device(h)) return SEEDLM_E_INVALID;
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
  if (!on_handle_device(h)) return SEEDLM_E_INVALID;
  int st = check_gemm(h, X, ntok, x_dtype, y_dtype);
  if (st != SEEDLM_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* part = nullptr;
  const size_t bytes = gemm_scratch_bytes(h, ntok);
  if (bytes > 0) {
    st = stream_scratch(h->device, s, bytes, &part);
    if (st != SEEDLM_OK) return st;
  }
  return launch_gemm(h, X, Y, ntok, static_cast<float*>(part), s);
}

int seedlm_gemm_scratch_bytes(seedlm_handle h, int64_t ntok, size_t* bytes) {
  if (!h || !bytes || ntok < 1) return SEEDLM_E_INVALID;
  *bytes = (h->is_4bit() || h->is_3bit()) ? gemm_scratch_bytes(h, ntok) : 0;
  return SEEDLM_OK;
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
