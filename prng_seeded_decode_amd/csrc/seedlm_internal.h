// Internal declarations shared by the host packer, the launch wrappers and the
// HIP kernels of libseedlm.  Not part of the public ABI (see include/seedlm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/seedlm.h"

namespace seedlm {

// Packed layout constants (documented in include/seedlm.h).
constexpr int kPanelBlocks = 32;  // blocks per panel
constexpr int kGroup = 4;         // slots per rotated group (one 16-byte load)
constexpr int kStateBits = 16;    // K
constexpr uint32_t kHalf = 1u << (kStateBits - 1);
constexpr uint32_t kPadWord = 0x00000001u;  // seed 1, t = 0, g = 0

}  // namespace seedlm

// The handle.  Immutable after seedlm_pack except for the workspace contents.
struct seedlm_matrix {
  int64_t rows = 0, cols = 0;
  int C = 0, P = 0, K = 0;
  int64_t nb = 0;       // blocks per row
  int64_t nbs = 0;      // stored blocks per row (last panel padded to 4 slots)
  int64_t np = 0;       // panels per row: ceil(nb / 32)
  int64_t Mp = 0;       // rows padded to a multiple of 8
  int64_t nwords = 0;   // Mp * nbs
  size_t bytes = 0;     // packed buffer size
  size_t exp_off = 0;   // byte offset of the exponent nibble array (P == 4)
  int device = 0;
  void* d_buf = nullptr;      // packed buffer (device)
  float* d_work = nullptr;    // split-reduction partials (device)
  size_t work_bytes = 0;
  uint32_t* d_ext_table = nullptr;  // 2^16-entry extension table (variant TABLE)
};

// An encoder: the per-seed table of one format on one device.
struct seedlm_encoder {
  int C = 0, P = 0, K = 0, Q = 0;
  int device = 0;
  void* d_table = nullptr;
  size_t table_bytes = 0;
};

namespace seedlm {

// Layout helpers (host and device).  Rows are padded to Mp = 8*ceil(rows/8).
// Panel p holds blocks 32p .. 32p+Wp-1; its stored width is Wp rounded up to a
// multiple of 4.  Panel p starts at word p*Mp*32 and stores its Mp rows one
// after another; inside a row, slot q sits at 4*(q/4) + ((q - r) mod 4), so the
// four words of one 16-byte load hold the group's slots rotated by the row.
__host__ __device__ inline int64_t panel_width(int64_t p, int64_t nb) {
  int64_t w = nb - (int64_t)kPanelBlocks * p;
  return w < kPanelBlocks ? w : kPanelBlocks;
}

__host__ __device__ inline int64_t panel_stored_width(int64_t p, int64_t nb) {
  return (panel_width(p, nb) + kGroup - 1) / kGroup * kGroup;
}

__host__ __device__ inline int64_t padded_rows(int64_t rows) { return (rows + 7) / 8 * 8; }

__host__ __device__ inline int64_t word_index(int64_t r, int64_t b, int64_t Mp, int64_t nb) {
  const int64_t p = b / kPanelBlocks, q = b % kPanelBlocks;
  return p * Mp * kPanelBlocks + r * panel_stored_width(p, nb) + (q & ~(int64_t)3) +
         ((q - r) & 3);
}

// Index of the uint16 that holds the exponent nibbles of (r, b)'s group, and the
// nibble number inside it (3-bit format).
__host__ __device__ inline int64_t exp_index(int64_t r, int64_t b, int64_t Mp, int64_t nb) {
  const int64_t p = b / kPanelBlocks, q = b % kPanelBlocks;
  return p * Mp * (kPanelBlocks / kGroup) + r * (panel_stored_width(p, nb) / kGroup) + q / kGroup;
}
__host__ __device__ inline int exp_nibble(int64_t r, int64_t b) {
  return (int)(((b % kPanelBlocks) - r) & 3);
}

// Launch wrappers implemented in the .hip files.  All return a status code.
int launch_decode(const seedlm_matrix* h, float* W, hipStream_t s);
int launch_gemv_simple(const seedlm_matrix* h, const void* x, void* y, int batch, int xdt,
                       int ydt, hipStream_t s);
int launch_gemv_lut(const seedlm_matrix* h, const void* x, void* y, int xdt, int ydt,
                    bool global_table, hipStream_t s);
// Up to 8 batch-1 4-bit matrices in one main launch (phases & 1: panel
// partials into the handles' workspaces) and one reduce launch (phases & 2: y).
int launch_gemv_lut_group(const seedlm_matrix* const* hs, const void* const* xs, void* const* ys,
                          int n, int xdt, int ydt, bool global_table, hipStream_t s, int phases);
// Matrix-core path (fp16 x and y only; E_UNSUPPORTED otherwise).
int launch_gemv_lut12_group(const seedlm_matrix* const* hs, const void* const* xs,
                            void* const* ys, int n, int xdt, int ydt, hipStream_t s, int phases);
int launch_gemv_mfma(const seedlm_matrix* h, const void* x, void* y, int batch, int xdt, int ydt,
                     hipStream_t s);
// Up to 8 matrices at batch > 1 (fp16): phases & 1 the decode-GEMM launches
// (one per format and tiling present), phases & 2 one reduction launch.
int launch_gemv_mfma_group(const seedlm_matrix* const* hs, const void* const* xs,
                           void* const* ys, int n, int batch, int xdt, int ydt, hipStream_t s,
                           int phases);
// Prefill GEMM (both packed formats, fp16 X and Y; E_UNSUPPORTED otherwise).
int launch_gemm(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, int xdt, int ydt,
                hipStream_t s);
int launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
// Prefill through a decoded fp16 copy of W in a caller workspace and hipBLASLt.
size_t decoded_bytes(const seedlm_matrix* h);
// GEMM scratch offered from a decoded-path workspace, past the decoded matrix.
constexpr size_t kDecodedScratchBytes = 32u << 20;
size_t decoded_workspace_bytes(const seedlm_matrix* h);
int launch_gemm_decoded(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, int xdt,
                        int ydt, void* ws, size_t ws_bytes, hipStream_t s);
int launch_fp16_gemv(const void* W, const void* x, void* y, int64_t rows, int64_t cols,
                     int batch, hipStream_t s);
int build_ext_table(seedlm_matrix* h);
// Seed search: per-seed QR table (bytes for format C) and the search itself.
bool encoder_format_supported(int C, int P, int K, int Q);
size_t encoder_table_bytes(int C, int P, int K, int Q);
int launch_seed_table(int C, int P, int K, int Q, void* table, hipStream_t s);
int launch_encode(int C, int P, int K, int Q, const void* table, const void* W, int64_t rows,
                  int64_t cols, void* seeds, int8_t* coeffs, int8_t* exps, float* err,
                  hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace seedlm

#define SEEDLM_HIP_CHECK(expr)                 \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return SEEDLM_E_DEVICE; \
  } while (0)
