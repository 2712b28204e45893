// Internal declarations shared by the host packer, the launch wrappers and the
// HIP kernels of libseedlm.  Not part of the public ABI (see include/seedlm.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/seedlm.h"
#include "../../include/seedlm_bench.h"

namespace seedlm {

// Packed layout constants (documented in include/seedlm.h).
constexpr int kPanelBlocks = 32;  // blocks per panel of the C = 8 formats
constexpr int kGroup = 4;         // slots per rotated group (one 16-byte load)
constexpr int kStateBits = 16;    // K of the two formats the fast kernels take
constexpr uint32_t kHalf = 1u << (kStateBits - 1);
constexpr uint32_t kPadWord = 0x00000001u;  // seed 1, t = 0, g = 0

// Blocks per panel: a panel row is 128 bytes of words for C = 8 and 64 bytes
// for C = 12, so that the batch-1 kernels' column unit (32 and 16 blocks) reads
// whole contiguous rows.
__host__ __device__ constexpr int panel_blocks(int C) { return C == 8 ? 32 : 16; }

// The packed formats (C, P, K) and their coefficient width Q: the word holds
// the seed in bits 0..K-1 and t_j in bits K+Q*j .. K+Q*j+Q-1; C = 8 formats
// keep g in bits 28..31, C = 12 formats in a nibble array.  0 = unsupported.
__host__ __device__ constexpr int packed_q(int C, int P, int K) {
  return (C == 8 && P == 3 && K == 16) || (C == 12 && P == 4 && K == 16) ||
                 (C == 12 && P == 3 && K == 20)
             ? 4
             : (C == 8 && P == 4 && K == 16 ? 3 : 0);
}

}  // namespace seedlm

// The handle.  Immutable after seedlm_pack: it owns the packed buffer and
// nothing else, so calls that share it may run concurrently.
struct seedlm_matrix {
  int64_t rows = 0, cols = 0;
  int C = 0, P = 0, K = 0, Q = 0;
  int pb = 0;           // blocks per panel (panel_blocks(C))
  int64_t nb = 0;       // blocks per row
  int64_t nbs = 0;      // stored blocks per row (last panel padded to 4 slots)
  int64_t np = 0;       // panels per row: ceil(nb / pb)
  int64_t Mp = 0;       // rows padded to a multiple of 8
  int64_t nwords = 0;   // Mp * nbs
  size_t bytes = 0;     // packed buffer size
  size_t exp_off = 0;   // byte offset of the exponent nibble array (C == 12)
  int device = 0;
  void* d_buf = nullptr;      // packed buffer (device)
  // The pages' formats, which the table-lookup and matrix-core kernels take;
  // the other packed formats run the exact per-lane kernel.
  bool is_4bit() const { return C == 8 && P == 3 && K == 16; }
  bool is_3bit() const { return C == 12 && P == 4 && K == 16; }
};

// An encoder: the per-seed table of one format on one device.
struct seedlm_encoder {
  int C = 0, P = 0, K = 0, Q = 0;
  int device = 0;
  void* d_table = nullptr;
  size_t table_bytes = 0;
};

namespace seedlm {

// Layout helpers (host and device), PB = blocks per panel.  Rows are padded to
// Mp = 8*ceil(rows/8).  Panel p holds blocks PB*p .. PB*p+Wp-1; its stored
// width is Wp rounded up to a multiple of 4.  Panel p starts at word p*Mp*PB
// and stores its Mp rows one after another; inside a row, slot q sits at
// 4*(q/4) + ((q - r) mod 4), so the four words of one 16-byte load hold the
// group's slots rotated by the row.
__host__ __device__ inline int64_t panel_width(int64_t p, int64_t nb, int PB) {
  int64_t w = nb - (int64_t)PB * p;
  return w < PB ? w : PB;
}

__host__ __device__ inline int64_t panel_stored_width(int64_t p, int64_t nb, int PB) {
  return (panel_width(p, nb, PB) + kGroup - 1) / kGroup * kGroup;
}

__host__ __device__ inline int64_t padded_rows(int64_t rows) { return (rows + 7) / 8 * 8; }

__host__ __device__ inline int64_t word_index(int64_t r, int64_t b, int64_t Mp, int64_t nb,
                                              int PB) {
  const int64_t p = b / PB, q = b % PB;
  return p * Mp * PB + r * panel_stored_width(p, nb, PB) + (q & ~(int64_t)3) + ((q - r) & 3);
}

// Index of the uint16 that holds the exponent nibbles of (r, b)'s group, and the
// nibble number inside it (C = 12 formats).
__host__ __device__ inline int64_t exp_index(int64_t r, int64_t b, int64_t Mp, int64_t nb,
                                             int PB) {
  const int64_t p = b / PB, q = b % PB;
  return p * Mp * (PB / kGroup) + r * (panel_stored_width(p, nb, PB) / kGroup) + q / kGroup;
}
__host__ __device__ inline int exp_nibble(int64_t r, int64_t b, int PB) {
  return (int)(((b % PB) - r) & 3);
}

// Launch wrappers implemented in the .hip files.  All return a status code.
//
// The batch-1 table-lookup kernels and the matrix-core kernel split a matrix's
// reduction over workgroups and write fp32 partials, which a second launch adds
// in a fixed order.  The partials live in caller-side scratch, not in the
// handle: *_partial_floats gives the floats one matrix needs, and the group
// launches take one partial pointer per matrix (`partials`, device memory).
int launch_decode(const seedlm_matrix* h, float* W, hipStream_t s);
int launch_gemv_simple(const seedlm_matrix* h, const void* x, void* y, int batch, int xdt,
                       int ydt, hipStream_t s);
int64_t lut_partial_floats(const seedlm_matrix* h);    // 4-bit, batch 1
int64_t lut12_partial_floats(const seedlm_matrix* h);  // 3-bit, batch 1
int64_t mfma_partial_floats(const seedlm_matrix* h, int batch);  // 0 when unsplit
// Up to 8 batch-1 4-bit matrices in one main launch (phases & 1: panel
// partials) and one reduce launch (phases & 2: y).  ext_table: NULL for the
// GF(2) byte tables in LDS, or the 2^16-entry table of extension bits.
int launch_gemv_lut_group(const seedlm_matrix* const* hs, const void* const* xs, void* const* ys,
                          float* const* partials, int n, int xdt, int ydt,
                          const uint32_t* ext_table, hipStream_t s, int phases);
int launch_gemv_lut12_group(const seedlm_matrix* const* hs, const void* const* xs,
                            void* const* ys, float* const* partials, int n, int xdt, int ydt,
                            hipStream_t s, int phases);
// Direct kernel (any packed format, batch 1..16, any dtypes): whole rows per
// workgroup, no partials, one launch.  direct_fits: x of the call fits its LDS.
bool direct_fits(const seedlm_matrix* h, int batch);
int launch_gemv_direct_group(const seedlm_matrix* const* hs, const void* const* xs,
                             void* const* ys, int n, int batch, int xdt, int ydt, hipStream_t s);
// Up to 8 matrices at batch > 1 (fp16): phases & 1 the decode-GEMM launches
// (one per format and tiling present), phases & 2 one reduction launch.
int launch_gemv_mfma_group(const seedlm_matrix* const* hs, const void* const* xs,
                           void* const* ys, float* const* partials, int n, int batch, int xdt,
                           int ydt, hipStream_t s, int phases);
// Prefill GEMM (both packed formats, fp16 X and Y): check_gemm gives
// E_UNSUPPORTED for what the kernels do not take, gemm_scratch_bytes the
// partial tiles a call writes (0 when it splits no tile), and launch_gemm runs
// a checked call with that much scratch at `part`.
int check_gemm(const seedlm_matrix* h, const void* x, int64_t ntok, int xdt, int ydt);
size_t gemm_scratch_bytes(const seedlm_matrix* h, int64_t ntok);
int launch_gemm(const seedlm_matrix* h, const void* x, void* y, int64_t ntok, float* part,
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
// The 2^16-entry table of extension bits (TABLE variant), one per device: built
// by the first seedlm_pack on a device; NULL before that.
int ensure_ext_table(int device);
const uint32_t* ext_table(int device);
// Seed search: per-seed QR table (bytes for format C) and the search itself.
bool encoder_format_supported(int C, int P, int K, int Q);
size_t encoder_table_bytes(int C, int P, int K, int Q);
int launch_seed_table(int C, int P, int K, int Q, void* table, hipStream_t s);
int launch_encode(int C, int P, int K, int Q, const void* table, const void* W, int64_t rows,
                  int64_t cols, void* seeds, int8_t* coeffs, int8_t* exps, float* err,
                  hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Timing of the main (decode-GEMV) kernels of one gemv call, for measurement
// only (seedlm_bench_time_next_call).  While a call launches its main kernels,
// main_launch_events() hands out the caller's events: the start event to the
// first main launch (recorded when that kernel starts), the stop event to every
// main launch (the last record wins, at the end of the last kernel).  Both are
// null when no timing was asked for.  Per host thread.
void main_launch_events(hipEvent_t* start, hipEvent_t* stop);

}  // namespace seedlm

#define SEEDLM_HIP_CHECK(expr)                 \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return SEEDLM_E_DEVICE; \
  } while (0)
