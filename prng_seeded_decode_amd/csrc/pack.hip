// Host packer and handle management of libseedlm.
//
// The packed buffer holds one 32-bit word per block {seed, coefficients,
// biased shared exponent} (C = 8 formats) or {seed, coefficients} plus a nibble
// array of exponents (C = 12 formats), grouped into panels of 32 (C = 8) or 16
// (C = 12) blocks whose rows hold groups of four slots rotated by the row
// index.  The record itself is the pages' {seed s, coefficients t, shared
// exponent} (atlas.scime.ai "Approach"; paperhub.cn rebuttal on shared
// exponents); the bit positions and the panel order are this library's.
#include <stdlib.h>
#include <string.h>

#include <new>
#include <vector>

#include "seedlm_internal.h"

using namespace seedlm;

namespace {

struct Layout {
  int Q, PB;
  int64_t nb, nbs, np, Mp, nwords;
  size_t exp_off, bytes;
};

Layout make_layout(int64_t rows, int64_t cols, int C, int P, int K) {
  Layout L;
  L.Q = packed_q(C, P, K);
  L.PB = panel_blocks(C);
  L.nb = (cols + C - 1) / C;
  L.np = (L.nb + L.PB - 1) / L.PB;
  L.nbs = (L.np - 1) * L.PB + panel_stored_width(L.np - 1, L.nb, L.PB);
  L.Mp = padded_rows(rows);
  L.nwords = L.Mp * L.nbs;
  if (C == 8) {
    L.exp_off = 0;
    L.bytes = (size_t)L.nwords * 4;
  } else {
    L.exp_off = ((size_t)L.nwords * 4 + 255) / 256 * 256;
    L.bytes = L.exp_off + (size_t)(L.nwords / kGroup) * 2;
  }
  return L;
}

// Seed k of the record arrays: uint16 for K <= 16, uint32 above.
uint32_t seed_at(const void* seeds, int K, int64_t k) {
  return K <= 16 ? static_cast<const uint16_t*>(seeds)[k] : static_cast<const uint32_t*>(seeds)[k];
}

int validate(const void* seeds, const int8_t* coeffs, const int8_t* exps, int64_t rows,
             int64_t cols, int C, int P, int K) {
  if (!seeds || !coeffs || !exps) return SEEDLM_E_INVALID;
  if (rows <= 0 || cols <= 0) return SEEDLM_E_INVALID;
  const int Q = packed_q(C, P, K);
  if (Q == 0) return SEEDLM_E_UNSUPPORTED;
  // Keep every index of the layout (and of the kernels' 32-bit row math) in range.
  if (rows > (1LL << 30) || cols > (1LL << 30)) return SEEDLM_E_INVALID;
  const int64_t nb = (cols + C - 1) / C;
  const int64_t n = rows * nb;
  for (int64_t k = 0; k < n; ++k) {
    const uint32_t s = seed_at(seeds, K, k);
    if (s == 0 || s >= (1u << K)) return SEEDLM_E_INVALID;
    if (exps[k] < -15 || exps[k] > 0) return SEEDLM_E_INVALID;
  }
  const int lo = -(1 << (Q - 1)), hi = (1 << (Q - 1)) - 1;
  for (int64_t k = 0; k < n * P; ++k)
    if (coeffs[k] < lo || coeffs[k] > hi) return SEEDLM_E_INVALID;
  return SEEDLM_OK;
}

void write_layout(const void* seeds, const int8_t* coeffs, const int8_t* exps, int64_t rows,
                  int C, int P, int K, const Layout& L, uint8_t* dst) {
  uint32_t* words = reinterpret_cast<uint32_t*>(dst);
  for (int64_t k = 0; k < L.nwords; ++k) words[k] = kPadWord;
  uint16_t* ex = nullptr;
  if (C == 12) {
    memset(dst + (size_t)L.nwords * 4, 0, L.exp_off - (size_t)L.nwords * 4);
    ex = reinterpret_cast<uint16_t*>(dst + L.exp_off);
    memset(ex, 0, L.bytes - L.exp_off);
  }
  const uint32_t qmask = (1u << L.Q) - 1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < L.nb; ++b) {
      const int64_t k = r * L.nb + b;
      uint32_t w = seed_at(seeds, K, k);
      for (int j = 0; j < P; ++j)
        w |= ((uint32_t)coeffs[k * P + j] & qmask) << (K + L.Q * j);
      const uint32_t g = (uint32_t)(exps[k] + 15);
      if (C == 8) {
        w |= g << 28;
      } else {
        ex[exp_index(r, b, L.Mp, L.nb, L.PB)] |= (uint16_t)(g << (4 * exp_nibble(r, b, L.PB)));
      }
      words[word_index(r, b, L.Mp, L.nb, L.PB)] = w;
    }
  }
}

}  // namespace

extern "C" {

const char* seedlm_status_string(int status) {
  switch (status) {
    case SEEDLM_OK: return "ok";
    case SEEDLM_E_INVALID: return "invalid argument";
    case SEEDLM_E_UNSUPPORTED: return "unsupported format or dtype";
    case SEEDLM_E_NOMEM: return "out of memory";
    case SEEDLM_E_DEVICE: return "HIP runtime error";
    case SEEDLM_E_SCRATCH_LIMIT: return "the call needs more scratch than the no-alloc maximum";
    default: return "unknown status";
  }
}

int seedlm_pack_host(const void* seeds, const int8_t* coeffs, const int8_t* exps,
                     int64_t rows, int64_t cols, int C, int P, int K, void* dst,
                     size_t* bytes) {
  if (!bytes) return SEEDLM_E_INVALID;
  int st = validate(seeds, coeffs, exps, rows, cols, C, P, K);
  if (st != SEEDLM_OK) return st;
  const Layout L = make_layout(rows, cols, C, P, K);
  if (!dst) {
    *bytes = L.bytes;
    return SEEDLM_OK;
  }
  if (*bytes < L.bytes) {
    *bytes = L.bytes;
    return SEEDLM_E_INVALID;
  }
  write_layout(seeds, coeffs, exps, rows, C, P, K, L, static_cast<uint8_t*>(dst));
  *bytes = L.bytes;
  return SEEDLM_OK;
}

int seedlm_pack(const void* seeds, const int8_t* coeffs, const int8_t* exps, int64_t rows,
                int64_t cols, int C, int P, int K, seedlm_handle* out) {
  if (!out) return SEEDLM_E_INVALID;
  *out = nullptr;
  int st = validate(seeds, coeffs, exps, rows, cols, C, P, K);
  if (st != SEEDLM_OK) return st;
  const Layout L = make_layout(rows, cols, C, P, K);

  uint8_t* host = nullptr;
  if (hipHostMalloc((void**)&host, L.bytes, hipHostMallocDefault) != hipSuccess)
    return SEEDLM_E_NOMEM;
  write_layout(seeds, coeffs, exps, rows, C, P, K, L, host);

  seedlm_matrix* h = new (std::nothrow) seedlm_matrix();
  if (!h) {
    (void)hipHostFree(host);
    return SEEDLM_E_NOMEM;
  }
  h->rows = rows;
  h->cols = cols;
  h->C = C;
  h->P = P;
  h->K = K;
  h->Q = L.Q;
  h->pb = L.PB;
  h->nb = L.nb;
  h->nbs = L.nbs;
  h->np = L.np;
  h->Mp = L.Mp;
  h->nwords = L.nwords;
  h->bytes = L.bytes;
  h->exp_off = L.exp_off;

  int rc = SEEDLM_OK;
  if (hipGetDevice(&h->device) != hipSuccess) rc = SEEDLM_E_DEVICE;
  if (rc == SEEDLM_OK && hipMalloc(&h->d_buf, L.bytes) != hipSuccess) rc = SEEDLM_E_NOMEM;
  if (rc == SEEDLM_OK && hipMemcpy(h->d_buf, host, L.bytes, hipMemcpyHostToDevice) != hipSuccess)
    rc = SEEDLM_E_DEVICE;
  (void)hipHostFree(host);
  // The device's 2^16-entry extension table (TABLE variant) is built here, once
  // per device, so that no gemv call allocates or synchronises for it.
  if (rc == SEEDLM_OK) rc = ensure_ext_table(h->device);
  if (rc != SEEDLM_OK) {
    seedlm_destroy(h);
    return rc;
  }
  *out = h;
  return SEEDLM_OK;
}

int seedlm_destroy(seedlm_handle h) {
  if (!h) return SEEDLM_OK;
  int rc = SEEDLM_OK;
  if (h->d_buf && hipFree(h->d_buf) != hipSuccess) rc = SEEDLM_E_DEVICE;
  delete h;
  return rc;
}

int seedlm_info(seedlm_handle h, seedlm_info_t* info) {
  if (!h || !info) return SEEDLM_E_INVALID;
  info->rows = h->rows;
  info->cols = h->cols;
  info->C = h->C;
  info->P = h->P;
  info->K = h->K;
  info->blocks_per_row = h->nb;
  info->stored_blocks_per_row = h->nbs;
  info->compressed_bytes = (int64_t)h->bytes;
  info->Q = h->Q;
  return SEEDLM_OK;
}

int seedlm_export(seedlm_handle h, void* host, size_t* bytes) {
  if (!h || !bytes) return SEEDLM_E_INVALID;
  if (!host) {
    *bytes = h->bytes;
    return SEEDLM_OK;
  }
  if (*bytes < h->bytes) {
    *bytes = h->bytes;
    return SEEDLM_E_INVALID;
  }
  SEEDLM_HIP_CHECK(hipMemcpy(host, h->d_buf, h->bytes, hipMemcpyDeviceToHost));
  *bytes = h->bytes;
  return SEEDLM_OK;
}

}  // extern "C"
