// Host-side driver for the sanitizer test (test_host_sanitizers.py).  It is
// linked against host-only objects of every library source built with
// AddressSanitizer and UndefinedBehaviorSanitizer, and runs the parts of the
// C-ABI that need no GPU:
//
//   host_abi_check pack <in> <out>
//       reads one record set (int64 rows, cols; int32 C, P, K; seeds as uint16
//       for K <= 16 else uint32; coefficients int8 [rows][nb][P]; exponents int8
//       [rows][nb]) into heap buffers of exactly their size, runs
//       seedlm_pack_host into an exactly sized destination (after checking the
//       size query and the too-small-buffer error) and writes the packed bytes.
//   host_abi_check abi
//       calls every entry point with null or out-of-range arguments and checks
//       the status each documents, without touching a device.
//
// Exit status 0 when every check holds; a sanitizer report aborts the run.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "seedlm.h"
#include "seedlm_bench.h"

namespace {

int g_failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    ++g_failures;
  }
}

// Reads exactly n bytes into a fresh heap block of exactly n bytes (at least 1).
void* read_exact(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p || (n && fread(p, 1, n, f) != n)) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

int run_pack(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (!f) return 2;
  int64_t dims[2];
  int32_t fmt[3];
  if (fread(dims, sizeof dims, 1, f) != 1 || fread(fmt, sizeof fmt, 1, f) != 1) return 2;
  const int64_t rows = dims[0], cols = dims[1];
  const int C = fmt[0], P = fmt[1], K = fmt[2];
  const int64_t nb = (cols + C - 1) / C;
  const size_t seed_bytes = (size_t)(rows * nb) * (K <= 16 ? 2 : 4);
  void* seeds = read_exact(f, seed_bytes);
  int8_t* coeffs = static_cast<int8_t*>(read_exact(f, (size_t)(rows * nb * P)));
  int8_t* exps = static_cast<int8_t*>(read_exact(f, (size_t)(rows * nb)));
  fclose(f);

  size_t bytes = 0;
  expect("pack_host size query", seedlm_pack_host(seeds, coeffs, exps, rows, cols, C, P, K,
                                                  nullptr, &bytes), SEEDLM_OK);
  const size_t need = bytes;
  unsigned char* dst = static_cast<unsigned char*>(malloc(need));
  size_t small = need - 1;
  expect("pack_host short buffer", seedlm_pack_host(seeds, coeffs, exps, rows, cols, C, P, K,
                                                    dst, &small), SEEDLM_E_INVALID);
  if (small != need) {
    fprintf(stderr, "FAIL short buffer reports %zu bytes, expected %zu\n", small, need);
    ++g_failures;
  }
  bytes = need;
  expect("pack_host", seedlm_pack_host(seeds, coeffs, exps, rows, cols, C, P, K, dst, &bytes),
         SEEDLM_OK);
  FILE* o = fopen(out_path, "wb");
  if (!o || fwrite(dst, 1, need, o) != need) return 2;
  fclose(o);
  free(dst);
  free(seeds);
  free(coeffs);
  free(exps);
  return g_failures ? 1 : 0;
}

int run_abi() {
  const int codes[] = {SEEDLM_OK, SEEDLM_E_INVALID, SEEDLM_E_UNSUPPORTED, SEEDLM_E_NOMEM,
                       SEEDLM_E_DEVICE, SEEDLM_E_SCRATCH_LIMIT, 7, -1000};
  for (int c : codes) {
    const char* s = seedlm_status_string(c);
    if (!s || !*s) {
      fprintf(stderr, "FAIL status string for %d\n", c);
      ++g_failures;
    }
  }

  // One valid 4-bit record set of 2 x 11 (two blocks per row, the second ragged).
  uint16_t seeds[4] = {1, 2, 0xFFFF, 77};
  int8_t coeffs[12] = {0, 1, -1, 7, -8, 3, 2, 2, 2, -3, 4, 5};
  int8_t exps[4] = {0, -15, -3, -7};
  size_t bytes = 0;
  expect("pack_host null bytes",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr, nullptr), SEEDLM_E_INVALID);
  expect("pack_host null seeds",
         seedlm_pack_host(nullptr, coeffs, exps, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  expect("pack_host null coeffs",
         seedlm_pack_host(seeds, nullptr, exps, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  expect("pack_host null exps",
         seedlm_pack_host(seeds, coeffs, nullptr, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  expect("pack_host zero rows",
         seedlm_pack_host(seeds, coeffs, exps, 0, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  expect("pack_host negative cols",
         seedlm_pack_host(seeds, coeffs, exps, 2, -5, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  expect("pack_host rows beyond 2^30",
         seedlm_pack_host(seeds, coeffs, exps, (1LL << 31), 11, 8, 3, 16, nullptr, &bytes),
         SEEDLM_E_INVALID);
  expect("pack_host unknown format",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 5, 16, nullptr, &bytes),
         SEEDLM_E_UNSUPPORTED);
  expect("pack_host C = 12 with K = 16 and P = 3",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 12, 3, 16, nullptr, &bytes),
         SEEDLM_E_UNSUPPORTED);
  expect("pack_host valid", seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr, &bytes),
         SEEDLM_OK);
  seeds[2] = 0;
  expect("pack_host zero seed",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  seeds[2] = 5;
  coeffs[11] = 8;
  expect("pack_host coefficient 8",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  coeffs[11] = 5;
  int8_t c3[8] = {0, 1, 2, 3, -4, -3, 3, -5};
  expect("pack_host 3-bit coefficient -5",
         seedlm_pack_host(seeds, c3, exps, 1, 11, 8, 4, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  c3[7] = -4;
  expect("pack_host 3-bit valid",
         seedlm_pack_host(seeds, c3, exps, 1, 11, 8, 4, 16, nullptr, &bytes), SEEDLM_OK);
  exps[3] = 1;
  expect("pack_host exponent 1",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  exps[3] = -16;
  expect("pack_host exponent -16",
         seedlm_pack_host(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr, &bytes), SEEDLM_E_INVALID);
  exps[3] = -7;
  uint32_t wide[2] = {1u << 20, 3};
  int8_t c12[8] = {0, 0, 0, 0, 0, 0};
  int8_t e12[2] = {0, 0};
  expect("pack_host 20-bit seed out of range",
         seedlm_pack_host(wide, c12, e12, 1, 24, 12, 3, 20, nullptr, &bytes), SEEDLM_E_INVALID);

  seedlm_handle h = reinterpret_cast<seedlm_handle>(0x1);
  expect("pack null out", seedlm_pack(seeds, coeffs, exps, 2, 11, 8, 3, 16, nullptr),
         SEEDLM_E_INVALID);
  exps[3] = 1;
  expect("pack bad record", seedlm_pack(seeds, coeffs, exps, 2, 11, 8, 3, 16, &h),
         SEEDLM_E_INVALID);
  exps[3] = -7;
  if (h != nullptr) {
    fprintf(stderr, "FAIL pack leaves *out set on error\n");
    ++g_failures;
  }

  float xbuf[16] = {0};
  float ybuf[16] = {0};
  const void* xs[1] = {xbuf};
  void* ys[1] = {ybuf};
  seedlm_handle none[1] = {nullptr};
  expect("gemv null handle", seedlm_gemv(nullptr, xbuf, ybuf, 1, SEEDLM_F32, SEEDLM_F32, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv batch 0", seedlm_gemv(nullptr, xbuf, ybuf, 0, SEEDLM_F32, SEEDLM_F32, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv batch above maximum",
         seedlm_gemv(nullptr, xbuf, ybuf, SEEDLM_MAX_BATCH + 1, SEEDLM_F32, SEEDLM_F32, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv unknown dtype", seedlm_gemv(nullptr, xbuf, ybuf, 1, 9, SEEDLM_F32, nullptr),
         SEEDLM_E_UNSUPPORTED);
  expect("gemv null x", seedlm_gemv(nullptr, nullptr, ybuf, 1, SEEDLM_F32, SEEDLM_F32, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv_variant null handle",
         seedlm_gemv_variant(nullptr, xbuf, ybuf, 1, SEEDLM_F16, SEEDLM_F16, SEEDLM_VARIANT_LUT,
                             nullptr),
         SEEDLM_E_INVALID);
  expect("gemv_many null arrays",
         seedlm_gemv_many(nullptr, xs, ys, 1, 1, SEEDLM_F32, SEEDLM_F32, nullptr), SEEDLM_E_INVALID);
  expect("gemv_many negative n",
         seedlm_gemv_many(none, xs, ys, -1, 1, SEEDLM_F32, SEEDLM_F32, nullptr), SEEDLM_E_INVALID);
  expect("gemv_many null entry",
         seedlm_gemv_many(none, xs, ys, 1, 1, SEEDLM_F32, SEEDLM_F32, nullptr), SEEDLM_E_INVALID);
  expect("gemv_many empty", seedlm_gemv_many(none, xs, ys, 0, 1, SEEDLM_F32, SEEDLM_F32, nullptr),
         SEEDLM_OK);
  expect("gemv_many_begin null entry",
         seedlm_gemv_many_begin(none, xs, ys, 1, 1, SEEDLM_F16, SEEDLM_F16, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv_many_end null entry",
         seedlm_gemv_many_end(none, xs, ys, 1, 1, SEEDLM_F16, SEEDLM_F16, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv_many_noalloc null entry",
         seedlm_gemv_many_noalloc(none, xs, ys, 1, 1, SEEDLM_F16, SEEDLM_F16, nullptr),
         SEEDLM_E_INVALID);
  expect("gemv_many_noalloc empty",
         seedlm_gemv_many_noalloc(none, xs, ys, 0, 1, SEEDLM_F16, SEEDLM_F16, nullptr), SEEDLM_OK);
  size_t sb = 123;
  expect("scratch_bytes null out",
         seedlm_gemv_scratch_bytes(none, 1, 1, SEEDLM_F16, SEEDLM_F16, nullptr), SEEDLM_E_INVALID);
  expect("scratch_bytes null entry",
         seedlm_gemv_scratch_bytes(none, 1, 1, SEEDLM_F16, SEEDLM_F16, &sb), SEEDLM_E_INVALID);
  expect("scratch_bytes bad batch",
         seedlm_gemv_scratch_bytes(none, 0, 0, SEEDLM_F16, SEEDLM_F16, &sb), SEEDLM_E_INVALID);
  expect("scratch_bytes empty", seedlm_gemv_scratch_bytes(none, 0, 1, SEEDLM_F16, SEEDLM_F16, &sb),
         SEEDLM_OK);
  if (sb != 0) {
    fprintf(stderr, "FAIL scratch_bytes of no matrices is %zu\n", sb);
    ++g_failures;
  }
  int ev = 0;
  expect("bench_time_next_call one event", seedlm_bench_time_next_call(&ev, nullptr),
         SEEDLM_E_INVALID);
  expect("bench_time_next_call cancel", seedlm_bench_time_next_call(nullptr, nullptr), SEEDLM_OK);

  expect("decode null handle", seedlm_decode(nullptr, xbuf, nullptr), SEEDLM_E_INVALID);
  expect("destroy null", seedlm_destroy(nullptr), SEEDLM_OK);
  seedlm_info_t info;
  expect("info null handle", seedlm_info(nullptr, &info), SEEDLM_E_INVALID);
  expect("export null handle", seedlm_export(nullptr, nullptr, &sb), SEEDLM_E_INVALID);
  expect("gemm null handle", seedlm_gemm(nullptr, xbuf, ybuf, 4, SEEDLM_F16, SEEDLM_F16, nullptr),
         SEEDLM_E_INVALID);
  expect("gemm_scratch_bytes null handle", seedlm_gemm_scratch_bytes(nullptr, 4, &sb),
         SEEDLM_E_INVALID);
  expect("gemm_decoded_bytes null handle", seedlm_gemm_decoded_bytes(nullptr, &sb),
         SEEDLM_E_INVALID);
  expect("gemm_decoded null handle",
         seedlm_gemm_decoded(nullptr, xbuf, ybuf, 4, SEEDLM_F16, SEEDLM_F16, ybuf, 64, nullptr),
         SEEDLM_E_INVALID);
  expect("stream_read null", seedlm_stream_read(nullptr, 16, nullptr, nullptr), SEEDLM_E_INVALID);
  expect("stream_read odd size", seedlm_stream_read(xbuf, 20, nullptr, nullptr), SEEDLM_E_INVALID);
  expect("fp16_gemv cols not a multiple of 8",
         seedlm_fp16_gemv(xbuf, xbuf, ybuf, 4, 12, 1, nullptr), SEEDLM_E_INVALID);
  expect("fp16_gemv batch 0", seedlm_fp16_gemv(xbuf, xbuf, ybuf, 4, 16, 0, nullptr),
         SEEDLM_E_INVALID);

  seedlm_encoder_handle e = nullptr;
  expect("encoder_create null out", seedlm_encoder_create(8, 3, 16, 4, nullptr), SEEDLM_E_INVALID);
  expect("encoder_create unknown format", seedlm_encoder_create(8, 9, 16, 4, &e),
         SEEDLM_E_UNSUPPORTED);
  expect("encoder_destroy null", seedlm_encoder_destroy(nullptr), SEEDLM_OK);
  int8_t cc[4], ee[4];
  expect("encode null encoder", seedlm_encode(nullptr, xbuf, 1, 8, seeds, cc, ee, nullptr, nullptr),
         SEEDLM_E_INVALID);

  printf("abi checks: %d failure(s)\n", g_failures);
  return g_failures ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc == 4 && strcmp(argv[1], "pack") == 0) return run_pack(argv[2], argv[3]);
  if (argc == 2 && strcmp(argv[1], "abi") == 0) return run_abi();
  fprintf(stderr, "usage: host_abi_check pack <in> <out> | abi\n");
  return 2;
}
