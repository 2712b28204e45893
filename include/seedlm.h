/*
 * seedlm.h -- C ABI of the SeedLM decompress-and-multiply library for MI355X (gfx950).
 *
 * The method (SeedLM, "Compressing LLM Weights into Seeds of Pseudo-Random
 * Generators"): each block of C weights is stored as a K-bit seed s, P 4-bit
 * coefficients t and a shared exponent e.  At inference the seed drives a
 * Linear Feedback Shift Register that emits the C x P matrix U(s), and the
 * block is rebuilt as w = 2^e * U(s) * t
 *   - paperdance.org/p/2410.10714, English abstract (seed fed to an LFSR that
 *     generates a random matrix, linearly combined with compressed coefficients);
 *   - atlas.scime.ai summary, "Approach" (blocks of C weights, P columns,
 *     K-bit seed, 4-bit quantized coefficients);
 *   - paperhub.cn OpenReview discussion, rebuttal text for the paragraph before
 *     Eq. (1) (s and t are fetched from memory, weights are rebuilt on the fly
 *     and used to compute activations; no full-precision weights are kept) and
 *     the rebuttal on shared exponents.
 *
 * Format fixed by this library (the pages leave these open):
 *   LFSR      K-bit Fibonacci, right shift: z' = (z >> 1) | (f << (K-1)); for
 *             K = 16, f = bit0 ^ bit2 ^ bit3 ^ bit5 of z (x^16 + x^5 + x^3 +
 *             x^2 + 1); for K = 20, f = bit0 ^ bit3 (x^20 + x^3 + 1); both of
 *             period 2^K - 1.  The seed is the first state, z_0 = s, s != 0.
 *   values    v_n = (z_n - 2^(K-1)) / 2^(K-1).
 *   U(s)      column-major: U[i][j] = v_{j*C + i}, i < C, j < P.
 *   block     w_i = 2^e * sum_j U[i][j] * t_j, t_j Q-bit two's complement
 *             ([-8, 7] for Q = 4), e in [-15, 0].
 *   blocks    lie along a row: block b of row r holds columns b*C .. b*C+C-1;
 *             nb = ceil(cols / C); the last block keeps its first
 *             cols - (nb-1)*C weights.
 *   formats   (C, P, K, Q): (8, 3, 16, 4) 4 bits per weight and (12, 4, 16, 4)
 *             3 bits per weight, the pages' formats; (8, 4, 16, 3) 4 bits and
 *             (12, 3, 20, 4) 3 bits, which spend the same bits on a fourth
 *             latent column with 3-bit coefficients or on a 20-bit seed (the
 *             knobs the pages name below 3 bits: paperhub.cn, answer on
 *             1.5-2.5 bits per weight).  Q follows from (C, P, K).
 *   word      uint32 per block: bits 0..K-1 seed, bits K+Q*j .. K+Q*j+Q-1 t_j;
 *             C = 8: bits 28..31 g = e + 15; C = 12: the word is full and g
 *             sits in a nibble array.
 *   panels    rows are padded to Mp = 8*ceil(rows/8); blocks are grouped in
 *             panels of PB = 32 (C = 8) or PB = 16 (C = 12) blocks: panel p
 *             holds blocks PB*p .. PB*p+Wp-1, Wp = min(PB, nb-PB*p), stored
 *             Wp' = 4*ceil(Wp/4) slots wide.  Padding (rows >= rows, slots
 *             >= Wp) holds pad words 0x00000001 (seed 1, t = 0, g = 0).  Panel
 *             p starts at word p*Mp*PB and stores its Mp rows one after
 *             another, Wp' words each; slot q of row r sits at
 *             4*(q/4) + ((q-r) mod 4) of the row (groups of four slots rotated
 *             by the row index).  For C = 12 the exponent of (r, b) is nibble
 *             ((q-r) mod 4) of uint16 number p*Mp*(PB/4) + r*(Wp'/4) + q/4 of
 *             an array starting at byte align256(4 * total words).
 *   Kernels   every call takes every format; the batch-1 table-lookup and
 *             matrix-core kernels run the pages' two formats, the other two
 *             run the direct per-lane kernel (seedlm_gemv) and seedlm_decode.
 *
 * Conventions: every call returns a status (0 = SEEDLM_OK, negative = error);
 * no C++ exception crosses this boundary.  "device" pointers are HIP device
 * memory of the current device; "host" pointers are ordinary host memory.
 * Streams are hipStream_t passed as void* (NULL = the null stream).  Kernel
 * launches are asynchronous: a fault inside a kernel is reported by the
 * caller's next synchronisation, not by these calls.
 */
#ifndef SEEDLM_H
#define SEEDLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SEEDLM_API __attribute__((visibility("default")))

/* Status codes. */
#define SEEDLM_OK 0
#define SEEDLM_E_INVALID (-1)     /* bad argument: null pointer, range, shape      */
#define SEEDLM_E_UNSUPPORTED (-2) /* (C, P, K) or dtype combination not supported  */
#define SEEDLM_E_NOMEM (-3)       /* host or device allocation failed              */
#define SEEDLM_E_DEVICE (-4)      /* a HIP runtime call failed                     */
#define SEEDLM_E_SCRATCH_LIMIT (-5) /* needs more than the no-alloc scratch maximum */

/* Element types for activations and outputs. */
#define SEEDLM_F32 0
#define SEEDLM_F16 1

/* Largest batch accepted by seedlm_gemv. */
#define SEEDLM_MAX_BATCH 16

typedef struct seedlm_matrix* seedlm_handle;

typedef struct seedlm_info_t {
  int64_t rows;             /* M */
  int64_t cols;             /* N */
  int32_t C, P, K;
  int64_t blocks_per_row;   /* nb = ceil(N / C) */
  int64_t stored_blocks_per_row; /* nb with the last panel padded to 4 slots */
  int64_t compressed_bytes; /* size of the packed buffer, padding included */
  int32_t Q;                /* coefficient width in bits */
} seedlm_info_t;

/*
 * seedlm_pack_host -- write the packed layout into host memory (no GPU use).
 *   seeds  host uint16 [rows][nb] (uint32 for K = 20), each in [1, 2^K - 1]
 *   coeffs host int8   [rows][nb][P], each Q-bit: in [-8, 7], or [-4, 3] for Q = 3
 *   exps   host int8   [rows][nb], each in [-15, 0]
 *   dst    host buffer of *bytes bytes, or NULL to query the size.
 * On entry *bytes is the capacity of dst; on return it is the layout size.
 * Errors: SEEDLM_E_INVALID (null pointers, rows/cols <= 0, out-of-range
 * record, dst too small), SEEDLM_E_UNSUPPORTED ((C,P,K) not supported).
 * Source: the per-block record {seed, coefficients, shared exponent} of the
 * pages (atlas.scime.ai "Approach"; paperhub.cn rebuttal on shared exponents).
 */
SEEDLM_API int seedlm_pack_host(const void* seeds, const int8_t* coeffs,
                                const int8_t* exps, int64_t rows, int64_t cols,
                                int C, int P, int K, void* dst, size_t* bytes);

/*
 * seedlm_pack -- validate and pack records, upload them to the current device
 * and return a handle that owns the device copy and nothing else: the device
 * memory of a packed matrix is its compressed bytes (seedlm_info).  The handle
 * is immutable, so any calls may share it concurrently.  Synchronous.  The
 * caller keeps ownership of the host arrays (layouts as for seedlm_pack_host).
 * The first pack on a device also builds that device's 256 KiB table of LFSR
 * extension bits (a measurement variant reads it; seedlm_bench.h).
 * Errors: as seedlm_pack_host, plus SEEDLM_E_NOMEM and SEEDLM_E_DEVICE.
 * Source: as seedlm_pack_host.
 */
SEEDLM_API int seedlm_pack(const void* seeds, const int8_t* coeffs,
                           const int8_t* exps, int64_t rows, int64_t cols,
                           int C, int P, int K, seedlm_handle* out);

/*
 * seedlm_gemv -- y = W x for a batch of activation vectors, with W rebuilt from
 * the handle's seeds and coefficients inside the kernel and never stored
 * (paperhub.cn rebuttal text before Eq. (1): weights are reconstructed on the
 * fly from s and t and used to compute the activations).
 *   x  device [batch][cols], x_dtype SEEDLM_F32 or SEEDLM_F16 (row-major)
 *   y  device [batch][rows], y_dtype SEEDLM_F32 or SEEDLM_F16 (fp16: round to
 *      nearest even); both caller-owned.
 *   batch in [1, SEEDLM_MAX_BATCH].  batch 1 runs the fused decode-GEMV
 *   (activation-side table lookups; small matrices, the direct kernel); batch
 *   > 1 with fp16 x and y decodes each weight tile once and contracts it on
 *   the matrix cores in fp16 with fp32 accumulation; fp32 x or y at batch > 1,
 *   and the two extra formats, run the direct kernel, which rebuilds every
 *   weight exactly in fp32 and needs no scratch.
 * Asynchronous on `stream`.  The kernels that split a row's reduction over
 * workgroups write fp32 partials into scratch that the library keeps per
 * (device, stream): calls on one stream share it in stream order, and calls on
 * different streams -- with the same handle or not -- use different scratch, so
 * they may overlap.  The first call on a stream, or one that needs more
 * scratch than any earlier call on that stream, allocates it (hipMalloc: not
 * inside graph capture, so run one call on a stream before capturing it);
 * outgrown scratch stays allocated, so graphs captured from earlier calls stay
 * valid, until seedlm_scratch_release frees all of it.
 * seedlm_gemv_scratch_bytes gives a call's size.  Call with the device h was
 * packed on current.  Inputs must be finite.
 * Errors: SEEDLM_E_INVALID (null, batch out of range, another device current),
 * SEEDLM_E_UNSUPPORTED (dtype), SEEDLM_E_NOMEM (scratch), SEEDLM_E_DEVICE
 * (launch failure).
 */
SEEDLM_API int seedlm_gemv(seedlm_handle h, const void* x, void* y, int batch,
                           int x_dtype, int y_dtype, void* stream);

/*
 * seedlm_gemv_many -- y[i] = W_i x[i] for n matrices, the same results as n
 * calls of seedlm_gemv on `stream`.  Up to 8 consecutive matrices are run
 * together -- at batch 1
 * those of one format, at batch > 1 with fp16 x and y any of them -- so that
 * small matrices share the GPU and the per-launch cost is paid once; a decoder
 * layer's q/k/v/o/gate/up/down is the intended use (the pages' inference step,
 * applied to every weight matrix: paperhub.cn rebuttal text before Eq. (1)).
 *   handles  host array of n handles (a handle may appear more than once)
 *   x, y     host arrays of n device pointers, layouts as for seedlm_gemv
 * Scratch as for seedlm_gemv: the partials of all n matrices, on `stream`.
 * Errors: as seedlm_gemv.
 */
SEEDLM_API int seedlm_gemv_many(const seedlm_handle* handles, const void* const* x,
                                void* const* y, int n, int batch, int x_dtype, int y_dtype,
                                void* stream);

/*
 * seedlm_gemv_many_begin / seedlm_gemv_many_end -- seedlm_gemv_many split in
 * two: _begin runs the fused decode-GEMV kernels (per-panel or per-chunk row
 * partials into the stream's scratch), _end adds the partials into y.  Called
 * with identical arguments on one stream they equal seedlm_gemv_many; the
 * split lets a caller time the two halves.  Between the two calls no other
 * gemv or gemm call may use that stream (it would reuse the scratch).
 */
SEEDLM_API int seedlm_gemv_many_begin(const seedlm_handle* handles, const void* const* x,
                                      void* const* y, int n, int batch, int x_dtype,
                                      int y_dtype, void* stream);
SEEDLM_API int seedlm_gemv_many_end(const seedlm_handle* handles, const void* const* x,
                                    void* const* y, int n, int batch, int x_dtype, int y_dtype,
                                    void* stream);

/*
 * seedlm_gemv_many_noalloc -- seedlm_gemv_many for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, results and arguments,
 * with the partials in a fixed scratch array of SEEDLM_NOALLOC_SCRATCH_BYTES
 * that every device the library runs on holds until the process ends (its
 * device address is looked up once per device, on the first call there).  No
 * hipMalloc, hipFree or other allocating call is made.  The array is shared by
 * every call on a device and keeps the last call's contents: calls that
 * overlap in time on one device race (serialise them, e.g. on one stream).
 * Nothing in it needs clearing between calls.  A call whose partials exceed
 * the array (seedlm_gemv_scratch_bytes) returns SEEDLM_E_SCRATCH_LIMIT before
 * launching anything: every batch-1 call on a Llama-3-70B layer fits (13.4 MB),
 * and its batch-8 call (41 MB).
 * Errors: as seedlm_gemv_many, and SEEDLM_E_SCRATCH_LIMIT.
 */
#define SEEDLM_NOALLOC_SCRATCH_BYTES (64u << 20)
SEEDLM_API int seedlm_gemv_many_noalloc(const seedlm_handle* handles, const void* const* x,
                                        void* const* y, int n, int batch, int x_dtype,
                                        int y_dtype, void* stream);

/*
 * seedlm_gemv_scratch_bytes -- the scratch bytes seedlm_gemv_many(handles, n,
 * batch, x_dtype, y_dtype) needs on its stream (0 when no kernel of the call
 * splits a reduction).  Host only; no GPU use.  A layer's batch-1 call needs
 * 4 bytes per (32-block panel, row) of each matrix: 13.4 MB for a Llama-3-70B
 * layer beside its 428 MB of packed weights.
 * Errors: SEEDLM_E_INVALID (null, batch), SEEDLM_E_UNSUPPORTED (dtype).
 */
SEEDLM_API int seedlm_gemv_scratch_bytes(const seedlm_handle* handles, int n, int batch,
                                         int x_dtype, int y_dtype, size_t* bytes);

/*
 * seedlm_scratch_release -- free the gemv and gemm scratch of every stream on
 * every device (each device is synchronised first; graphs captured from earlier
 * calls must not be replayed afterwards).  Later calls allocate again.  Call
 * it after destroying a stream that gemv or gemm calls used, before a new
 * stream could take over its handle value.  Errors: SEEDLM_E_DEVICE.
 */
SEEDLM_API int seedlm_scratch_release(void);

/*
 * seedlm_decode -- write the dense weights W[rows][cols] as fp32 (row-major,
 * caller-owned device memory).  Bit-exact: the block's integer sum times a
 * power of two is exact in fp32.  Asynchronous on `stream`; no scratch.  Call
 * with the device h was packed on current.
 * Source: the block reconstruction of the abstract (paperdance.org) and the
 * "Approach" section (atlas.scime.ai).
 * Errors: SEEDLM_E_INVALID (null, another device current), SEEDLM_E_DEVICE.
 */
SEEDLM_API int seedlm_decode(seedlm_handle h, float* W_out, void* stream);

/* seedlm_destroy -- free the handle's device memory; NULL is a no-op. */
SEEDLM_API int seedlm_destroy(seedlm_handle h);

/* seedlm_info -- shape, format and compressed size of a packed matrix. */
SEEDLM_API int seedlm_info(seedlm_handle h, seedlm_info_t* info);

/* seedlm_export -- copy the packed buffer back to host memory (synchronous).
 * On entry *bytes is the capacity of host (host may be NULL to query). */
SEEDLM_API int seedlm_export(seedlm_handle h, void* host, size_t* bytes);

/* seedlm_status_string -- a static message for a status code. */
SEEDLM_API const char* seedlm_status_string(int status);

/*
 * seedlm_gemm -- Y = X W^T for any number of activation rows (prefill), with W
 * rebuilt from the handle's records inside the kernel and never stored in HBM
 * (paperhub.cn rebuttal text before Eq. (1): weights are reconstructed on the
 * fly from s and t and used to compute the activations).  Each 128-row tile of
 * W is decoded exactly once per 256 or 512 activation rows and contracted on
 * the matrix cores (fp16 operands, fp32 accumulation).  Where the tiles would
 * leave over half of the compute units idle in the last round of workgroups
 * (or a small matrix has too few tiles to fill them), those tiles split their K
 * range over up to 8 workgroups, which write fp32 partial tiles that another
 * launch adds in a fixed order: results are deterministic for a given shape
 * and device.
 *   X  device fp16 [ntok][cols], 16-byte aligned (row-major)
 *   Y  device fp16 [ntok][rows] (round to nearest even); both caller-owned
 *   ntok >= 1.  Both packed formats (C = 8 and C = 12) with cols a multiple of
 *   8, fp16 X and Y only; other dtypes return SEEDLM_E_UNSUPPORTED (for up to
 *   16 rows seedlm_gemv covers them), as do X or the packed buffer of 2 GiB or
 *   more and ntok above 16,776,960.
 * Asynchronous on `stream`.  Split tiles keep their partials in the stream's
 * scratch, the gemv scratch (same rules: calls on different streams may
 * overlap, a call that needs more than the stream has allocates -- not inside
 * graph capture -- and seedlm_scratch_release frees it);
 * seedlm_gemm_scratch_bytes gives a call's size (at most 64 MiB on a
 * 256-compute-unit device).  Call with the device h was packed on current.
 * Errors: SEEDLM_E_INVALID (null, ntok < 1, another device current),
 * SEEDLM_E_UNSUPPORTED (format, dtype, alignment), SEEDLM_E_NOMEM (scratch),
 * SEEDLM_E_DEVICE (launch failure).
 */
SEEDLM_API int seedlm_gemm(seedlm_handle h, const void* X, void* Y, int64_t ntok,
                           int x_dtype, int y_dtype, void* stream);

/*
 * seedlm_gemm_scratch_bytes -- the scratch bytes seedlm_gemm(h, ., ., ntok, ...)
 * uses on the current device (0 when it splits no tile).  *bytes is set on
 * success.
 * Errors: SEEDLM_E_INVALID (null, ntok < 1).
 */
SEEDLM_API int seedlm_gemm_scratch_bytes(seedlm_handle h, int64_t ntok, size_t* bytes);

/*
 * seedlm_gemm_decoded -- the same product through a decoded copy of W: the
 * matrix is rebuilt once, exactly, into `workspace` as fp16(w * 2^10) (the
 * values the matrix-core kernels feed their MFMAs), then multiplied by a
 * hipBLASLt matmul (fp16 operands, fp32 accumulation, alpha = 2^-10).  With
 * several hundred activation rows or more (from between 256 and 512 on a
 * 4-bit Llama-3-70B layer) the product is compute-bound and this path is
 * faster than seedlm_gemm; below that seedlm_gemm is.  The weights are
 * still rebuilt from the records (paperhub.cn rebuttal text before Eq. (1));
 * the copy lives only in the caller's workspace, for the duration of the call.
 *   X, Y       as for seedlm_gemm (fp16, cols a multiple of 8, X 16-byte aligned)
 *   workspace  device memory, 16-byte aligned, caller-owned, at least
 *              rows * cols * 2 bytes; on return its first rows * cols * 2
 *              bytes hold the decoded matrix, row-major.  Bytes past the
 *              matrix (from the next multiple of 256, up to 32 MiB) serve as
 *              the GEMM's scratch; seedlm_gemm_decoded_bytes(h) is the size
 *              that includes the full 32 MiB
 * Asynchronous on `stream`.  Uses one hipBLASLt handle per device, created on
 * the first call, and caches one matmul plan per device, shape and scratch
 * size (the first call with a new shape also runs the library's heuristic
 * query); calls from several host threads serialise on a lock while they
 * enqueue.  Calls that share a workspace must not overlap.
 * Call it with the device that h was packed on current.
 * Errors: SEEDLM_E_INVALID (null pointer, ntok < 1, workspace too small,
 * another device current), SEEDLM_E_UNSUPPORTED (dtype, alignment, cols not a
 * multiple of 8, sizes of 2^31 or more), SEEDLM_E_DEVICE (launch failure, or no
 * hipBLASLt algorithm for the shape: then nothing has been enqueued).
 */
SEEDLM_API int seedlm_gemm_decoded(seedlm_handle h, const void* X, void* Y, int64_t ntok,
                                   int x_dtype, int y_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* seedlm_gemm_decoded_bytes -- the workspace size for seedlm_gemm_decoded on h:
 * the decoded matrix rounded up to 256 bytes, plus 32 MiB of GEMM scratch. */
SEEDLM_API int seedlm_gemm_decoded_bytes(seedlm_handle h, size_t* bytes);

/*
 * Seed search (compression).  SeedLM picks, for every block w of C weights, the
 * seed s, coefficients t and shared exponent e that make 2^e U(s) t closest to
 * w, searching all seeds (atlas.scime.ai "Approach"), with the pseudo-inverses
 * of every seed computed once and cached and the search run in parallel over
 * blocks and seeds (paperhub.cn rebuttal on compression cost).  The rule this
 * library applies per seed: t* = pinv(U(s)) w; e = the smallest exponent in
 * [-15, 0] at which every round-half-even(t*_j / 2^e) lies in [-8, 7] (0 if
 * none); t = clamp(round-half-even(t* / 2^e), -8, 7); score ||w - 2^e U t||^2;
 * the lowest score wins, the smaller seed on ties.  Scores are computed in
 * fp32, so near-ties between seeds may resolve differently from an exact
 * computation; the chosen record is always a valid one whose fp32 score is the
 * minimum over all 65535 seeds.
 */
typedef struct seedlm_encoder* seedlm_encoder_handle;

/*
 * seedlm_encoder_create -- build, on the current device, the per-seed table of
 * format (C, P, K, Q) the search reads: the thin QR factors of U(s) for all
 * 2^K - 1 seeds (12 MiB for (8,3,16,4), 23 MiB for (12,4,16,4)).  Q is the
 * coefficient width (t in [-2^(Q-1), 2^(Q-1) - 1]).  Synchronous.  The handle
 * owns the table.
 * Formats: the packed formats (8,3,16,4) and (12,4,16,4), and for studying
 * the design space (records only; seedlm_pack takes the packed formats alone,
 * and the seed width and coefficient width are the pages' knobs below 3 bits:
 * paperhub.cn, answer on 1.5-2.5 bits per weight): with K = 16, Q = 4 the
 * (C, P) pairs (6,1) (7,2) (9,4) (10,5) (11,6) (12,7) (8,1) (9,1) (10,2) (11,3)
 * (8,2) (8,4); with other seed widths (7,3,12,4) (8,2,12,4) (9,3,20,4)
 * (12,3,20,4); with 3-bit coefficients (8,4,16,3) (10,3,16,3).  The K-bit
 * LFSRs: x^12+x^6+x^4+x+1, x^16+x^5+x^3+x^2+1 (the format's), x^20+x^3+1.
 * Errors: SEEDLM_E_INVALID (null out), SEEDLM_E_UNSUPPORTED (format not
 * supported), SEEDLM_E_NOMEM, SEEDLM_E_DEVICE.
 */
SEEDLM_API int seedlm_encoder_create(int C, int P, int K, int Q, seedlm_encoder_handle* out);

/* seedlm_encoder_destroy -- free the encoder's table; NULL is a no-op. */
SEEDLM_API int seedlm_encoder_destroy(seedlm_encoder_handle e);

/*
 * seedlm_encode -- exhaustive seed search for every block of a dense matrix.
 *   W      device bf16 [rows][cols] (raw bf16 bit patterns, row-major); 16-byte
 *          aligned when C = 8 and cols is a multiple of 8, 2-byte aligned
 *          otherwise; finite values.  When cols is not a multiple of C, a row's
 *          last block holds its cols - (nb-1) C weights followed by zeros, and is
 *          searched as a full block (seedlm_decode drops the padding columns)
 *   seeds  device uint16 [rows][nb] (uint32 for K > 16), nb = ceil(cols / C) (out)
 *   coeffs device int8   [rows][nb][P]                 (out)
 *   exps   device int8   [rows][nb]                    (out)
 *   err    device float  [rows][nb], the fp32 score of the chosen record, or
 *          NULL                                        (out)
 * The outputs are the record arrays seedlm_pack takes (after a copy to host).
 * All buffers are caller-owned.  Asynchronous on `stream`; the encoder must have
 * been created on the current device.  Calls sharing an encoder may overlap.
 * Errors: SEEDLM_E_INVALID (null pointer, shape, alignment, other device),
 * SEEDLM_E_UNSUPPORTED (grid too large), SEEDLM_E_DEVICE (launch failure).
 */
SEEDLM_API int seedlm_encode(seedlm_encoder_handle e, const void* W, int64_t rows,
                             int64_t cols, void* seeds, int8_t* coeffs, int8_t* exps,
                             float* err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SEEDLM_H */
