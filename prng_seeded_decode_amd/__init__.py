"""SeedLM decompress-and-multiply on MI355X (gfx950).

A small C-ABI library (libseedlm.so: hand-written HIP kernels) plus this
ctypes binding.  Weights are stored per block as a 16-bit LFSR seed, 4-bit
coefficients and a shared exponent, and rebuilt inside the kernels while
multiplying (SeedLM: paperdance.org abstract; atlas.scime.ai "Approach").
"""
from ._binding import (  # noqa: F401
    E_DEVICE,
    E_INVALID,
    E_NOMEM,
    E_SCRATCH_LIMIT,
    NOALLOC_SCRATCH_BYTES,
    E_UNSUPPORTED,
    F16,
    F32,
    MAX_BATCH,
    OK,
    STREAM_READ_SINK,
    VARIANT_AUTO,
    VARIANT_DIRECT,
    VARIANT_MFMA,
    VARIANT_LUT,
    VARIANT_SIMPLE,
    VARIANT_TABLE,
    GemvManyCall,
    SeedLMEncoder,
    SeedLMError,
    SeedLMMatrix,
    lib,
    pack_host_status,
    seedlm_bench_time_next_call,
    seedlm_decode,
    seedlm_encode,
    seedlm_export,
    seedlm_fp16_gemv,
    seedlm_gemm,
    seedlm_gemm_decoded,
    seedlm_gemm_decoded_bytes,
    seedlm_gemv,
    seedlm_gemv_many,
    seedlm_gemv_many_noalloc,
    seedlm_gemv_scratch_bytes,
    seedlm_pack,
    seedlm_pack_host,
    seedlm_scratch_release,
    seedlm_stream_read,
    status_string,
)
