"""CPU-only tests of the C-ABI library: it loads, exports every symbol the
header declares, and its host packer writes exactly the layout the oracle's
own writer produces (and rejects bad records with the documented status)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import prng_seeded_decode_amd as S

    return S


def test_library_exports_every_declared_symbol():
    S = _lib()
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            header = open(os.path.join(ROOT, "include", h)).read()
            names += re.findall(r"SEEDLM_API\s+[\w\s\*]+?\b(seedlm_\w+)\s*\(", header)
    assert len(names) >= 10 and len(names) == len(set(names))
    L = S.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(S._binding.EXPORTED)


def test_status_strings():
    S = _lib()
    for code in (S.OK, S.E_INVALID, S.E_UNSUPPORTED, S.E_NOMEM, S.E_DEVICE, S.E_SCRATCH_LIMIT):
        assert S.status_string(code) not in ("", "unknown status")
    assert S.status_string(12345) == "unknown status"


@pytest.mark.parametrize("C,P,K,rows,cols", [
    (8, 3, 16, 1, 1), (8, 3, 16, 5, 320), (8, 3, 16, 9, 8 * 77 + 3), (12, 4, 16, 6, 401),
    (12, 4, 16, 4, 12 * 64), (12, 4, 16, 3, 12 * 37 + 5), (8, 4, 16, 7, 8 * 45 + 1),
    (12, 3, 20, 5, 12 * 35 + 7),
])
def test_host_packer_matches_oracle_writer_and_reader(C, P, K, rows, cols):
    S = _lib()
    from oracle import seedlm_oracle as O

    rng = np.random.default_rng(rows * 1000 + cols)
    nb = -(-cols // C)
    Q = O.PACKED_FORMATS[(C, P, K)]
    s = rng.integers(1, 1 << K, (rows, nb)).astype(np.uint16 if K <= 16 else np.uint32)
    c = rng.integers(-(1 << (Q - 1)), 1 << (Q - 1), (rows, nb, P)).astype(np.int8)
    e = rng.integers(-15, 1, (rows, nb)).astype(np.int8)
    buf = S.seedlm_pack_host(s, c, e, rows, cols, C, P, K)
    assert buf == O.write_packed(s, c, e, rows, cols, C, P, K=K)
    s2, c2, e2 = O.read_packed(buf, rows, cols, C, P, K=K)
    assert (s2 == s).all() and (c2 == c).all() and (e2 == e).all()


def test_host_packer_rejects_bad_records():
    S = _lib()
    rows, cols = 3, 20
    s = np.ones((rows, 3), np.uint16)
    c = np.zeros((rows, 3, 3), np.int8)
    e = np.zeros((rows, 3), np.int8)
    assert S.pack_host_status(s, c, e, rows, cols, 8, 3) == S.OK
    bad = s.copy(); bad[1, 2] = 0
    assert S.pack_host_status(bad, c, e, rows, cols, 8, 3) == S.E_INVALID
    bad = c.copy(); bad[0, 0, 1] = 8
    assert S.pack_host_status(s, bad, e, rows, cols, 8, 3) == S.E_INVALID
    bad = c.copy(); bad[0, 0, 1] = -9
    assert S.pack_host_status(s, bad, e, rows, cols, 8, 3) == S.E_INVALID
    bad = e.copy(); bad[2, 0] = 1
    assert S.pack_host_status(s, c, bad, rows, cols, 8, 3) == S.E_INVALID
    bad = e.copy(); bad[2, 0] = -16
    assert S.pack_host_status(s, c, bad, rows, cols, 8, 3) == S.E_INVALID
    assert S.pack_host_status(s, c, e, 0, cols, 8, 3) == S.E_INVALID
    assert S.pack_host_status(s, c, e, rows, 0, 8, 3) == S.E_INVALID
    assert S.pack_host_status(s, c, e, rows, cols, 8, 3, K=12) == S.E_UNSUPPORTED
    assert S.pack_host_status(s, c, e, rows, cols, 16, 3) == S.E_UNSUPPORTED
    assert S.pack_host_status(s, c, e, rows, cols, 12, 3, K=16) == S.E_UNSUPPORTED
    # (8, 4, 16) takes 3-bit coefficients: [-4, 3]
    c4 = np.zeros((rows, 3, 4), np.int8)
    c4[1, 1] = (3, -4, 0, 1)
    assert S.pack_host_status(s, c4, e, rows, cols, 8, 4) == S.OK
    bad = c4.copy(); bad[2, 2, 3] = 4
    assert S.pack_host_status(s, bad, e, rows, cols, 8, 4) == S.E_INVALID
    bad = c4.copy(); bad[0, 0, 0] = -5
    assert S.pack_host_status(s, bad, e, rows, cols, 8, 4) == S.E_INVALID
    # (12, 3, 20) takes 20-bit seeds: [1, 2^20 - 1]
    s20 = np.full((rows, 2), (1 << 20) - 1, np.uint32)
    c3, e2 = np.zeros((rows, 2, 3), np.int8), np.zeros((rows, 2), np.int8)
    assert S.pack_host_status(s20, c3, e2, rows, cols, 12, 3, K=20) == S.OK
    bad = s20.copy(); bad[1, 1] = 1 << 20
    assert S.pack_host_status(bad, c3, e2, rows, cols, 12, 3, K=20) == S.E_INVALID
    # null pointers and a too-small destination
    L = S.lib()
    n = ctypes.c_size_t(0)
    assert L.seedlm_pack_host(None, None, None, rows, cols, 8, 3, 16, None, ctypes.byref(n)) == S.E_INVALID
    sp = s.ctypes.data_as(ctypes.c_void_p)
    cp = c.ctypes.data_as(ctypes.c_void_p)
    ep = e.ctypes.data_as(ctypes.c_void_p)
    assert L.seedlm_pack_host(sp, cp, ep, rows, cols, 8, 3, 16, None, None) == S.E_INVALID
    assert L.seedlm_pack_host(sp, cp, ep, rows, cols, 8, 3, 16, None, ctypes.byref(n)) == S.OK
    assert n.value == 4 * 4 * 8  # 3 rows padded to 8, 3 blocks padded to 4 slots
    small = ctypes.create_string_buffer(8)
    n2 = ctypes.c_size_t(8)
    assert L.seedlm_pack_host(sp, cp, ep, rows, cols, 8, 3, 16, ctypes.cast(small, ctypes.c_void_p),
                              ctypes.byref(n2)) == S.E_INVALID


def test_device_entry_points_reject_null_handles_without_touching_the_gpu():
    S = _lib()
    L = S.lib()
    x = ctypes.c_void_p(16)
    assert L.seedlm_gemv(None, x, x, 1, S.F16, S.F16, None) == S.E_INVALID
    assert L.seedlm_decode(None, x, None) == S.E_INVALID
    assert L.seedlm_destroy(None) == S.OK
    assert L.seedlm_info(None, None) == S.E_INVALID
    assert L.seedlm_fp16_gemv(None, x, x, 4, 8, 1, None) == S.E_INVALID
    assert L.seedlm_fp16_gemv(x, x, x, 4, 12, 1, None) == S.E_INVALID
    assert L.seedlm_gemm(None, x, x, 4, S.F16, S.F16, None) == S.E_INVALID
    assert L.seedlm_stream_read(None, 16, x, None) == S.E_INVALID
    assert L.seedlm_stream_read(x, 16, None, None) == S.E_INVALID
    assert L.seedlm_stream_read(x, 0, x, None) == S.E_INVALID
    assert L.seedlm_stream_read(x, 24, x, None) == S.E_INVALID
    assert L.seedlm_stream_read(ctypes.c_void_p(8), 16, x, None) == S.E_INVALID
    h = ctypes.c_void_p()
    assert L.seedlm_encoder_create(8, 5, 16, 4, ctypes.byref(h)) == S.E_UNSUPPORTED
    assert L.seedlm_encoder_create(12, 3, 16, 4, ctypes.byref(h)) == S.E_UNSUPPORTED
    assert L.seedlm_encoder_create(8, 3, 12, 4, ctypes.byref(h)) == S.E_UNSUPPORTED
    assert L.seedlm_encoder_create(8, 3, 16, 5, ctypes.byref(h)) == S.E_UNSUPPORTED
    assert L.seedlm_encoder_create(13, 4, 16, 4, ctypes.byref(h)) == S.E_UNSUPPORTED
    assert L.seedlm_encoder_create(8, 3, 16, 4, None) == S.E_INVALID
    assert L.seedlm_encoder_destroy(None) == S.OK
    assert L.seedlm_encode(None, x, 4, 64, x, x, x, x, None) == S.E_INVALID
