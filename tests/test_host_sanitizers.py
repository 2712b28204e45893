"""Host AddressSanitizer + UndefinedBehaviorSanitizer run of the packer and the
C-ABI's argument checks (CPU only).

Every library source is compiled with the sanitizers on its host side only
(device code is built as usual; no sanitizer runs on the GPU) and linked with
tests/host_abi_check.cpp into one executable.  Its "abi" mode calls each entry
point with null and out-of-range arguments and checks the documented status;
its "pack" mode packs record sets read from a file into exactly sized heap
buffers, whose bytes must equal the oracle's layout writer.  Any heap overflow,
use after free, leak or undefined operation in that host code aborts the run.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Sanitizers for the host compilation only (each flag behind -Xarch_host).
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("hostsan")
    sources = sorted(glob.glob(os.path.join(ROOT, "prng_seeded_decode_amd", "csrc", "*.hip")))
    sources.append(os.path.join(ROOT, "tests", "host_abi_check.cpp"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), *HOST_SAN]

    def compile_one(src):
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, sources))
    exe = str(out / "host_abi_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, *objs, "-lhipblaslt", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe, out


def _run(exe, *args):
    env = dict(os.environ, **SAN_ENV)
    r = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=120)
    return r.returncode, r.stdout + r.stderr


def test_abi_argument_checks_under_sanitizers(checker):
    exe, _ = checker
    rc, log = _run(exe, "abi")
    assert rc == 0, log
    assert "abi checks: 0 failure(s)" in log
    assert "ERROR: AddressSanitizer" not in log and "runtime error" not in log


@pytest.mark.parametrize("C,P,K,rows,cols", [
    (8, 3, 16, 1, 1), (8, 3, 16, 3, 8 * 33 + 5), (8, 3, 16, 2, 8 * 64),
    (12, 4, 16, 1, 7), (12, 4, 16, 5, 12 * 16), (12, 4, 16, 3, 12 * 49 + 11),
    (8, 4, 16, 4, 8 * 40 + 3), (12, 3, 20, 3, 12 * 21 + 1),
])
def test_packer_under_sanitizers_matches_oracle_writer(checker, C, P, K, rows, cols):
    from oracle import seedlm_oracle as O

    exe, out = checker
    Q = O.PACKED_FORMATS[(C, P, K)]
    nb = -(-cols // C)
    rng = np.random.default_rng([C, P, K, rows, cols])
    s = rng.integers(1, 1 << K, (rows, nb)).astype(np.uint16 if K <= 16 else np.uint32)
    c = rng.integers(-(1 << (Q - 1)), 1 << (Q - 1), (rows, nb, P)).astype(np.int8)
    e = rng.integers(-15, 1, (rows, nb)).astype(np.int8)
    src = str(out / f"in_{C}_{P}_{K}_{rows}_{cols}.bin")
    dst = str(out / f"out_{C}_{P}_{K}_{rows}_{cols}.bin")
    with open(src, "wb") as f:
        f.write(np.array([rows, cols], np.int64).tobytes())
        f.write(np.array([C, P, K], np.int32).tobytes())
        f.write(s.tobytes() + c.tobytes() + e.tobytes())
    rc, log = _run(exe, "pack", src, dst)
    assert rc == 0, log
    with open(dst, "rb") as f:
        assert f.read() == O.write_packed(s, c, e, rows, cols, C, P, K=K)
