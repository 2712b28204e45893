"""GPU parity over every coefficient combination of both pages' formats.

Each kernel turns the packed coefficient nibbles into numbers its own way: the
batch-1 table kernels as t/16 (v_cvt_off_f32_i4 and an fp16 pair table), the
matrix-core and prefill decodes as sign-extended integers beside a scale built
from the exponent nibble, the exact kernels by plain extraction.  Here a matrix
holds every (t0, t1, t2) of the 4-bit format (4096 blocks) and every
(t0, t1, t2, t3) of the 3-bit format (65536 blocks), with all sixteen exponents,
and every path is compared with the CPU oracle at the usual bars: decode
bit-exact, fp32 output normwise <= 1e-5, fp16 output normwise <= 2e-3 (per
token row for the prefill product).
"""
import numpy as np
import pytest

from oracle import seedlm_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3}
VARIANTS = {"auto": 0, "lut": 1, "simple": 3, "mfma": 4, "direct": 5}


def _S():
    import prng_seeded_decode_amd as S

    return S


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _all_combinations(C, P, nb):
    """Records whose blocks run through all 16^P coefficient tuples (block
    index n: t_j = nibble j of n, minus 8) and all 16 exponents."""
    n = 16 ** P
    rows = n // nb
    idx = np.arange(n).reshape(rows, nb)
    coeffs = np.stack([((idx >> (4 * j)) & 15) - 8 for j in range(P)], axis=-1).astype(np.int8)
    exps = (-((idx * 7 + idx // nb) % 16)).astype(np.int8)
    seeds = np.random.default_rng(16 ** P + C).integers(1, 65536, (rows, nb)).astype(np.uint16)
    return seeds, coeffs, exps, rows, nb * C


@pytest.mark.parametrize("C,P,nb", [(8, 3, 64), (12, 4, 256)], ids=["4bit", "3bit"])
def test_every_coefficient_tuple_through_every_path(C, P, nb):
    S = _S()
    dev = _dev()
    s, c, e, rows, cols = _all_combinations(C, P, nb)
    assert sorted(set(e.reshape(-1).tolist())) == list(range(-15, 1))
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, 16)
    W_ref = O.decode_rows(s, c, e, cols, C, P)
    print(f"decode C={C} {rows}x{cols}", flush=True)
    W = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    S.seedlm_decode(m, W)
    torch.cuda.synchronize()
    assert np.array_equal(W.cpu().numpy(), W_ref.astype(np.float32))

    rng = np.random.default_rng(C * 1000 + P)
    ran = set()
    for name, variant in VARIANTS.items():
        for batch, dt in ((1, "f32"), (1, "f16"), (4, "f16")):
            if name == "mfma" and (batch == 1 or dt == "f32"):
                continue  # the matrix-core path takes fp16 at batch > 1 only
            if name == "lut" and batch > 1:
                continue  # the table kernels are the batch-1 path
            npdt = np.float16 if dt == "f16" else np.float32
            tdt = torch.float16 if dt == "f16" else torch.float32
            x = rng.standard_normal((batch, cols)).astype(npdt)
            y = torch.empty((batch, rows), dtype=tdt, device=dev)
            print(f"gemv C={C} {name} batch={batch} {dt}", flush=True)
            try:
                S.seedlm_gemv(m, torch.from_numpy(x).to(dev), y, batch=batch, variant=variant)
            except S.SeedLMError as exc:
                if exc.status == S.E_UNSUPPORTED:
                    continue  # this kernel does not take these dtypes
                raise
            torch.cuda.synchronize()
            err = O.normwise_error(y.float().cpu().numpy().astype(np.float64), O.gemv(W_ref, x))
            assert err <= TOL[dt], (name, batch, dt, err)
            ran.add((name, batch, dt))
    # the default path, both batch-1 table kernels' dtypes and the matrix-core path ran
    assert {("auto", 1, "f32"), ("auto", 1, "f16"), ("auto", 4, "f16"), ("lut", 1, "f32"),
            ("lut", 1, "f16"), ("mfma", 4, "f16")} <= ran, ran

    # The prefill product (fp16 X and Y), every token row against the oracle.
    ntok = 37
    X = rng.standard_normal((ntok, cols)).astype(np.float16)
    Y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    print(f"gemm C={C} {ntok} tokens", flush=True)
    S.seedlm_gemm(m, torch.from_numpy(X).to(dev), Y)
    torch.cuda.synchronize()
    Y_ref = O.gemv(W_ref, X)
    Yg = Y.float().cpu().numpy().astype(np.float64)
    for t in range(ntok):
        assert O.normwise_error(Yg[t], Y_ref[t]) <= TOL["f16"], t
    m.destroy()
