"""GPU parity of the batch-1 3-bit table-lookup kernel (C=12, P=4) against the
CPU oracle, through the C ABI.

The kernel works on column units of 16 blocks (one packed 3-bit panel) and on
16-row slabs, so the edge cases here are: a last slab holding only 8 rows
(Mp = 8 mod 16), last panels of every stored width class (1, 4, 15, 16 blocks
and the steps between), a single block, the extreme exponents and
coefficients, and several matrices in one grouped launch.  Bars as in the other GPU parity tests
(normwise error against the float64 oracle): 2e-3 for fp16 output, 1e-5 for
fp32 output; repeated calls must agree bit for bit.
"""
import math

import numpy as np
import pytest

from oracle import seedlm_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3}
LUT = 1  # SEEDLM_VARIANT_LUT


def _S():
    import prng_seeded_decode_amd as S

    return S


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _records(rng, rows, cols, erange=(-15, 0), crange=(-8, 7)):
    nb = math.ceil(cols / 12)
    s = rng.integers(1, 65536, (rows, nb)).astype(np.uint16)
    c = rng.integers(crange[0], crange[1] + 1, (rows, nb, 4)).astype(np.int8)
    e = rng.integers(erange[0], erange[1] + 1, (rows, nb)).astype(np.int8)
    return s, c, e


def _gemv(m, x_np, ydt, variant=LUT):
    dev = _dev()
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dev)
    y = torch.empty((1, m.rows), dtype=torch.float16 if ydt == "f16" else torch.float32,
                    device=dev)
    _S().seedlm_gemv(m, x, y, batch=1, variant=variant)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


# (rows, nb): rows 40 and 24 leave an 8-row last slab; nb mod 16 = 1, 4, 15, 0,
# 1, 4, 15 and 0 give last panels of 1 block (stored 4 wide), 4, 15 (stored 16)
# and a full 16.
SHAPES = [(40, 33), (24, 36), (16, 47), (8, 48), (56, 49), (72, 52), (33, 63), (48, 64),
          (1, 1), (129, 342), (200, 96)]


@pytest.mark.parametrize("rows,nb", SHAPES, ids=[f"{r}x{n}blk" for r, n in SHAPES])
@pytest.mark.parametrize("xdt,ydt", [("f16", "f16"), ("f32", "f32")])
def test_lut12_matches_oracle(rows, nb, xdt, ydt):
    rng = np.random.default_rng(rows * 1009 + nb)
    cols = 12 * nb - (nb % 5)  # ragged tail on most shapes
    cols = max(cols, 1)
    s, c, e = _records(rng, rows, cols)
    m = _S().seedlm_pack(s, c, e, rows, cols, 12, 4, 16)
    W = O.decode_rows(s, c, e, cols, 12, 4)
    x = rng.standard_normal((1, cols)).astype(np.float16 if xdt == "f16" else np.float32)
    _say(f"lut12 {rows}x{cols} {xdt}->{ydt}")
    y = _gemv(m, x, ydt)
    assert O.normwise_error(y, O.gemv(W, x)) <= TOL[ydt]


def test_lut12_extreme_records():
    """Exponents at both ends, coefficients at -8 and 7, and seeds 1 and 65535."""
    rng = np.random.default_rng(12)
    rows, cols = 48, 12 * 70
    s, c, e = _records(rng, rows, cols)
    e[: rows // 2] = -15
    e[rows // 2:] = 0
    c[::2, ::3] = -8
    c[1::2, ::3] = 7
    s[:, 0] = 1
    s[:, -1] = 65535
    m = _S().seedlm_pack(s, c, e, rows, cols, 12, 4, 16)
    W = O.decode_rows(s, c, e, cols, 12, 4)
    x = rng.standard_normal((1, cols)).astype(np.float32)
    y = _gemv(m, x, "f32")
    # rows with e = -15 are 2^15 times smaller than the others: check each half
    # against its own scale
    y_ref = O.gemv(W, x)
    for sl in (slice(0, rows // 2), slice(rows // 2, rows)):
        assert O.normwise_error(y[:, sl], y_ref[:, sl]) <= TOL["f32"]


def test_lut12_grouped_launch_matches_single_calls_and_repeats():
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(77)
    shapes = [(40, 12 * 33), (1024, 4096), (16, 12 * 17 - 3), (300, 1000)]
    mats, refs, xs = [], [], []
    for rows, cols in shapes:
        s, c, e = _records(rng, rows, cols, erange=(-12, -6))
        mats.append(S.seedlm_pack(s, c, e, rows, cols, 12, 4, 16))
        refs.append(O.decode_rows(s, c, e, cols, 12, 4))
        xs.append(rng.standard_normal((1, cols)).astype(np.float16))
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    ys = [torch.empty((1, m.rows), dtype=torch.float16, device=dev) for m in mats]
    _say(f"lut12 gemv_many {len(mats)} matrices")
    S.seedlm_gemv_many(mats, xd, ys)
    torch.cuda.synchronize()
    for y, W, x in zip(ys, refs, xs):
        assert O.normwise_error(y.float().cpu().numpy(), O.gemv(W, x)) <= TOL["f16"]
    ys2 = [torch.empty_like(y) for y in ys]
    for m, x, y in zip(mats, xd, ys2):
        S.seedlm_gemv(m, x, y)
    ys3 = [torch.empty_like(y) for y in ys]
    S.seedlm_gemv_many(mats, xd, ys3)
    torch.cuda.synchronize()
    for a, b, c3 in zip(ys, ys2, ys3):
        assert torch.equal(a, b) and torch.equal(a, c3)


def test_lut12_agrees_with_exact_kernel():
    """Against the per-lane exact kernel (SIMPLE) at fp32 output, on a shape with
    several units and slabs."""
    rng = np.random.default_rng(5)
    rows, cols = 136, 12 * 100 + 7
    s, c, e = _records(rng, rows, cols, erange=(-12, -6))
    m = _S().seedlm_pack(s, c, e, rows, cols, 12, 4, 16)
    x = rng.standard_normal((1, cols)).astype(np.float16)
    y_lut = _gemv(m, x, "f32", variant=LUT)
    y_simple = _gemv(m, x, "f32", variant=3)
    assert O.normwise_error(y_lut, y_simple) <= TOL["f32"]
