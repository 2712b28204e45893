"""seedlm_gemv_many_noalloc: the allocation-free variant of seedlm_gemv_many.

It runs the same kernels with the partials in the library's fixed device
scratch, so its outputs must equal seedlm_gemv_many's bit for bit, and both must
meet the oracle's bar (normwise 2e-3 for fp16 output, 1e-5 for fp32).  Two calls
in a row, the second with a smaller input, check that nothing of the first
call's scratch contents leaks into the second.
"""
import math

import numpy as np
import pytest

from oracle import seedlm_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3}


def _S():
    import prng_seeded_decode_amd as S

    return S


def _records(rng, rows, cols, C, P):
    nb = math.ceil(cols / C)
    s = rng.integers(1, 65536, (rows, nb)).astype(np.uint16)
    c = rng.integers(-8, 8, (rows, nb, P)).astype(np.int8)
    e = rng.integers(-12, -5, (rows, nb)).astype(np.int8)
    return s, c, e


def _problem(rng, shapes, batch, xdt):
    S = _S()
    dev = torch.device("cuda:0")
    mats, refs, xs = [], [], []
    for C, P, rows, cols in shapes:
        s, c, e = _records(rng, rows, cols, C, P)
        mats.append(S.seedlm_pack(s, c, e, rows, cols, C, P, 16))
        refs.append(O.decode_rows(s, c, e, cols, C, P))
        xs.append(rng.standard_normal((batch, cols)).astype(np.float16 if xdt == "f16"
                                                            else np.float32))
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    return mats, refs, xs, xd


@pytest.mark.parametrize("batch,ydt", [(1, "f16"), (1, "f32"), (4, "f16")])
def test_noalloc_matches_gemv_many_on_two_calls(batch, ydt):
    S = _S()
    dev = torch.device("cuda:0")
    tdt = torch.float16 if ydt == "f16" else torch.float32
    rng = np.random.default_rng(500 + batch)
    big = [(8, 3, 1024, 8 * 300 + 3), (8, 3, 300, 4096), (12, 4, 257, 12 * 90 + 7),
           (8, 3, 2048, 2048), (8, 3, 64, 1000)]
    small = [(8, 3, 40, 8 * 20 + 5), (12, 4, 30, 400)]
    stream = torch.cuda.Stream()
    for k, shapes in enumerate((big, small)):
        mats, refs, xs, xd = _problem(rng, shapes, batch, "f16")
        ys = [torch.full((batch, m.rows), float("nan"), dtype=tdt, device=dev) for m in mats]
        want = [torch.empty_like(y) for y in ys]
        print(f"noalloc call {k}: {len(mats)} matrices, batch {batch}, y {ydt}", flush=True)
        with torch.cuda.stream(stream):
            S.seedlm_gemv_many_noalloc(mats, xd, ys, batch=batch, stream=stream)
            S.seedlm_gemv_many(mats, xd, want, batch=batch, stream=stream)
        stream.synchronize()
        for y, w, W_ref, x in zip(ys, want, refs, xs):
            assert torch.equal(y, w)
            assert O.normwise_error(y.double().cpu().numpy(), O.gemv(W_ref, x)) <= TOL[ydt]


def test_noalloc_makes_no_allocation_and_rejects_oversized_calls():
    S = _S()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(9)
    rows, cols = 8192, 8192
    s, c, e = _records(rng, rows, cols, 8, 3)
    m = S.seedlm_pack(s, c, e, rows, cols, 8, 3, 16)
    x = torch.from_numpy(rng.standard_normal((16, cols)).astype(np.float16)).to(dev)
    y = torch.empty((16, rows), dtype=torch.float16, device=dev)
    # batch 16 on five copies of the handle needs more than the static scratch
    need = S.seedlm_gemv_scratch_bytes([m] * 5, batch=16)
    assert need > S.NOALLOC_SCRATCH_BYTES
    with pytest.raises(S.SeedLMError) as err:
        S.seedlm_gemv_many_noalloc([m] * 5, [x] * 5, [y] * 5, batch=16)
    assert err.value.status == S.E_SCRATCH_LIMIT
    # On a fresh stream seedlm_gemv_many allocates its scratch (1 MiB per copy
    # of the handle at batch 1: 32 panels x 8192 rows) and the no-alloc call
    # must not.  Each stream first runs a torch kernel, so that whatever the
    # runtime sets up for a new stream is in place before free memory is read.
    need = S.seedlm_gemv_scratch_bytes([m] * 8, batch=1)
    assert need == 8 << 20
    x1 = x[:1].contiguous()
    ys = [torch.empty((1, rows), dtype=torch.float16, device=dev) for _ in range(8)]

    def used_by(fn):
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            ys[0].zero_()
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info(dev)
        fn(st)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info(dev)
        return free0 - free1

    grew = used_by(lambda st: S.seedlm_gemv_many([m] * 8, [x1] * 8, ys, stream=st))
    assert grew >= need  # the measurement sees a scratch allocation
    none = used_by(lambda st: S.seedlm_gemv_many_noalloc([m] * 8, [x1] * 8, ys, stream=st))
    print(f"device memory taken: seedlm_gemv_many {grew} B, noalloc {none} B", flush=True)
    assert none < need
    pick = np.arange(0, rows, 97)
    W_ref = O.decode_rows(s[pick], c[pick], e[pick], cols, 8, 3)
    for yk in ys:
        got = yk.double().cpu().numpy()[:, pick]
        assert O.normwise_error(got, O.gemv(W_ref, x1.cpu().numpy())) <= TOL["f16"]
