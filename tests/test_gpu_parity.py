"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (written here, applied below):
  * seedlm_decode: bit-exact fp32 (the integer block sum times a power of two
    is exact in fp32).
  * seedlm_gemv, normwise error max|y - y_ref| / max|y_ref| against the
    float64 oracle: <= 1e-5 for fp32 output, <= 2e-3 for fp16 output.
Small cases run the oracle on every output; the full configuration shapes are
checked on sampled rows, which the oracle computes one by one.
"""
import math

import numpy as np
import pytest

from oracle import seedlm_oracle as O
from workloads import CONFIGS, gen_records, gen_x

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-3}


def _S():
    import prng_seeded_decode_amd as S

    return S


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _pack(seeds, coeffs, exps, rows, cols, C, P):
    return _S().seedlm_pack(seeds, coeffs, exps, rows, cols, C, P, 16)


def _decode_gpu(m, rows, cols):
    W = torch.empty((rows, cols), dtype=torch.float32, device=_dev())
    _S().seedlm_decode(m, W)
    torch.cuda.synchronize()
    return W


def _gemv_gpu(m, x_np, ydt, variant=0):
    dev = _dev()
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dev)
    y = torch.empty((x.shape[0], m.rows), dtype=torch.float16 if ydt == "f16" else torch.float32,
                    device=dev)
    _S().seedlm_gemv(m, x, y, batch=x.shape[0], variant=variant)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _random_records(rng, rows, cols, C, P, erange=(-15, 0)):
    nb = math.ceil(cols / C)
    s = rng.integers(1, 65536, (rows, nb)).astype(np.uint16)
    c = rng.integers(-8, 8, (rows, nb, P)).astype(np.int8)
    e = rng.integers(erange[0], erange[1] + 1, (rows, nb)).astype(np.int8)
    return s, c, e


SMALL = [
    # (C, P, rows, cols, batch, xdt, ydt)
    (8, 3, 512, 512, 1, "f32", "f32"),
    (8, 3, 37, 8 * 45 + 5, 1, "f16", "f16"),
    (8, 3, 300, 8 * 70, 1, "f16", "f32"),
    (8, 3, 64, 1000, 1, "f32", "f16"),
    (12, 4, 30, 12 * 70 + 7, 1, "f16", "f16"),
    (12, 4, 129, 4096, 1, "f16", "f32"),
    (8, 3, 40, 520, 4, "f16", "f16"),
    (8, 3, 33, 8 * 33, 8, "f16", "f16"),
    (12, 4, 70, 12 * 40 + 4, 16, "f16", "f16"),
    (12, 4, 20, 300, 3, "f32", "f32"),
    (8, 3, 1, 1, 1, "f32", "f32"),
    (12, 4, 1, 5, 2, "f16", "f16"),
]


@pytest.mark.parametrize("C,P,rows,cols,batch,xdt,ydt", SMALL,
                         ids=[f"C{c[0]}_{c[2]}x{c[3]}_b{c[4]}_{c[5]}{c[6]}" for c in SMALL])
def test_small_full_parity(C, P, rows, cols, batch, xdt, ydt):
    rng = np.random.default_rng(rows * 7919 + cols * 31 + batch)
    s, c, e = _random_records(rng, rows, cols, C, P)
    m = _pack(s, c, e, rows, cols, C, P)
    W_ref = O.decode_rows(s, c, e, cols, C, P)
    _say(f"decode C={C} {rows}x{cols}")
    W = _decode_gpu(m, rows, cols).cpu().numpy()
    assert np.array_equal(W, W_ref.astype(np.float32)), "decode must be bit-exact"
    x = rng.standard_normal((batch, cols)).astype(np.float16 if xdt == "f16" else np.float32)
    y_ref = O.gemv(W_ref, x)
    _say(f"gemv C={C} {rows}x{cols} batch={batch} {xdt}->{ydt}")
    y = _gemv_gpu(m, x, ydt)
    assert O.normwise_error(y, y_ref) <= TOL[ydt]


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5],
                         ids=["auto", "lut", "table", "simple", "mfma", "direct"])
@pytest.mark.parametrize("C,P,rows,cols", [(8, 3, 203, 8 * 97 + 3), (12, 4, 96, 12 * 77 + 8)])
def test_variants_agree_with_oracle(variant, C, P, rows, cols):
    S = _S()
    rng = np.random.default_rng(variant + 100 * rows)
    s, c, e = _random_records(rng, rows, cols, C, P)
    m = _pack(s, c, e, rows, cols, C, P)
    W_ref = O.decode_rows(s, c, e, cols, C, P)
    ran = 0
    for xdt, ydt in (("f16", "f16"), ("f32", "f32"), ("f16", "f32")):
        x = rng.standard_normal((1, cols)).astype(np.float16 if xdt == "f16" else np.float32)
        _say(f"variant {variant} C={C} {rows}x{cols} {xdt}->{ydt}")
        try:
            y = _gemv_gpu(m, x, ydt, variant=variant)
        except S.SeedLMError as err:
            if err.status == S.E_UNSUPPORTED:
                continue  # this variant does not take these dtypes / this format
            raise
        assert O.normwise_error(y, O.gemv(W_ref, x)) <= TOL[ydt]
        ran += 1
    if not ran:
        pytest.skip(f"variant {variant} not available for C={C}")


MFMA_CASES = [
    # (C, P, rows, cols, batch, erange): one panel (single chunk, direct store),
    # many panels (chunk partials + reduction), ragged rows and tails, every
    # batch width class, extreme exponents.
    (8, 3, 64, 256, 16, (-12, -6)),
    (8, 3, 300, 8 * 97 + 3, 8, (-15, 0)),
    (8, 3, 517, 4096, 2, (-12, -6)),
    (8, 3, 8, 8 * 33 + 1, 5, (-15, 0)),
    (8, 3, 1000, 1000, 1, (-12, -6)),
    (12, 4, 96, 12 * 77 + 8, 4, (-12, -6)),
    (12, 4, 250, 4096, 16, (-15, 0)),
    (12, 4, 9, 12 * 32, 3, (-12, -6)),
    (12, 4, 333, 14336 // 4, 1, (-12, -6)),
]


@pytest.mark.parametrize("C,P,rows,cols,batch,erange", MFMA_CASES,
                         ids=[f"C{c[0]}_{c[2]}x{c[3]}_b{c[4]}" for c in MFMA_CASES])
def test_mfma_path_against_oracle(C, P, rows, cols, batch, erange):
    rng = np.random.default_rng(rows * 131 + cols + 7 * batch)
    s, c, e = _random_records(rng, rows, cols, C, P, erange)
    m = _pack(s, c, e, rows, cols, C, P)
    W_ref = O.decode_rows(s, c, e, cols, C, P)
    x = rng.standard_normal((batch, cols)).astype(np.float16)
    _say(f"mfma C={C} {rows}x{cols} batch={batch}")
    y = _gemv_gpu(m, x, "f16", variant=4)
    assert O.normwise_error(y, O.gemv(W_ref, x)) <= TOL["f16"]
    # deterministic: the same bits again
    assert np.array_equal(y, _gemv_gpu(m, x, "f16", variant=4))


def test_mfma_path_rejects_fp32():
    S = _S()
    rng = np.random.default_rng(3)
    s, c, e = _random_records(rng, 16, 64, 8, 3)
    m = _pack(s, c, e, 16, 64, 8, 3)
    x = rng.standard_normal((2, 64)).astype(np.float16)
    with pytest.raises(S.SeedLMError) as err:
        _gemv_gpu(m, x, "f32", variant=4)
    assert err.value.status == S.E_UNSUPPORTED


def test_edge_records_extremes():
    # All coefficients at the ends of the 4-bit range, exponents at both ends,
    # seeds 1 and 65535, zero activations, and a single-column matrix.
    rows, cols, C, P = 16, 8 * 40, 8, 3
    nb = cols // C
    s = np.where(np.arange(rows * nb).reshape(rows, nb) % 2 == 0, 1, 65535).astype(np.uint16)
    c = np.full((rows, nb, P), -8, np.int8)
    c[::2] = 7
    e = np.zeros((rows, nb), np.int8)
    e[:, ::3] = -15
    m = _pack(s, c, e, rows, cols, C, P)
    W_ref = O.decode_rows(s, c, e, cols, C, P)
    W = _decode_gpu(m, rows, cols).cpu().numpy()
    assert np.array_equal(W, W_ref.astype(np.float32))
    x0 = np.zeros((1, cols), np.float32)
    assert np.all(_gemv_gpu(m, x0, "f32") == 0)
    x = np.random.default_rng(1).standard_normal((1, cols)).astype(np.float32)
    assert O.normwise_error(_gemv_gpu(m, x, "f32"), O.gemv(W_ref, x)) <= TOL["f32"]


def test_repeated_runs_are_bit_identical():
    rng = np.random.default_rng(99)
    rows, cols, C, P = 1024, 4096, 8, 3
    s, c, e = _random_records(rng, rows, cols, C, P, (-12, -6))
    m = _pack(s, c, e, rows, cols, C, P)
    x = rng.standard_normal((1, cols)).astype(np.float16)
    ys = [_gemv_gpu(m, x, "f16") for _ in range(3)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def _sample_rows(rows, rng, n=16):
    picks = set(range(min(4, rows))) | set(range(max(0, rows - 4), rows))
    picks |= set(int(v) for v in rng.choice(rows, size=min(n, rows), replace=False))
    return np.array(sorted(picks))


FULL = []
for cid in (0, 1, 2, 3, 4):
    cfg = CONFIGS[cid]
    for mid, mat in enumerate(cfg.matrices):
        FULL.append((cid, mid))


def _dot_scale_error(y, W_ref, x):
    """Element-wise error against the dot-product scale: max over outputs of
    |y - y_ref| / sum_c |W[r][c] x[c]| (well-posed where y_ref is near 0)."""
    scale = np.abs(x.astype(np.float64)) @ np.abs(W_ref).T  # [batch][rows]
    return float(np.max(np.abs(y - O.gemv(W_ref, x)) / np.maximum(scale, 1e-300)))


@pytest.mark.parametrize("cid,mid", FULL,
                         ids=[f"c{c}_{CONFIGS[c].matrices[m].name}" for c, m in FULL])
def test_full_size_sampled_parity(cid, mid):
    cfg = CONFIGS[cid]
    mat = cfg.matrices[mid]
    rows, cols, C, P = mat.rows, mat.cols, cfg.C, cfg.P
    s, c, e = gen_records(cid, mid, rows, cols, C, P)
    m = _pack(s, c, e, rows, cols, C, P)
    rng = np.random.default_rng([cid, mid, 777])
    # the 512x512 case is small enough to check every row
    pick = np.arange(rows) if rows * cols <= 1 << 20 else _sample_rows(rows, rng)
    W_ref = O.decode_rows(s[pick], c[pick], e[pick], cols, C, P)
    _say(f"full decode c{cid} {mat.name} {rows}x{cols}")
    W = _decode_gpu(m, rows, cols)
    Wp = W[torch.from_numpy(pick).to(W.device)].cpu().numpy()
    del W
    assert np.array_equal(Wp, W_ref.astype(np.float32)), "decode must be bit-exact"
    ydt = cfg.x_dtype
    for batch in cfg.batches:
        x = gen_x(cid, mid, batch, cols, cfg.x_dtype)
        _say(f"full gemv c{cid} {mat.name} {rows}x{cols} batch={batch}")
        y = _gemv_gpu(m, x, ydt)
        y_ref = O.gemv(W_ref, x)
        err = O.normwise_error(y[:, pick], y_ref)
        dot_err = _dot_scale_error(y[:, pick], W_ref, x)
        _say(f"  normwise {err:.3e}, element-wise against sum|W x| {dot_err:.3e}")
        assert err <= TOL[ydt], (cid, mat.name, batch)
        assert dot_err <= TOL[ydt], (cid, mat.name, batch)


def test_fp16_gemv_baseline_against_torch_fp32():
    dev = _dev()
    S = _S()
    g = torch.Generator(device="cpu").manual_seed(5)
    for rows, cols, batch in ((4096, 4096, 1), (1024, 8192, 8), (300, 520, 3)):
        W = torch.randn(rows, cols, generator=g).half()
        x = torch.randn(batch, cols, generator=g).half()
        ref = (x.float() @ W.float().T).numpy()
        Wd, xd = W.to(dev), x.to(dev)
        y = torch.empty(batch, rows, dtype=torch.float16, device=dev)
        _say(f"fp16 gemv {rows}x{cols} b{batch}")
        S.seedlm_fp16_gemv(Wd, xd, y, batch=batch)
        torch.cuda.synchronize()
        assert O.normwise_error(y.float().cpu().numpy(), ref) <= TOL["f16"]


def test_gemv_many_matches_oracle_and_single_calls():
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(4242)
    shapes = [(8, 3, 300, 1000), (8, 3, 64, 8 * 40 + 3), (12, 4, 50, 600), (8, 3, 1000, 256),
              (8, 3, 17, 5000), (8, 3, 8, 8)]
    mats, refs, xs = [], [], []
    for C, P, rows, cols in shapes:
        s, c, e = _random_records(rng, rows, cols, C, P)
        mats.append(_pack(s, c, e, rows, cols, C, P))
        refs.append(O.decode_rows(s, c, e, cols, C, P))
        xs.append(rng.standard_normal((1, cols)).astype(np.float16))
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    for ydt in ("f16", "f32"):
        tdt = torch.float16 if ydt == "f16" else torch.float32
        ys = [torch.empty((1, m.rows), dtype=tdt, device=dev) for m in mats]
        _say(f"gemv_many {len(mats)} matrices -> {ydt}")
        S.seedlm_gemv_many(mats, xd, ys)
        torch.cuda.synchronize()
        for y, W_ref, x in zip(ys, refs, xs):
            assert O.normwise_error(y.float().cpu().numpy(), O.gemv(W_ref, x)) <= TOL[ydt]
        # begin + end gives the same bits as the one-shot call and as single calls
        ys2 = [torch.empty_like(y) for y in ys]
        S.seedlm_gemv_many(mats, xd, ys2, phase="begin")
        S.seedlm_gemv_many(mats, xd, ys2, phase="end")
        ys3 = [torch.empty_like(y) for y in ys]
        for m, x, y in zip(mats, xd, ys3):
            S.seedlm_gemv(m, x, y)
        # the same call marshalled once and run twice
        ys4 = [torch.empty_like(y) for y in ys]
        call = S.GemvManyCall(mats, xd, ys4)
        call()
        call(phase="begin")
        call(phase="end")
        torch.cuda.synchronize()
        for a, b, c3, c4 in zip(ys, ys2, ys3, ys4):
            assert torch.equal(a, b) and torch.equal(a, c3) and torch.equal(a, c4)


def test_gemv_many_takes_a_repeated_handle():
    # The handle holds no scratch, so one matrix may appear twice in a call.
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(1)
    rows, cols = 300, 8 * 100
    s, c, e = _random_records(rng, rows, cols, 8, 3)
    m = _pack(s, c, e, rows, cols, 8, 3)
    W_ref = O.decode_rows(s, c, e, cols, 8, 3)
    xs = [rng.standard_normal((1, cols)).astype(np.float16) for _ in range(2)]
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    ys = [torch.empty((1, rows), dtype=torch.float16, device=dev) for _ in range(2)]
    S.seedlm_gemv_many([m, m], xd, ys)
    single = [torch.empty_like(y) for y in ys]
    for x, y in zip(xd, single):
        S.seedlm_gemv(m, x, y)
    torch.cuda.synchronize()
    for y, y1, x in zip(ys, single, xs):
        assert O.normwise_error(y.float().cpu().numpy(), O.gemv(W_ref, x)) <= TOL["f16"]
        assert torch.equal(y, y1)


@pytest.mark.parametrize("batch", [1, 8])
def test_one_handle_on_two_streams_at_once(batch):
    # The handle is immutable and each stream has its own scratch: calls on two
    # streams that overlap on the GPU give the results of calls made alone.
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(2024 + batch)
    rows, cols = 8192, 8192
    s, c, e = _random_records(rng, rows, cols, 8, 3, (-12, -6))
    m = _pack(s, c, e, rows, cols, 8, 3)
    pick = _sample_rows(rows, rng)
    W_ref = O.decode_rows(s[pick], c[pick], e[pick], cols, 8, 3)
    xs = [rng.standard_normal((batch, cols)).astype(np.float16) for _ in range(2)]
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    alone = [torch.empty((batch, rows), dtype=torch.float16, device=dev) for _ in range(2)]
    for x, y in zip(xd, alone):
        S.seedlm_gemv(m, x, y, batch=batch)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(alone[0]) for _ in range(6)] for _ in range(2)]
    _say(f"two streams, batch {batch}")
    for k in range(6):  # interleaved launches, no synchronisation between them
        for i in range(2):
            S.seedlm_gemv(m, xd[i], outs[i][k], batch=batch, stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        for y in outs[i]:
            assert torch.equal(y, alone[i])
        yv = alone[i].float().cpu().numpy()[:, pick]
        assert O.normwise_error(yv, O.gemv(W_ref, xs[i])) <= TOL["f16"]


def test_packed_matrix_holds_only_its_compressed_bytes():
    # Device memory of packed matrices = their compressed bytes; the batch-1
    # scratch of a Llama-3-70B layer is 4 bytes per (panel, row).
    S = _S()
    dev = _dev()
    cfg = CONFIGS[4]
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info(dev)
    mats = []
    for mid, mat in enumerate(cfg.matrices):
        s, c, e = gen_records(4, mid, mat.rows, mat.cols, cfg.C, cfg.P)
        mats.append(_pack(s, c, e, mat.rows, mat.cols, cfg.C, cfg.P))
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(dev)
    packed = sum(m.compressed_bytes for m in mats)
    assert packed == 427819008
    used = free0 - free1
    _say(f"70B layer: {used} B of device memory for {packed} compressed bytes")
    assert used <= packed + (16 << 20)  # allocation granularity only
    def panels_times_padded_rows(mat):
        nb = -(-mat.cols // 8)
        return -(-nb // 32) * (-(-mat.rows // 8) * 8)

    want = 4 * sum(panels_times_padded_rows(mat) for mat in cfg.matrices)
    assert S.seedlm_gemv_scratch_bytes(mats, batch=1) == want == 13369344
    for m in mats:
        m.destroy()


@pytest.mark.parametrize("cid", [4, 3, 2], ids=["llama3_70b_4bit", "llama3_8b_3bit",
                                                "llama2_7b_4bit"])
def test_full_layer_gemv_many_sampled(cid):
    # The launch configuration the benchmark times: a whole layer in one call.
    S = _S()
    dev = _dev()
    cfg = CONFIGS[cid]
    mats, recs, xs, ys = [], [], [], []
    for mid, mat in enumerate(cfg.matrices):
        s, c, e = gen_records(cid, mid, mat.rows, mat.cols, cfg.C, cfg.P)
        mats.append(_pack(s, c, e, mat.rows, mat.cols, cfg.C, cfg.P))
        rng = np.random.default_rng([cid, mid, 888])
        pick = _sample_rows(mat.rows, rng, n=8)
        recs.append((pick, O.decode_rows(s[pick], c[pick], e[pick], mat.cols, cfg.C, cfg.P)))
        x = gen_x(cid, mid, 1, mat.cols, "f16")
        xs.append(x)
        ys.append(torch.empty((1, mat.rows), dtype=torch.float16, device=dev))
    _say(f"gemv_many over the {cfg.name} layer")
    S.seedlm_gemv_many(mats, [torch.from_numpy(x).to(dev) for x in xs], ys)
    torch.cuda.synchronize()
    for (pick, W_ref), x, y in zip(recs, xs, ys):
        yv = y.float().cpu().numpy()[:, pick]
        assert O.normwise_error(yv, O.gemv(W_ref, x)) <= TOL["f16"]


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_many_graph_replays_match_eager(batch):
    # A captured step (main + reduce launches; at batch 4 the grouped
    # matrix-core launches, both tilings and both formats) replayed several
    # times, with eager work and synchronizations between the replays; every
    # replay must give the eager call's bits.
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(777)
    shapes = [(8, 3, 512, 2048), (8, 3, 128, 2048), (8, 3, 1024, 640 + 5)]
    if batch > 1:
        shapes += [(12, 4, 300, 12 * 40 + 8), (8, 3, 8192, 8192)]  # the last: 256-row tiles
    mats, xs = [], []
    for C, P, rows, cols in shapes:
        s, c, e = _random_records(rng, rows, cols, C, P)
        mats.append(_pack(s, c, e, rows, cols, C, P))
        xs.append(torch.from_numpy(rng.standard_normal((batch, cols)).astype(np.float16)).to(dev))
    ys = [torch.empty((batch, m.rows), dtype=torch.float16, device=dev) for m in mats]
    ref = [torch.empty_like(y) for y in ys]
    S.seedlm_gemv_many(mats, xs, ref, batch=batch)
    # The capture stream gets its scratch from one eager call before capture
    # (allocation is not allowed while capturing).
    cs = torch.cuda.Stream()
    S.seedlm_gemv_many(mats, xs, ys, batch=batch, stream=cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        S.seedlm_gemv_many(mats, xs, ys, batch=batch, stream=cs)
    for k in range(4):
        for y in ys:
            y.fill_(float("nan"))
        # eager work between replays: the same matrices into other outputs
        other = [torch.empty_like(y) for y in ys]
        S.seedlm_gemv_many(mats, xs, other, batch=batch)
        torch.cuda.synchronize()
        _say(f"graph replay {k}")
        g.replay()
        torch.cuda.synchronize()
        for a, b, o in zip(ys, ref, other):
            assert torch.equal(a, b) and torch.equal(o, b)


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_many_more_than_one_group(batch):
    # Eleven matrices (more than one grouped launch), mixed formats, batch 1 and
    # 4 (the matrix-core path): every output against the oracle and against a
    # single seedlm_gemv call.
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(31 + batch)
    shapes = [(8, 3, 40 + 16 * k, 8 * (20 + 7 * k) + (k % 3)) for k in range(9)]
    shapes += [(12, 4, 50, 12 * 30 + 5), (8, 3, 8, 8)]
    mats, refs, xs = [], [], []
    for C, P, rows, cols in shapes:
        s, c, e = _random_records(rng, rows, cols, C, P)
        mats.append(_pack(s, c, e, rows, cols, C, P))
        refs.append(O.decode_rows(s, c, e, cols, C, P))
        xs.append(rng.standard_normal((batch, cols)).astype(np.float16))
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    ys = [torch.empty((batch, m.rows), dtype=torch.float16, device=dev) for m in mats]
    _say(f"gemv_many {len(mats)} matrices batch={batch}")
    S.seedlm_gemv_many(mats, xd, ys, batch=batch)
    single = [torch.empty_like(y) for y in ys]
    for m, x, y in zip(mats, xd, single):
        S.seedlm_gemv(m, x, y, batch=batch)
    torch.cuda.synchronize()
    for y, y1, W_ref, x in zip(ys, single, refs, xs):
        assert O.normwise_error(y.float().cpu().numpy(), O.gemv(W_ref, x)) <= TOL["f16"]
        assert torch.equal(y, y1)


def test_bench_timing_events_span_the_main_kernels():
    # seedlm_bench_time_next_call: the next call's main kernels record the two
    # events; the interval lies inside the call's own bracket, and the results
    # are those of an untimed call.
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(61)
    shapes = [(8, 3, 4096, 4096), (8, 3, 1024, 4096)]
    mats, xs = [], []
    for C, P, rows, cols in shapes:
        s, c, e = _random_records(rng, rows, cols, C, P, (-12, -6))
        mats.append(_pack(s, c, e, rows, cols, C, P))
        xs.append(torch.from_numpy(rng.standard_normal((1, cols)).astype(np.float16)).to(dev))
    ref = [torch.empty((1, m.rows), dtype=torch.float16, device=dev) for m in mats]
    S.seedlm_gemv_many(mats, xs, ref)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    stream = torch.cuda.current_stream()
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    ys = [torch.empty_like(y) for y in ref]
    ev[0].record(stream)
    S.seedlm_bench_time_next_call(ev[1], ev[2])
    S.seedlm_gemv_many(mats, xs, ys)
    ev[3].record(stream)
    torch.cuda.synchronize()
    kern, whole = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    _say(f"main kernel {kern * 1e3:.1f} us of a {whole * 1e3:.1f} us call")
    assert 0 < kern < whole
    assert all(torch.equal(a, b) for a, b in zip(ys, ref))
    with pytest.raises(S.SeedLMError):
        S.seedlm_bench_time_next_call(ev[1], None)


# The two packed formats beside the pages' ones: (8, 4, 16) with 3-bit
# coefficients and (12, 3, 20) with a 20-bit seed.  seedlm_decode must be
# bit-exact and seedlm_gemv (the exact per-lane kernel for these formats) meet
# the same bars, at ragged shapes, several batch sizes and every dtype pair.
OTHER_FORMATS = [
    # (C, P, K, rows, cols, batch, xdt, ydt)
    (8, 4, 16, 37, 8 * 45 + 5, 1, "f16", "f16"),
    (8, 4, 16, 300, 8 * 70, 3, "f32", "f32"),
    (8, 4, 16, 64, 1000, 8, "f16", "f32"),
    (12, 3, 20, 30, 12 * 70 + 7, 1, "f16", "f16"),
    (12, 3, 20, 129, 4096, 2, "f32", "f32"),
    (12, 3, 20, 70, 12 * 40 + 4, 16, "f16", "f16"),
    (12, 3, 20, 1, 5, 1, "f32", "f16"),
]


def _records_k(rng, rows, cols, C, P, K, Q, erange=(-15, 0)):
    nb = math.ceil(cols / C)
    s = rng.integers(1, 1 << K, (rows, nb)).astype(np.uint16 if K <= 16 else np.uint32)
    c = rng.integers(-(1 << (Q - 1)), 1 << (Q - 1), (rows, nb, P)).astype(np.int8)
    e = rng.integers(erange[0], erange[1] + 1, (rows, nb)).astype(np.int8)
    return s, c, e


@pytest.mark.parametrize("C,P,K,rows,cols,batch,xdt,ydt", OTHER_FORMATS,
                         ids=[f"C{c[0]}P{c[1]}K{c[2]}_{c[3]}x{c[4]}_b{c[5]}_{c[6]}{c[7]}"
                              for c in OTHER_FORMATS])
def test_other_packed_formats_decode_and_gemv(C, P, K, rows, cols, batch, xdt, ydt):
    S = _S()
    Q = O.PACKED_FORMATS[(C, P, K)]
    rng = np.random.default_rng(rows * 31 + cols + K)
    s, c, e = _records_k(rng, rows, cols, C, P, K, Q)
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, K)
    assert (m.C, m.P, m.K, m.Q) == (C, P, K, Q)
    W_ref = O.decode_rows(s, c, e, cols, C, P, K=K)
    _say(f"decode C={C} P={P} K={K} {rows}x{cols}")
    W = _decode_gpu(m, rows, cols).cpu().numpy()
    assert np.array_equal(W, W_ref.astype(np.float32)), "decode must be bit-exact"
    x = rng.standard_normal((batch, cols)).astype(np.float16 if xdt == "f16" else np.float32)
    _say(f"gemv C={C} P={P} K={K} batch={batch} {xdt}->{ydt}")
    y = _gemv_gpu(m, x, ydt)
    assert O.normwise_error(y, O.gemv(W_ref, x)) <= TOL[ydt]
    # the fast kernels take only the pages' formats
    for variant in (1, 4):
        with pytest.raises(S.SeedLMError) as err:
            _gemv_gpu(m, x, ydt, variant=variant)
        assert err.value.status == S.E_UNSUPPORTED


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_many_over_all_packed_formats(batch):
    # One call over matrices of all four formats: the pages' formats go through
    # their grouped kernels, the others through the exact kernel, and every
    # output equals a single call's and meets the oracle's bar.
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(808 + batch)
    shapes = [(8, 3, 16, 300, 1000), (8, 4, 16, 200, 8 * 50 + 3), (12, 4, 16, 50, 600),
              (12, 3, 20, 90, 12 * 30 + 5), (8, 3, 16, 1000, 256), (12, 3, 20, 8, 48)]
    mats, refs, xs = [], [], []
    for C, P, K, rows, cols in shapes:
        Q = O.PACKED_FORMATS[(C, P, K)]
        s, c, e = _records_k(rng, rows, cols, C, P, K, Q)
        mats.append(S.seedlm_pack(s, c, e, rows, cols, C, P, K))
        refs.append(O.decode_rows(s, c, e, cols, C, P, K=K))
        xs.append(rng.standard_normal((batch, cols)).astype(np.float16))
    xd = [torch.from_numpy(x).to(dev) for x in xs]
    ys = [torch.empty((batch, m.rows), dtype=torch.float16, device=dev) for m in mats]
    _say(f"gemv_many over four formats, batch {batch}")
    S.seedlm_gemv_many(mats, xd, ys, batch=batch)
    single = [torch.empty_like(y) for y in ys]
    for m, x, y in zip(mats, xd, single):
        S.seedlm_gemv(m, x, y, batch=batch)
    torch.cuda.synchronize()
    for y, y1, W_ref, x in zip(ys, single, refs, xs):
        assert torch.equal(y, y1)
        assert O.normwise_error(y.float().cpu().numpy(), O.gemv(W_ref, x)) <= TOL["f16"]


def test_prefill_paths_reject_the_other_formats():
    S = _S()
    dev = _dev()
    rng = np.random.default_rng(5)
    for C, P, K in ((8, 4, 16), (12, 3, 20)):
        Q = O.PACKED_FORMATS[(C, P, K)]
        rows, cols = 64, C * 32
        s, c, e = _records_k(rng, rows, cols, C, P, K, Q)
        m = S.seedlm_pack(s, c, e, rows, cols, C, P, K)
        X = torch.zeros((32, cols), dtype=torch.float16, device=dev)
        Y = torch.empty((32, rows), dtype=torch.float16, device=dev)
        with pytest.raises(S.SeedLMError) as err:
            S.seedlm_gemm(m, X, Y)
        assert err.value.status == S.E_UNSUPPORTED
        ws = torch.empty((S.seedlm_gemm_decoded_bytes(m) // 2,), dtype=torch.float16, device=dev)
        with pytest.raises(S.SeedLMError) as err:
            S.seedlm_gemm_decoded(m, X, Y, ws)
        assert err.value.status == S.E_UNSUPPORTED


DIRECT_CASES = [
    # (C, P, K, rows, cols, batch, xdt, ydt): the direct kernel in every format,
    # ragged rows, panels and blocks, batch 1 to 16, every dtype pair
    (8, 3, 16, 203, 8 * 97 + 3, 1, "f32", "f32"),
    (8, 3, 16, 2048, 2048, 1, "f16", "f16"),
    (8, 3, 16, 40, 520, 5, "f16", "f32"),
    (8, 3, 16, 1, 1, 16, "f32", "f16"),
    (12, 4, 16, 96, 12 * 77 + 8, 1, "f16", "f16"),
    (12, 4, 16, 17, 12 * 45 + 5, 16, "f32", "f32"),
    (8, 4, 16, 300, 8 * 70, 2, "f16", "f16"),
    (12, 3, 20, 70, 12 * 40 + 4, 1, "f32", "f32"),
    (12, 3, 20, 33, 12 * 33, 16, "f16", "f16"),
]


@pytest.mark.parametrize("C,P,K,rows,cols,batch,xdt,ydt", DIRECT_CASES,
                         ids=[f"C{c[0]}P{c[1]}K{c[2]}_{c[3]}x{c[4]}_b{c[5]}_{c[6]}{c[7]}"
                              for c in DIRECT_CASES])
def test_direct_kernel_against_oracle(C, P, K, rows, cols, batch, xdt, ydt):
    S = _S()
    Q = O.PACKED_FORMATS[(C, P, K)]
    rng = np.random.default_rng(rows * 7 + cols * 3 + batch)
    s, c, e = _records_k(rng, rows, cols, C, P, K, Q)
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, K)
    W_ref = O.decode_rows(s, c, e, cols, C, P, K=K)
    x = rng.standard_normal((batch, cols)).astype(np.float16 if xdt == "f16" else np.float32)
    _say(f"direct C={C} P={P} K={K} {rows}x{cols} batch={batch} {xdt}->{ydt}")
    y = _gemv_gpu(m, x, ydt, variant=5)
    assert O.normwise_error(y, O.gemv(W_ref, x)) <= TOL[ydt]
    assert np.array_equal(y, _gemv_gpu(m, x, ydt, variant=5))  # deterministic


def test_direct_kernel_on_long_rows_agrees_with_the_per_row_kernel():
    # A 14400-column (12,3,20) matrix (75 panels, x read from global memory),
    # the direct kernel against the oracle and against the one-wave-per-row
    # kernel, at the fp32 bar.
    S = _S()
    rows, cols, C, P, K = 24, 12 * 1200, 12, 3, 20
    rng = np.random.default_rng(12)
    s, c, e = _records_k(rng, rows, cols, C, P, K, 4)
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, K)
    x = rng.standard_normal((2, cols)).astype(np.float32)
    y_ref = O.gemv(O.decode_rows(s, c, e, cols, C, P, K=K), x)
    y = _gemv_gpu(m, x, "f32")
    assert O.normwise_error(y, y_ref) <= TOL["f32"]
    assert O.normwise_error(_gemv_gpu(m, x, "f32", variant=3), y_ref) <= TOL["f32"]
