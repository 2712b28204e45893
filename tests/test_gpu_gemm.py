"""GPU prefill GEMM (seedlm_gemm, through the C ABI) against the CPU oracle, in
both packed formats (4-bit C = 8, 3-bit C = 12).

Y = X W^T with W from the oracle's float64 decode of the same records and X the
same fp16 values.  Every token row of Y is a GEMV with fp16 output, so the bar
is that of the fp16-output GEMV: normwise max|y - y_ref| / max|y_ref| <= 2e-3
per token row.  Small shapes are checked on every output (ragged row, panel,
block-group and token tails included, for both token tilings: 256 tokens per
workgroup for short inputs, 512 otherwise); the full 8192x8192, 2048-token
shape on sampled rows and tokens, which the oracle computes one by one.  Small
grids of the 4-bit kernel split tiles along K (partials added by a second
launch); one launch with both whole and split tiles is checked on samples too.
"""
import ctypes

import numpy as np
import pytest

from oracle import seedlm_oracle as O
from workloads import gen_records, gen_x

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-3


def _S():
    import prng_seeded_decode_amd as S

    return S


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _run(cfg_id, rows, cols, ntok, C=8, P=3):
    dev = _dev()
    S = _S()
    s, c, e = gen_records(cfg_id, 0, rows, cols, C, P)
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, 16)
    X = gen_x(cfg_id, 0, ntok, cols, "f16")
    Xd = torch.from_numpy(X).to(dev)
    Y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    S.seedlm_gemm(m, Xd, Y)
    torch.cuda.synchronize()
    return (s, c, e), X, Y.cpu().numpy().astype(np.float64), m, Xd, Y


def _rowwise_err(Yg, Yr):
    return max(O.normwise_error(Yg[t], Yr[t]) for t in range(Yr.shape[0]))


@pytest.mark.parametrize("rows,cols,ntok", [
    (200, 296, 300),   # 37 blocks: a full and a 5-block panel; two token tiles, ragged
    (100, 64, 1),      # one K step, one token, rows not a multiple of 8
    (130, 520, 17),    # row tile tail of 2 rows
    (1000, 2048, 513),
    (4000, 256, 4100),  # enough tiles for the 512-token tiling, ragged rows and tokens
])
def test_gemm_matches_oracle_everywhere(rows, cols, ntok):
    _say(f"gemm {rows}x{cols} ntok={ntok}")
    (s, c, e), X, Yg, *_ = _run(61, rows, cols, ntok)
    W = O.decode_rows(s, c, e, cols, 8, 3)
    Yr = X.astype(np.float64) @ W.T
    err = _rowwise_err(Yg, Yr)
    _say(f"  max per-token normwise error {err:.2e}")
    assert err <= TOL


def test_gemm_full_shape_sampled():
    """The benchmark's shape: Llama-3-70B q_proj (8192x8192), 2048 tokens."""
    rows, cols, ntok = 8192, 8192, 2048
    _say(f"gemm sampled {rows}x{cols} ntok={ntok}")
    (s, c, e), X, Yg, *_ = _run(4, rows, cols, ntok)
    rng = np.random.default_rng(3)
    rs = np.concatenate([[0, rows - 1], rng.choice(rows, 30, replace=False)])
    ts = np.concatenate([[0, ntok - 1], rng.choice(ntok, 14, replace=False)])
    W = O.decode_rows(s[rs], c[rs], e[rs], cols, 8, 3)
    Yr = X[ts].astype(np.float64) @ W.T  # (tokens, sampled rows)
    err = _rowwise_err(Yg[np.ix_(ts, rs)], Yr)
    _say(f"  sampled max per-token normwise error {err:.2e}")
    assert err <= TOL


def test_gemm_whole_and_split_tiles_sampled():
    """320 tiles of 128 rows x 512 tokens: on 256 compute units the last 64 (the
    second token tile's rows 12288..20479) run as four K parts each, whose fp32
    partials the fixup launch adds; the other 256 run whole."""
    S = _S()
    rows, cols, ntok = 20480, 1024, 1024
    _say(f"gemm sampled {rows}x{cols} ntok={ntok} (whole and split tiles)")
    (s, c, e), X, Yg, m, *_ = _run(67, rows, cols, ntok)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus == 256:  # 64 tiles x 4 parts x 128 x 512 fp32 partials
        assert S.seedlm_gemm_scratch_bytes(m, ntok) == 64 * 4 * 128 * 512 * 4
    rng = np.random.default_rng(7)
    rs = np.concatenate([[0, rows - 1, 12287, 12288], rng.choice(rows, 40, replace=False)])
    ts = np.concatenate([[0, 511, 512, ntok - 1], rng.choice(ntok, 12, replace=False)])
    W = O.decode_rows(s[rs], c[rs], e[rs], cols, 8, 3)
    Yr = X[ts].astype(np.float64) @ W.T
    err = _rowwise_err(Yg[np.ix_(ts, rs)], Yr)
    _say(f"  sampled max per-token normwise error {err:.2e}")
    assert err <= TOL


def test_gemm_scratch_bytes():
    """A matrix with too few K steps to split needs no scratch; a small grid's
    tiles split (on 256 compute units), in both formats."""
    S = _S()
    _dev()
    s, c, e = gen_records(68, 0, 256, 64, 8, 3)
    m0 = S.seedlm_pack(s, c, e, 256, 64, 8, 3, 16)
    assert S.seedlm_gemm_scratch_bytes(m0, 600) == 0  # 2 K steps
    s, c, e = gen_records(68, 1, 256, 1024, 8, 3)
    m = S.seedlm_pack(s, c, e, 256, 1024, 8, 3, 16)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 2 x 2 tiles of 512 tokens, 32 K steps -> 4 parts of 8 steps
        assert S.seedlm_gemm_scratch_bytes(m, 600) == 4 * 4 * 128 * 512 * 4
        # one token: 2 tiles of 256 tokens, 4 parts
        assert S.seedlm_gemm_scratch_bytes(m, 1) == 2 * 4 * 128 * 256 * 4
    s3, c3, e3 = gen_records(68, 2, 256, 1200, 12, 4)
    m3 = S.seedlm_pack(s3, c3, e3, 256, 1200, 12, 4, 16)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 3-bit: 2 x 3 tiles of 128 x 256, 25 K steps -> 3 parts (9, 9 and 7 steps)
        assert S.seedlm_gemm_scratch_bytes(m3, 600) == 6 * 3 * 128 * 256 * 4


# 3-bit format (C = 12, P = 4): K steps of 48 columns (4 blocks) and 256-token
# tiles.  cols = 8 mod 12 ends inside a block; nb = 1, 2, 3 mod 4 leave a short
# last group (zero-padded slots); nb = 33, 37 leave a short last panel.
@pytest.mark.parametrize("rows,cols,ntok", [
    (200, 400, 300),   # 34 blocks (last one 4 columns short), two token tiles, ragged
    (100, 48, 1),      # one K step, one token
    (130, 440, 17),    # 37 blocks: row tile tail of 2 rows, 1-block last group
    (8, 24, 5),        # two blocks
    (1000, 2048, 513),  # 171 blocks (6 panels), ragged tokens
    (300, 4096, 256),  # exactly one token tile
])
def test_gemm_3bit_matches_oracle_everywhere(rows, cols, ntok):
    _say(f"gemm 3-bit {rows}x{cols} ntok={ntok}")
    (s, c, e), X, Yg, *_ = _run(63, rows, cols, ntok, C=12, P=4)
    W = O.decode_rows(s, c, e, cols, 12, 4)
    Yr = X.astype(np.float64) @ W.T
    err = _rowwise_err(Yg, Yr)
    _say(f"  max per-token normwise error {err:.2e}")
    assert err <= TOL


def test_gemm_3bit_layer_shape_sampled():
    """Llama-3-8B gate projection (14336x4096, 3-bit), 2048 tokens, sampled."""
    rows, cols, ntok = 14336, 4096, 2048
    _say(f"gemm 3-bit sampled {rows}x{cols} ntok={ntok}")
    (s, c, e), X, Yg, *_ = _run(3, rows, cols, ntok, C=12, P=4)
    rng = np.random.default_rng(4)
    rs = np.concatenate([[0, rows - 1], rng.choice(rows, 30, replace=False)])
    ts = np.concatenate([[0, ntok - 1], rng.choice(ntok, 14, replace=False)])
    W = O.decode_rows(s[rs], c[rs], e[rs], cols, 12, 4)
    Yr = X[ts].astype(np.float64) @ W.T
    err = _rowwise_err(Yg[np.ix_(ts, rs)], Yr)
    _say(f"  sampled max per-token normwise error {err:.2e}")
    assert err <= TOL


def test_gemm_3bit_matches_batched_gemv():
    """For a few tokens the prefill GEMM and the skinny matrix-core GEMV compute
    the same exact-decode products (fp32 accumulation, different order)."""
    dev = _dev()
    S = _S()
    rows, cols, ntok = 520, 12 * 90 + 8, 16
    (s, c, e), X, Yg, m, Xd, _ = _run(64, rows, cols, ntok, C=12, P=4)
    Yb = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    S.seedlm_gemv(m, Xd, Yb, batch=ntok)
    torch.cuda.synchronize()
    assert _rowwise_err(Yg, Yb.cpu().numpy().astype(np.float64)) <= TOL


def test_gemm_deterministic_and_rejects_unsupported():
    dev = _dev()
    S = _S()
    _, _, Y1, m, Xd, Y = _run(62, 256, 512, 260)
    S.seedlm_gemm(m, Xd, Y)
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), Y1)
    # fp32 activations: not supported by this entry point
    with pytest.raises(S.SeedLMError):
        S.seedlm_gemm(m, Xd.float(), Y)
    # 3-bit: deterministic too; cols not a multiple of 8 is rejected
    _, _, Y3a, m3, X3, Y3 = _run(62, 300, 480, 260, C=12, P=4)
    S.seedlm_gemm(m3, X3, Y3)
    torch.cuda.synchronize()
    assert np.array_equal(Y3.cpu().numpy().astype(np.float64), Y3a)
    s, c, e = gen_records(62, 1, 64, 100, 12, 4)
    m4 = S.seedlm_pack(s, c, e, 64, 100, 12, 4, 16)
    X4 = torch.zeros((8, 100), dtype=torch.float16, device=dev)
    Y4 = torch.empty((8, 64), dtype=torch.float16, device=dev)
    with pytest.raises(S.SeedLMError):
        S.seedlm_gemm(m4, X4, Y4)
    # more token tiles than grid.y holds: rejected before any launch (the
    # pointers are never read)
    for mm in (m, m3):
        assert S.lib().seedlm_gemm(mm.handle, ctypes.c_void_p(Xd.data_ptr()),
                                   ctypes.c_void_p(Y.data_ptr()), 65535 * 256 + 1, S.F16, S.F16,
                                   None) == S.E_UNSUPPORTED


# seedlm_gemm_decoded: W rebuilt once into a caller workspace as fp16(w * 2^10),
# then hipBLASLt.  The workspace is checked bit for bit against the oracle's
# float64 weights times 2^10 rounded to fp16 (round to nearest even, as the
# kernel's conversion); the product at the GEMV bar per token row.
@pytest.mark.parametrize("C,P,rows,cols,ntok", [
    (8, 3, 200, 296, 300),      # 37 blocks: a full and a 5-block panel, ragged tokens
    (8, 3, 130, 520, 17),       # rows not a multiple of 8
    (12, 4, 200, 400, 300),     # 34 blocks, the last 4 columns short
    (12, 4, 130, 440, 513),     # 37 blocks, last block 8 columns
    (12, 4, 1000, 2048, 600),   # 171 blocks over 6 panels
])
def test_gemm_decoded_matches_oracle_and_exact_workspace(C, P, rows, cols, ntok):
    dev = _dev()
    S = _S()
    s, c, e = gen_records(65, 0, rows, cols, C, P)
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, 16)
    X = gen_x(65, 0, ntok, cols, "f16")
    Xd = torch.from_numpy(X).to(dev)
    Y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    nbytes = S.seedlm_gemm_decoded_bytes(m)
    assert nbytes == ((rows * cols * 2 + 255) // 256) * 256 + (32 << 20)
    ws = torch.full((nbytes // 2,), float("nan"), dtype=torch.float16, device=dev)
    _say(f"gemm decoded C={C} {rows}x{cols} ntok={ntok}")
    S.seedlm_gemm_decoded(m, Xd, Y, ws)
    torch.cuda.synchronize()
    W = O.decode_rows(s, c, e, cols, C, P)
    want = (W * 1024.0).astype(np.float16)
    got = ws[: rows * cols].cpu().numpy().reshape(rows, cols)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), "decoded workspace must be exact"
    err = _rowwise_err(Y.cpu().numpy().astype(np.float64), X.astype(np.float64) @ W.T)
    _say(f"  max per-token normwise error {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("C,P,rows,cols,ntok,extra", [
    (8, 3, 264, 512, 1, 1000),     # one token; scratch not a multiple of 256
    (12, 4, 96, 480, 5, 37),       # five tokens; 37 bytes past the matrix: no scratch
    (8, 3, 72, 136, 3, 0),         # exactly the decoded size
])
def test_gemm_decoded_few_tokens_and_odd_scratch(C, P, rows, cols, ntok, extra):
    """Token counts below the GEMV batch limit and workspaces whose scratch part is
    short, ragged or absent: the product is still at the GEMV bar."""
    dev = _dev()
    S = _S()
    s, c, e = gen_records(66, 0, rows, cols, C, P)
    m = S.seedlm_pack(s, c, e, rows, cols, C, P, 16)
    X = gen_x(66, 0, ntok, cols, "f16")
    Xd = torch.from_numpy(X).to(dev)
    Y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    ws = torch.empty((rows * cols * 2 + extra,), dtype=torch.uint8, device=dev)
    _say(f"gemm decoded C={C} {rows}x{cols} ntok={ntok} extra={extra}")
    S.seedlm_gemm_decoded(m, Xd, Y, ws)
    torch.cuda.synchronize()
    W = O.decode_rows(s, c, e, cols, C, P)
    assert _rowwise_err(Y.cpu().numpy().astype(np.float64), X.astype(np.float64) @ W.T) <= TOL


def test_gemm_decoded_from_two_host_threads():
    """Two host threads call seedlm_gemm_decoded at once (the binding releases the
    interpreter lock during the call), each on its own stream and workspace, over
    shapes whose plans are not cached yet; every result matches a call made alone."""
    import threading

    dev = _dev()
    S = _S()
    shapes = [(8, 3, 520, 1024, 40), (12, 4, 384, 960, 24)]
    jobs = []
    for k, (C, P, rows, cols, ntok) in enumerate(shapes):
        s, c, e = gen_records(67, k, rows, cols, C, P)
        m = S.seedlm_pack(s, c, e, rows, cols, C, P, 16)
        Xd = torch.from_numpy(gen_x(67, k, ntok, cols, "f16")).to(dev)
        ws = torch.empty((S.seedlm_gemm_decoded_bytes(m),), dtype=torch.uint8, device=dev)
        outs = [torch.empty((ntok, rows), dtype=torch.float16, device=dev) for _ in range(6)]
        jobs.append((m, Xd, ws, outs, torch.cuda.Stream(device=dev)))
    torch.cuda.synchronize()  # inputs uploaded before the side streams read them
    errors = []

    def work(job):
        m, Xd, ws, outs, st = job
        try:
            for Y in outs:
                S.seedlm_gemm_decoded(m, Xd, Y, ws, stream=st)
            st.synchronize()
        except Exception as ex:  # reported by the main thread
            errors.append(ex)

    _say("gemm decoded from two threads")
    ts = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    for m, Xd, ws, outs, _ in jobs:
        alone = torch.empty_like(outs[0])
        S.seedlm_gemm_decoded(m, Xd, alone, ws)
        torch.cuda.synchronize()
        ref = alone.cpu().numpy().astype(np.float64)
        for Y in outs:
            assert _rowwise_err(Y.cpu().numpy().astype(np.float64), ref) <= 1e-3


def test_gemm_decoded_full_shape_sampled_and_rejects():
    """Llama-3-70B gate projection (28672x8192, 4-bit), 2048 tokens, sampled; and
    the argument checks."""
    dev = _dev()
    S = _S()
    rows, cols, ntok = 28672, 8192, 2048
    s, c, e = gen_records(4, 4, rows, cols, 8, 3)
    m = S.seedlm_pack(s, c, e, rows, cols, 8, 3, 16)
    X = gen_x(4, 4, ntok, cols, "f16")
    Xd = torch.from_numpy(X).to(dev)
    Y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    ws = torch.empty((rows * cols,), dtype=torch.float16, device=dev)
    _say(f"gemm decoded sampled {rows}x{cols} ntok={ntok}")
    S.seedlm_gemm_decoded(m, Xd, Y, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rs = np.concatenate([[0, rows - 1], rng.choice(rows, 30, replace=False)])
    ts = np.concatenate([[0, ntok - 1], rng.choice(ntok, 14, replace=False)])
    W = O.decode_rows(s[rs], c[rs], e[rs], cols, 8, 3)
    Yr = X[ts].astype(np.float64) @ W.T
    Yg = Y.cpu().numpy().astype(np.float64)
    assert _rowwise_err(Yg[np.ix_(ts, rs)], Yr) <= TOL
    # the fused kernel computes the same product
    Yf = torch.empty_like(Y)
    S.seedlm_gemm(m, Xd, Yf)
    torch.cuda.synchronize()
    assert _rowwise_err(Yg, Yf.cpu().numpy().astype(np.float64)) <= TOL
    # the workspace above leaves the GEMM no scratch; again with the full size
    ws2 = torch.empty((S.seedlm_gemm_decoded_bytes(m) // 2,), dtype=torch.float16, device=dev)
    Y2 = torch.empty_like(Y)
    S.seedlm_gemm_decoded(m, Xd, Y2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(ws2[: rows * cols], ws)
    assert _rowwise_err(Y2.cpu().numpy().astype(np.float64), Yg) <= TOL
    del ws2, Y2
    # workspace one element short; fp32 activations
    with pytest.raises(S.SeedLMError):
        S.seedlm_gemm_decoded(m, Xd, Y, ws[: rows * cols - 1])
    with pytest.raises(S.SeedLMError):
        S.seedlm_gemm_decoded(m, Xd.float(), Y, ws)


@pytest.mark.parametrize("ntok", [512, 1024])
def test_gemm_decoded_long_k_shape(ntok):
    """Llama-3-70B down projection (8192x28672, 4-bit): at 512 and 1024 tokens
    hipBLASLt's first heuristic candidate wants more scratch than the workspace
    offers, and the plan must fall back to one that fits.  Sampled against the
    oracle, and equal to the fused kernel within the bar."""
    dev = _dev()
    S = _S()
    rows, cols = 8192, 28672
    s, c, e = gen_records(4, 6, rows, cols, 8, 3)
    m = S.seedlm_pack(s, c, e, rows, cols, 8, 3, 16)
    X = gen_x(4, 6, ntok, cols, "f16")
    Xd = torch.from_numpy(X).to(dev)
    ws = torch.empty((S.seedlm_gemm_decoded_bytes(m) // 2,), dtype=torch.float16, device=dev)
    Y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
    _say(f"gemm decoded sampled {rows}x{cols} ntok={ntok}")
    S.seedlm_gemm_decoded(m, Xd, Y, ws)
    Yf = torch.empty_like(Y)
    S.seedlm_gemm(m, Xd, Yf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(ntok)
    rs = np.concatenate([[0, rows - 1], rng.choice(rows, 24, replace=False)])
    ts = np.concatenate([[0, ntok - 1], rng.choice(ntok, 10, replace=False)])
    W = O.decode_rows(s[rs], c[rs], e[rs], cols, 8, 3)
    Yr = X[ts].astype(np.float64) @ W.T
    Yg = Y.cpu().numpy().astype(np.float64)
    assert _rowwise_err(Yg[np.ix_(ts, rs)], Yr) <= TOL
    assert _rowwise_err(Yg, Yf.cpu().numpy().astype(np.float64)) <= TOL


def test_gemm_split_tiles_graph_replays_and_two_streams():
    """Split-tile calls (three launches and the stream's scratch) captured in a HIP
    graph and replayed with eager work between the replays, and run on two streams
    at once: every result must equal the eager call's bits."""
    dev = _dev()
    S = _S()
    shapes = [(8, 3, 1024, 2048, 600), (12, 4, 1000, 2048, 513)]
    mats, xs, ref = [], [], []
    for k, (C, P, rows, cols, ntok) in enumerate(shapes):
        s, c, e = gen_records(69, k, rows, cols, C, P)
        m = S.seedlm_pack(s, c, e, rows, cols, C, P, 16)
        x = torch.from_numpy(gen_x(69, k, ntok, cols, "f16")).to(dev)
        y = torch.empty((ntok, rows), dtype=torch.float16, device=dev)
        S.seedlm_gemm(m, x, y)
        mats.append(m)
        xs.append(x)
        ref.append(y)
    torch.cuda.synchronize()
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert all(S.seedlm_gemm_scratch_bytes(m, x.shape[0]) > 0 for m, x in zip(mats, xs))
    # graph: the capture stream gets its scratch from one eager call first
    cs = torch.cuda.Stream()
    ys = [torch.empty_like(y) for y in ref]
    for m, x, y in zip(mats, xs, ys):
        S.seedlm_gemm(m, x, y, stream=cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for m, x, y in zip(mats, xs, ys):
            S.seedlm_gemm(m, x, y, stream=cs)
    for k in range(4):
        for y in ys:
            y.fill_(float("nan"))
        other = [torch.empty_like(y) for y in ref]
        for m, x, o in zip(mats, xs, other):
            S.seedlm_gemm(m, x, o)
        torch.cuda.synchronize()
        _say(f"gemm graph replay {k}")
        g.replay()
        torch.cuda.synchronize()
        for a, b, o in zip(ys, ref, other):
            assert torch.equal(a, b) and torch.equal(o, b)
    # two streams at once, interleaved, no synchronisation between the calls
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(ref[i]) for _ in range(4)] for i in range(2)]
    _say("gemm on two streams")
    for k in range(4):
        for i in range(2):
            S.seedlm_gemm(mats[i], xs[i], outs[i][k], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        for y in outs[i]:
            assert torch.equal(y, ref[i])
