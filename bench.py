"""Benchmark: SeedLM fused decode-GEMV on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 4] [--batch 1]

One step = one batch-1 pass of the fused decode-GEMV over every weight matrix
of one synthetic Llama-3-70B decoder layer (q, k, v, o 8192x8192 / 1024x8192,
gate, up 28672x8192, down 8192x28672), 4-bit SeedLM (C=8, P=3, K=16), fp16 x
and y, inputs resident in HBM.  Records are drawn by workloads.gen_records
(seeds uniform in [1, 65535], coefficients uniform in [-8, 7], exponents uniform
in [-12, -6]); x is N(0,1) fp16.  Two copies of the layer's packed buffers are
rotated so that consecutive steps do not find their weights in the 256 MB MALL.

Prints one JSON line: effective weights/s (value), compressed HBM GB/s and its
fraction of 8 TB/s, the roofline of the fused kernel (HIP events on the launch
stream), the measured streaming-read ceiling of the device and the kernel's
fraction of it, the same-chip fp16 GEMV baseline and its speed-up, and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py --encode [--encode-bits 4|3] [--steps K] [--warmup W]

times the seed-search encoder instead, and

    python bench.py --gemm [--tokens 2048]

(--sweep: the design-space sweep of the encoder over (C, P) on Gaussian
weights) or the prefill decode-GEMM (one step = the layer's 7 matrices at that many
tokens, with torch's dense fp16 GEMM on the same shapes beside it).  In the
encoder mode one step = one 8192x8192 bf16 matrix (Llama-3-70B q_proj shape)
encoded by exhaustive search over all 65535 seeds.  Each mode prints its own
JSON line with its dominant kernel's roofline and the oracle timed on a
bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
def _csrc(*names):
    return [os.path.join(ROOT, "prng_seeded_decode_amd", "csrc", f) for f in names]


# Committed HBM-traffic counter summaries of the batch-1 fused kernels, per workload
# (config id), with the kernel sources they were taken on.
TRAFFIC_FILES = {
    4: (os.path.join(ROOT, "profiles", "gemv_lut_kernel_llama3_70b_layer_4bit_traffic.txt"),
        _csrc("gemv_lut.hip", "lut_common.h")),
    2: (os.path.join(ROOT, "profiles", "gemv_lut_kernel_llama2_7b_layer_4bit_traffic.txt"),
        _csrc("gemv_lut.hip", "lut_common.h")),
    3: (os.path.join(ROOT, "profiles", "gemv_lut12_kernel_llama3_8b_layer_3bit_counters.txt"),
        _csrc("gemv_lut12.hip", "lut_common.h")),
}


def measured_traffic(config_id):
    """HBM bytes per launch of the fused kernel from the committed counter summary,
    or None when there is none for the workload or the kernel source has changed
    since the counters were taken."""
    import hashlib

    if config_id not in TRAFFIC_FILES:
        return None
    path_txt, sources = TRAFFIC_FILES[config_id]
    try:
        with open(path_txt) as f:
            kv = dict(line.split(None, 1) for line in f
                      if line.strip() and not line.startswith("#"))
        h = hashlib.sha256()
        for path in sources:
            with open(path, "rb") as f:
                h.update(f.read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    if kv.get("source_sha256", "").strip() != digest:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))
METRIC = "effective weights/s + compressed HBM GB/s (% peak), 4-bit decode-GEMV bs=1"


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # Warm-up steps (default 20; 3 seed searches).  The decode-GEMV modes then run
    # a fixed-duration settle phase (--settle-ms) before timing: the part needs
    # tens of milliseconds of load to reach its steady clocks, so a step count
    # alone would make the result depend on the step's length.
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--config", type=int, default=4)
    p.add_argument("--batch", type=int, default=1)
    p.add_argument("--variant", type=int, default=0)
    p.add_argument("--copies", type=int, default=0,
                   help="rotated copies of the packed layer (default: enough to exceed 600 MB, "
                        "2 to 64)")
    p.add_argument("--settle-ms", type=float, default=150.0,
                   help="wall-clock milliseconds of the same steps run after the warm-up and "
                        "before timing, so that the GPU clocks have settled")
    p.add_argument("--no-fp16", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-read-ceiling", action="store_true",
                   help="skip the streaming-read ceiling measurement")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--per-matrix", action="store_true",
                   help="also time one seedlm_gemv per matrix (extra launches of the same kernels)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one plain fp32 copy kernel of this many MiB first (counter calibration)")
    p.add_argument("--decode", action="store_true",
                   help="also time seedlm_decode (dense fp32 W) on the largest matrix")
    p.add_argument("--graph", type=int, default=0,
                   help="1: replay each step as a captured HIP graph (one per rotated copy)")
    p.add_argument("--gemm", action="store_true",
                   help="time the prefill decode-GEMM instead (one step = a layer at --tokens)")
    p.add_argument("--tokens", type=int, default=2048)
    p.add_argument("--sweep", action="store_true",
                   help="design-space sweep: reconstruction error of Gaussian blocks per (C, P)")
    p.add_argument("--encode", action="store_true",
                   help="time the seed-search encoder instead (one step = one matrix encoded)")
    p.add_argument("--encode-bits", type=int, default=4, choices=(3, 4))
    p.add_argument("--encode-shape", type=str, default="",
                   help="rows,cols of the encoded matrix (default: the Llama-3-70B q_proj "
                        "shape, columns rounded up to a multiple of C)")
    return p.parse_args()


def cpu_baseline(cfg, budget_s):
    """Time the oracle (decode + float64 matvec) on sampled rows of each matrix,
    on one host thread (BLAS limited to one thread for the matvec too)."""
    from oracle import seedlm_oracle as O
    from workloads import gen_records, gen_x

    rows_per = 8
    weights = 0
    t_dec = t_mv = 0.0
    rounds = 0
    recs = []
    for mid, mat in enumerate(cfg.matrices):
        s, c, e = gen_records(cfg.config_id, mid, mat.rows, mat.cols, cfg.C, cfg.P)
        x = gen_x(cfg.config_id, mid, 1, mat.cols, cfg.x_dtype)
        recs.append((mat, s, c, e, x))
    rng = np.random.default_rng(12345)
    import contextlib

    try:
        from threadpoolctl import threadpool_limits

        one_thread = threadpool_limits(limits=1)
    except Exception:
        one_thread = contextlib.nullcontext()
    with one_thread:
        while t_dec + t_mv < budget_s:
            for mat, s, c, e, x in recs:
                pick = rng.choice(mat.rows, size=min(rows_per, mat.rows), replace=False)
                t0 = time.perf_counter()
                W = O.decode_rows(s[pick], c[pick], e[pick], mat.cols, cfg.C, cfg.P)
                t1 = time.perf_counter()
                O.gemv(W, x)
                t2 = time.perf_counter()
                t_dec += t1 - t0
                t_mv += t2 - t1
                weights += len(pick) * mat.cols
            rounds += 1
            rows_per = min(rows_per * 2, 256)
    n = len(cfg.matrices)
    return {
        "value": weights / (t_dec + t_mv),
        "unit": "weights/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{weights} weights from sampled rows of the {n} matri"
                   f"{'ces' if n > 1 else 'x'} ({rounds} rounds), one host thread: "
                   f"decode {t_dec:.2f} s, float64 matvec {t_mv:.2f} s; host cores "
                   f"available {len(os.sched_getaffinity(0))}"),
    }


ENC_METRIC = "encoded weights/s (bf16 -> SeedLM, exhaustive search over all 65535 seeds)"
BF16_MFMA_PEAK_TFLOPS = 2500.0


def cpu_encode_baseline(bits, C, P, budget_s):
    """Time the oracle's exhaustive encoder on whole blocks sampled from the matrix."""
    from oracle import seedlm_oracle as O
    from workloads import bf16_to_float64

    Wb = bf16_to_float64(bits).reshape(-1, C)
    rng = np.random.default_rng(4321)
    n, blocks, t = 8, 0, 0.0
    while t < budget_s:
        pick = rng.choice(Wb.shape[0], size=n, replace=False)
        t0 = time.perf_counter()
        O.encode_exhaustive(Wb[pick], C, P)
        t += time.perf_counter() - t0
        blocks += n
        n = min(2 * n, 256)
    try:
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {
        "value": blocks * C / t,
        "unit": "weights/s",
        "cores": int(max(1, blas)),
        "kind": "oracle",
        "sample": (f"{blocks} blocks ({blocks * C} weights) sampled from the matrix, each "
                   f"searched over all 65535 seeds by encode_exhaustive (NumPy float64) in "
                   f"{t:.2f} s; host cores available {len(os.sched_getaffinity(0))}"),
    }


def encode_main(args):
    import torch

    import prng_seeded_decode_amd as S
    from workloads import gen_bf16_weights

    C, P = (8, 3) if args.encode_bits == 4 else (12, 4)
    if args.encode_shape:
        rows, cols = (int(v) for v in args.encode_shape.split(","))
    else:
        rows, cols = 8192, -(-8192 // C) * C
    bits = gen_bf16_weights(40, C, rows, cols, scale=0.02)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    W = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    enc = S.SeedLMEncoder(C, P, 16)
    outs = S.seedlm_encode(enc, W, stream=stream)
    for _ in range(args.warmup):
        S.seedlm_encode(enc, W, *outs, stream=stream)
    torch.cuda.synchronize()
    evs = []
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        S.seedlm_encode(enc, W, *outs, stream=stream)
        b.record(stream)
        evs.append((a, b))
    ev1.record(stream)
    ev1.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kern_s = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3
    nblk = rows * cols // C
    pairs = nblk * 65535
    # Roofline of the search kernel: the algorithmic contraction is the pages'
    # t* = pinv(U(s)) w for every block and seed, 2*C*P flops per (block, seed)
    # pair, priced at the bf16 matrix-core peak (the kernel's operand type).
    alg_flops = 2.0 * C * P * pairs
    achieved = alg_flops / kern_s / 1e12
    out = {
        "metric": ENC_METRIC,
        "value": rows * cols / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"seed search: {rows}x{cols} bf16 N(0, 0.02^2) weights (Llama-3-70B "
                         f"q_proj shape) -> SeedLM C={C} P={P} K=16, all 65535 seeds per block"),
            "blocks": nblk,
            "block_seed_pairs": pairs,
        },
        "pairs_per_s": pairs / kern_s,
        "kernel_ms_per_launch": round(kern_s * 1e3, 3),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_encode_baseline(bits, C, P, args.cpu_seconds)
    enc.destroy()
    print(json.dumps(out), flush=True)


GEMM_METRIC = "prefill tokens/s through one decoder layer (decode-GEMM on the matrix cores)"
F16_MFMA_PEAK_TFLOPS = 2500.0


def cpu_gemm_baseline(cfg, ntok, budget_s):
    """Time the oracle (decode + float64 product) on sampled rows x sampled tokens."""
    from oracle import seedlm_oracle as O
    from workloads import gen_records, gen_x

    rng = np.random.default_rng(777)
    flops, t, rounds = 0.0, 0.0, 0
    nr, nt = 4, 16
    while t < budget_s:
        for mid, mat in enumerate(cfg.matrices):
            s, c, e = gen_records(cfg.config_id, mid, mat.rows, mat.cols, cfg.C, cfg.P)
            pick = rng.choice(mat.rows, size=nr, replace=False)
            X = gen_x(cfg.config_id, mid, nt, mat.cols, "f16").astype(np.float64)
            t0 = time.perf_counter()
            W = O.decode_rows(s[pick], c[pick], e[pick], mat.cols, cfg.C, cfg.P)
            X @ W.T
            t += time.perf_counter() - t0
            flops += 2.0 * nr * nt * mat.cols
        rounds += 1
        nr = min(2 * nr, 64)
    layer_flops_per_token = 2.0 * sum(m.rows * m.cols for m in cfg.matrices)
    try:
        from threadpoolctl import threadpool_info

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {
        "value": flops / t / layer_flops_per_token,
        "unit": "tokens/s",
        "cores": int(max(1, blas)),
        "kind": "oracle",
        "sample": (f"sampled rows x 16 tokens of the 7 layer matrices ({rounds} rounds, "
                   f"{flops / 1e9:.1f} GFLOP) in {t:.2f} s: oracle decode (NumPy) + float64 "
                   f"product, scaled to whole-layer tokens/s; host cores available "
                   f"{len(os.sched_getaffinity(0))}"),
    }


def gemm_main(args):
    import torch

    import prng_seeded_decode_amd as S
    from workloads import CONFIGS, gen_records

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ntok = args.tokens
    mats, xs, ys = [], [], []
    for mid, mat in enumerate(cfg.matrices):
        s, c, e = gen_records(cfg.config_id, mid, mat.rows, mat.cols, cfg.C, cfg.P)
        mats.append(S.seedlm_pack(s, c, e, mat.rows, mat.cols, cfg.C, cfg.P, cfg.K))
        g = torch.Generator(device=dev).manual_seed(1000 + mid)
        xs.append(torch.randn((ntok, mat.cols), generator=g, device=dev).half())
        ys.append(torch.empty((ntok, mat.rows), dtype=torch.float16, device=dev))

    def step():
        for m, x, y in zip(mats, xs, ys):
            S.seedlm_gemm(m, x, y, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    ev1.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    # the dominant kernel: the 28672x8192 / 8192x28672 launches, timed alone
    big = max(range(len(mats)), key=lambda i: cfg.matrices[i].rows * cfg.matrices[i].cols)
    evs = []
    for _ in range(args.steps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        S.seedlm_gemm(mats[big], xs[big], ys[big], stream=stream)
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    kern_s = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3
    bm = cfg.matrices[big]
    alg_flops = 2.0 * bm.rows * bm.cols * ntok
    achieved = alg_flops / kern_s / 1e12
    layer_weights = sum(m.rows * m.cols for m in cfg.matrices)
    # the same step through seedlm_gemm_decoded: W rebuilt into one shared fp16
    # workspace per matrix in turn (with the GEMM's scratch), then hipBLASLt
    ws = torch.empty((max(S.seedlm_gemm_decoded_bytes(m) for m in mats) // 2,),
                     dtype=torch.float16, device=dev)

    def step_decoded():
        for m, x, y in zip(mats, xs, ys):
            S.seedlm_gemm_decoded(m, x, y, ws, stream=stream)

    for _ in range(args.warmup):
        step_decoded()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step_decoded()
    ev1.record(stream)
    ev1.synchronize()
    dec_ms = ev0.elapsed_time(ev1) / args.steps
    del ws
    # same-chip dense fp16 baseline (torch.matmul -> hipBLASLt) on the same shapes
    dense = None
    if not args.no_fp16:
        Ws = [torch.randn((m.rows, m.cols), device=dev).half() for m in cfg.matrices]
        for _ in range(args.warmup):
            for W, x, y in zip(Ws, xs, ys):
                torch.matmul(x, W.t(), out=y)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            for W, x, y in zip(Ws, xs, ys):
                torch.matmul(x, W.t(), out=y)
        ev1.record(stream)
        ev1.synchronize()
        dms = ev0.elapsed_time(ev1) / args.steps
        dense = {"ms_per_step": round(dms, 4),
                 "TFLOPs": round(2.0 * layer_weights * ntok / (dms * 1e-3) / 1e12, 1),
                 "seedlm_over_dense_time": round(ms / dms, 3)}
        del Ws
    out = {
        "metric": GEMM_METRIC,
        "value": ntok / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: q,k,v,o,gate,up,down decode-GEMM, {ntok} tokens, "
                         f"SeedLM C={cfg.C} P={cfg.P} K={cfg.K}, fp16 X/Y"),
            "tokens": ntok,
        },
        "TFLOPs": round(2.0 * layer_weights * ntok / (ms * 1e-3) / 1e12, 1),
        "kernel_ms_per_launch": round(kern_s * 1e3, 3),
        "kernel_shape": [bm.rows, bm.cols, ntok],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": F16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / F16_MFMA_PEAK_TFLOPS, 4),
            "traffic": None,
        },
        "dense_fp16_baseline": dense,
        "decoded_path": {
            "entry": "seedlm_gemm_decoded (exact fp16 rebuild into a workspace, then hipBLASLt)",
            "ms_per_step": round(dec_ms, 4),
            "tokens_per_s": ntok / (dec_ms * 1e-3),
            "TFLOPs": round(2.0 * layer_weights * ntok / (dec_ms * 1e-3) / 1e12, 1),
            "over_dense_time": (round(dec_ms / dense["ms_per_step"], 3) if dense else None),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_gemm_baseline(cfg, ntok, args.cpu_seconds)
    print(json.dumps(out), flush=True)


# (C, P, K, Q): block length, latent dimension, seed width, coefficient width
SWEEP_FORMATS = [(c, p, 16, 4) for c, p in
                 [(6, 1), (7, 2), (8, 3), (9, 4), (10, 5), (11, 6), (12, 7),   # 4 bits/weight
                  (8, 1), (9, 1), (10, 2), (11, 3), (12, 4),                    # <= 3 bits/weight
                  (8, 2), (8, 4)]]                                              # C = 8 curve
SWEEP_FORMATS += [(7, 3, 12, 4), (9, 3, 20, 4),      # 4 bits/weight, other seed widths
                  (8, 2, 12, 4), (12, 3, 20, 4),     # 3 bits/weight, other seed widths
                  (8, 4, 16, 3), (10, 3, 16, 3)]     # 3-bit coefficients


def sweep_main(args):
    """Relative reconstruction MSE of N(0,1) blocks (bf16) for each supported
    (C, P, K, Q), with every block searched over all 2^K - 1 seeds on the GPU
    and sampled blocks re-scored and re-searched by the oracle."""
    import torch

    import prng_seeded_decode_amd as S
    from oracle import seedlm_oracle as O
    from workloads import bf16_to_float64, gen_bf16_weights

    dev = torch.device("cuda:0")
    rows, nb = 2048, 256
    table, total_pairs, total_s = [], 0, 0.0
    rng = np.random.default_rng(99)
    t_oracle = 0.0
    for C, P, K, Q in SWEEP_FORMATS:
        print(f"# sweep C={C} P={P} K={K} Q={Q}", file=sys.stderr, flush=True)
        nseed = (1 << K) - 1
        bits = gen_bf16_weights(50, 100 * C + P, rows, nb * C)
        W = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        enc = S.SeedLMEncoder(C, P, K, Q)
        outs = S.seedlm_encode(enc, W)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        S.seedlm_encode(enc, W, *outs)
        b.record()
        b.synchronize()
        t = a.elapsed_time(b) * 1e-3
        sd, cf, ex, err = (o.cpu().numpy() for o in outs)
        Wb = bf16_to_float64(bits).reshape(-1, C)
        wn = np.sum(Wb ** 2, axis=1)
        err = err.reshape(-1).astype(np.float64)
        rel = float(err.sum() / wn.sum())
        # oracle: re-score the GPU's records in float64 and re-search sampled blocks
        pick = rng.choice(Wb.shape[0], size=4, replace=False)
        t0 = time.perf_counter()
        sd = sd.view(np.uint16 if K <= 16 else np.uint32)
        dec = O.decode_rows(sd.reshape(-1, 1)[pick], cf.reshape(-1, 1, P)[pick],
                            ex.reshape(-1, 1)[pick], C, C, P, K=K)
        e64 = np.sum((Wb[pick] - dec) ** 2, axis=1)
        _, _, _, _, eo = O.encode_exhaustive(Wb[pick], C, P, K=K, Q=Q)
        t_oracle += time.perf_counter() - t0
        nblk = Wb.shape[0]
        table.append({
            "C": C, "P": P, "K": K, "Q": Q,
            "bits_per_weight": round((K + Q * P + 4) / C, 4),
            "rel_mse": round(rel, 6),
            "snr_db": round(-10 * np.log10(rel), 3),
            "gpu_ms": round(t * 1e3, 3),
            "pairs_per_s": nblk * nseed / t,
            "oracle_max_score_gap_over_wn": float(np.max(np.abs(e64 - eo.reshape(-1)) / wn[pick])),
        })
        total_pairs += nblk * nseed
        total_s += t
        enc.destroy()
        del W, outs
    best4 = min((r for r in table if r["bits_per_weight"] <= 4.0), key=lambda r: r["rel_mse"])
    best3 = min((r for r in table if r["bits_per_weight"] <= 3.0), key=lambda r: r["rel_mse"])
    out = {
        "metric": "seed-search design-space sweep: block-seed pairs/s over all formats",
        "value": total_pairs / total_s,
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 1,
        "ms_per_step": round(total_s * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{len(table)} (C, P, K, Q) formats, each on {rows}x{nb}C "
                                f"N(0,1) bf16 weights, every block against all 2^K - 1 seeds")},
        "best_4bit": {k: best4[k] for k in ("C", "P", "K", "Q", "rel_mse")},
        "best_3bit": {k: best3[k] for k in ("C", "P", "K", "Q", "rel_mse")},
        "sweep": table,
        "oracle_seconds": round(t_oracle, 2),
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse_args()
    if args.warmup is None:
        args.warmup = 3 if args.encode else 20
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU per process only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.encode:
        encode_main(args)
        return
    if args.gemm:
        gemm_main(args)
        return
    if args.sweep:
        sweep_main(args)
        return

    import torch

    import prng_seeded_decode_amd as S
    from workloads import CONFIGS, gen_records, gen_x

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    ydt = torch.float16 if cfg.x_dtype == "f16" else torch.float32
    xdt = ydt
    batch = args.batch

    # ---- pack the layer (copies for rotation) ----
    if args.copies <= 0:
        # Enough copies that consecutive steps never find their weights in the
        # 256 MB MALL (above 600 MB in all), between 2 and 64.
        nbytes = sum(mat.rows * -(-mat.cols // cfg.C) * (4.5 if cfg.C == 12 else 4.0)
                     for mat in cfg.matrices)
        args.copies = int(min(64, max(2, -(-600e6 // nbytes))))
    mats = []  # per matrix: dict
    for mid, mat in enumerate(cfg.matrices):
        s, c, e = gen_records(cfg.config_id, mid, mat.rows, mat.cols, cfg.C, cfg.P)
        copies = [S.seedlm_pack(s, c, e, mat.rows, mat.cols, cfg.C, cfg.P, cfg.K)
                  for _ in range(args.copies)]
        del s, c, e
        x = torch.from_numpy(gen_x(cfg.config_id, mid, batch, mat.cols, cfg.x_dtype)).to(dev)
        y = torch.empty((batch, mat.rows), dtype=ydt, device=dev)
        mats.append({"mat": mat, "copies": copies, "x": x, "y": y,
                     "bytes": copies[0].compressed_bytes})
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        # A plain copy of known size: its counter readings scale the kernel's.
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    xs_all = [d["x"] for d in mats]
    ys_all = [d["y"] for d in mats]

    # The step's seedlm_gemv_many call per rotated copy, marshalled once, so the
    # host issues a step with one C call (small layers are otherwise host-bound).
    calls = [S.GemvManyCall([d["copies"][k] for d in mats], xs_all, ys_all, batch=batch,
                            stream=stream)
             for k in range(args.copies)]

    def eager_step(k, phase="all", st=None):
        # One step = the whole layer through seedlm_gemv_many (grouped launch);
        # --variant != 0 times per-matrix seedlm_gemv calls of that variant.
        if args.variant == 0:
            calls[k % args.copies](stream=st, phase=phase)
            return
        st = stream if st is None else st
        for d in mats:
            S.seedlm_gemv(d["copies"][k % args.copies], d["x"], d["y"], batch=batch,
                          stream=st, variant=args.variant)

    graphs = []
    if args.graph:
        # Capture one step per rotated copy on a stream of our own; an eager
        # step on it first gives it its scratch (no allocation while capturing).
        cs = torch.cuda.Stream()
        for k in range(args.copies):
            eager_step(k, st=cs)
        torch.cuda.synchronize()
        for k in range(args.copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cs):
                eager_step(k, st=cs)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(k, phase="all"):
        if graphs and phase == "all":
            graphs[k % args.copies].replay()
        else:
            eager_step(k, phase)

    # ---- clock settle, then whole-step timing ----
    # The collector stays off while launches are timed: a collection pause in the
    # host loop could otherwise leave the GPU idle inside a timed interval.
    import gc

    def settle(step_fn):
        """Run step_fn for args.settle_ms of wall-clock time (the part needs tens
        of milliseconds of load to reach its steady clocks); returns the count."""
        n, t0 = 0, time.perf_counter()
        while True:
            for _ in range(10):
                step_fn(n)
                n += 1
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= args.settle_ms:
                return n

    gc.disable()
    for k in range(args.warmup):
        run_step(k)
    torch.cuda.synchronize()
    settle_steps = settle(run_step)
    # The timed loop: events bracket the K steps (the step time).  The dominant
    # kernel's time comes from the same K steps run again right behind them, with
    # no pause in between (the GPU never idles, so clocks stay where the timed
    # loop left them): there every step's fused decode-GEMV launch records its own
    # start and end (seedlm_bench_time_next_call: the events ride on the kernel
    # dispatch, so they hold the kernel's execution and not the launch gap before
    # it).  The events are not taken inside the timed loop itself because they
    # slow the step: interleaved runs measured 117.7-120.1 us per Llama-3-70B step
    # with them against 111.2-114.4 us without, and 48.4-49.7 against 44.2-44.3 us
    # for the Llama-3-8B 3-bit layer.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    timed_kernel = args.variant == 0 and not graphs
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps if timed_kernel else 0)]
    for a, b in kev:  # torch creates an event at its first record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    import ctypes

    time_next = S.lib().seedlm_bench_time_next_call
    kev_ptr = [(ctypes.c_void_p(a.cuda_event), ctypes.c_void_p(b.cuda_event)) for a, b in kev]
    ev0.record(stream)
    for k in range(args.steps):
        run_step(k)
    ev1.record(stream)
    if timed_kernel:
        for k in range(args.steps):
            time_next(*kev_ptr[k])
            run_step(k)
    # A third pass right behind: the same steps' main launches alone, back to back
    # between two events, so that their mean holds the kernel and the short gap
    # between dispatches but no per-launch event work (a cross-check of the
    # per-launch events, which read a few percent above a kernel trace).
    bb0 = torch.cuda.Event(enable_timing=True)
    bb1 = torch.cuda.Event(enable_timing=True)
    if timed_kernel:
        bb0.record(stream)
        for k in range(args.steps):
            run_step(k, phase="begin")
        bb1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kern_ms = [a.elapsed_time(b) for a, b in kev]
    back_to_back_us = (round(bb0.elapsed_time(bb1) / args.steps * 1e3, 2)
                       if timed_kernel else None)
    # The dominant kernel is part of every step, so its mean time must not exceed
    # the step's; the line reports whether it holds (a profiler attached to the
    # process can inflate the kernel events of tiny steps).
    # A launch of a few microseconds can read longer than the step interval: its
    # events include dispatch work that back-to-back launches overlap.  The
    # roofline then uses the step time, which bounds the kernel's.
    kernel_within_step = (float(np.mean(kern_ms)) <= ms_per_step) if kern_ms else None
    gc.enable()

    # ---- per-matrix timing: one seedlm_gemv per matrix, events around each ----
    per = {d["mat"].name: [] for d in mats}
    evs = []
    for k in range(args.steps if args.per_matrix else 0):
        for d in mats:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            S.seedlm_gemv(d["copies"][k % args.copies], d["x"], d["y"], batch=batch,
                          stream=stream, variant=args.variant)
            b.record(stream)
            evs.append((d["mat"].name, a, b))
    torch.cuda.synchronize()
    for name, a, b in evs:
        per[name].append(a.elapsed_time(b))

    torch.cuda.synchronize()

    layer_weights = sum(d["mat"].rows * d["mat"].cols for d in mats)
    layer_bytes = sum(d["bytes"] for d in mats)
    act_bytes = sum(batch * (d["mat"].cols + d["mat"].rows) * (2 if ydt == torch.float16 else 4)
                    for d in mats)
    per_matrix = {}
    for d in mats if args.per_matrix else []:
        n = d["mat"].name
        t = float(np.median(per[n])) * 1e-3
        per_matrix[n] = {
            "shape": [d["mat"].rows, d["mat"].cols],
            "us": round(t * 1e6, 2),
            "compressed_GBps": round(d["bytes"] / t / 1e9, 1),
            "weights_per_s": d["mat"].rows * d["mat"].cols / t,
        }
    # Roofline of the dominant kernel (the fused decode-GEMV launch of a step):
    # algorithmic bytes = the layer's packed words (0.5 B per weight, padding
    # included) + the activations x it reads, over the launch's mean duration.
    x_bytes = sum(batch * d["mat"].cols * (2 if xdt == torch.float16 else 4) for d in mats)
    alg_bytes = layer_bytes + x_bytes
    if kern_ms and kernel_within_step:
        achieved = alg_bytes / (float(np.mean(kern_ms)) * 1e-3) / 1e9
    else:  # the step's launches together (per-matrix variants, launch-bound steps)
        achieved = alg_bytes / (ms_per_step * 1e-3) / 1e9
    t_step = ms_per_step * 1e-3
    traffic = (measured_traffic(args.config)
               if kern_ms and batch == 1 and args.variant == 0 else None)
    matrix_names = ",".join(mat.name for mat in cfg.matrices)

    # ---- fp16 baselines on the same shapes ----
    fp16 = None
    if not args.no_fp16:
        Ws = []
        for d in mats:
            r, ccol = d["mat"].rows, d["mat"].cols
            Ws.append([torch.randn(r, ccol, device=dev, dtype=torch.float16) for _ in range(2)])
        xs = [d["x"].half() for d in mats]
        ys = [torch.empty((batch, d["mat"].rows), dtype=torch.float16, device=dev) for d in mats]

        # the library baseline's arguments marshalled once, as for the SeedLM step
        import ctypes

        vp = ctypes.c_void_p
        own_args = [[(vp(Ws[i][k].data_ptr()), vp(xs[i].data_ptr()), vp(ys[i].data_ptr()),
                      d["mat"].rows, d["mat"].cols, batch, vp(stream.cuda_stream))
                     for i, d in enumerate(mats)] for k in range(2)]
        fp16_fn = S.lib().seedlm_fp16_gemv

        def fp16_step(k, own):
            if own:
                for a in own_args[k % 2]:
                    if fp16_fn(*a) != 0:
                        raise RuntimeError("seedlm_fp16_gemv failed")
                return
            for i in range(len(mats)):
                torch.nn.functional.linear(xs[i], Ws[i][k % 2], out=ys[i])

        res = {}
        gc.disable()
        for own, name in ((True, "own_fp16_gemv"), (False, "torch_linear_fp16")):
            for k in range(args.warmup):
                fp16_step(k, own)
            torch.cuda.synchronize()
            settle(lambda k, own=own: fp16_step(k, own))
            ev0.record(stream)
            for k in range(args.steps):
                fp16_step(k, own)
            ev1.record(stream)
            ev1.synchronize()
            res[name] = ev0.elapsed_time(ev1) / args.steps
        gc.enable()
        best = min(res.values())
        fp16 = {"ms_per_step": {k: round(v, 4) for k, v in res.items()},
                "fp16_GBps": round(sum(2 * r * c for r, c in ((d["mat"].rows, d["mat"].cols) for d in mats))
                                   / (best * 1e-3) / 1e9, 1),
                "speedup_vs_best_fp16": round(best / ms_per_step, 3)}
        del Ws

    # ---- measured streaming-read ceiling: a plain 16-byte-load read of a 2 GiB
    # buffer (8x the 256 MB MALL), the rate a bandwidth-bound kernel can approach
    ceiling = None
    if not args.no_read_ceiling:
        rb = torch.zeros(2 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(S.STREAM_READ_SINK, dtype=torch.int32, device=dev)
        for _ in range(3):
            S.seedlm_stream_read(rb, sink, stream=stream)
        torch.cuda.synchronize()
        rev = []
        for _ in range(10):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            S.seedlm_stream_read(rb, sink, stream=stream)
            b.record(stream)
            rev.append((a, b))
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) for a, b in rev])) * 1e-3
        ceiling = {"GBps": round(rb.numel() / t / 1e9, 1), "buffer_bytes": rb.numel(),
                   "kernel": "seedlm_stream_read: contiguous range per workgroup, 16-byte loads"}
        del rb, sink

    decode = None
    if args.decode:
        # seedlm_decode of the largest matrix into a dense fp32 W: reads the packed
        # words, writes 4 bytes per weight (HBM-write bound).
        big = max(mats, key=lambda d: d["mat"].rows * d["mat"].cols)
        W = torch.empty((big["mat"].rows, big["mat"].cols), dtype=torch.float32, device=dev)
        for k in range(3):
            S.seedlm_decode(big["copies"][k % args.copies], W, stream=stream)
        torch.cuda.synchronize()
        dev_ms = []
        for k in range(max(5, args.steps // 2)):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            S.seedlm_decode(big["copies"][k % args.copies], W, stream=stream)
            b.record(stream)
            dev_ms.append((a, b))
        torch.cuda.synchronize()
        t = float(np.mean([a.elapsed_time(b) for a, b in dev_ms])) * 1e-3
        moved = big["bytes"] + 4 * big["mat"].rows * big["mat"].cols
        decode = {"matrix": big["mat"].name, "shape": [big["mat"].rows, big["mat"].cols],
                  "us": round(t * 1e6, 2), "GBps_read_plus_write": round(moved / t / 1e9, 1),
                  "pct_hbm_peak": round(100 * moved / t / 1e9 / HBM_PEAK_GBPS, 2)}
        del W

    out = {
        "metric": METRIC,
        "value": layer_weights / t_step,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic of the path: fp32 table lookups and sums at batch 1
        # (and for fp32 activations); fp16 MFMA operands with fp32 accumulation
        # for an fp16 batch > 1
        "dtype": "f16" if (batch > 1 and cfg.x_dtype == "f16") else "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {matrix_names} fused decode-GEMV, "
                         f"SeedLM C={cfg.C} P={cfg.P} K={cfg.K}, batch {batch}, "
                         f"x/y {cfg.x_dtype}"),
            "batch": batch,
            "io_dtype": cfg.x_dtype,
            "compressed_bytes_per_step": layer_bytes,
            "weights_per_step": layer_weights,
            "rotated_copies": args.copies,
            "variant": args.variant,
            "graph": bool(graphs),
        },
        "clock_settle": {"ms": args.settle_ms, "steps": settle_steps},
        "compressed_GBps": round(layer_bytes / t_step / 1e9, 1),
        "pct_hbm_peak": round(100 * layer_bytes / t_step / 1e9 / HBM_PEAK_GBPS, 2),
        "activation_bytes_per_step": act_bytes,
        "per_matrix": per_matrix or None,
        "kernel_us_per_launch": round(float(np.mean(kern_ms)) * 1e3, 2) if kern_ms else None,
        "kernel_us_median": round(float(np.median(kern_ms)) * 1e3, 2) if kern_ms else None,
        "kernel_us_back_to_back": back_to_back_us,
        "kernel_timing": ("HIP events recorded by the fused decode-GEMV launch of each step "
                          "itself (hipExtLaunchKernel start/stop events on the launch stream), "
                          "in a second pass of the same steps queued right behind the timed "
                          "loop" + ("" if kernel_within_step else
                                    "; the roofline uses the step time, which is shorter")
                          if kern_ms else "the step's launches together"),
        "kernel_within_step": kernel_within_step,
        "kernel_alg_bytes_per_launch": int(alg_bytes),
        "roofline": {
            "bound": "hbm",
            "achieved": round(float(achieved), 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(float(achieved) / HBM_PEAK_GBPS, 4),
            # counters were taken at batch 1 with the default kernel choice
            "traffic": traffic,
        },
        "traffic_source": (f"stored: FETCH_SIZE + WRITE_SIZE per launch from two rocprofv3 "
                           f"--pmc runs of this workload, scaled by a plain copy kernel's "
                           f"reading ({os.path.relpath(TRAFFIC_FILES[args.config][0], ROOT)}); "
                           f"valid while the kernel sources hash as they did then"
                           if traffic is not None else None),
        "fp16_baseline": fp16,
        "read_ceiling": ceiling,
        "pct_read_ceiling": (round(100 * float(achieved) / ceiling["GBps"], 2) if ceiling else None),
    }
    if decode:
        out["decode"] = decode
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
