"""Benchmark: Spark FFN decode on one MI355X.

Workload: a stack of 26 independent Spark FFN layers (d_model 2304, d_ff 9216,
r 1152, k 737 = 8% of d_ff), bf16 weights N(0, 1/fan_in), fp32 queries
N(0, 1), RMS normalisation between layers; batch 1.  One step = one token
through the whole stack (one spark_ffn_decode call with T = 1), inputs
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

value = tokens/s.  roofline: the decode kernel's algorithmic HBM bytes per
launch (K1 slab of every layer + the selected K2 and V rows, from the actual
per-layer counts, + the small vectors) / its average launch time measured with
HIP events on the launch stream.  cpu_baseline: the fp64 oracle on a bounded
sample of tokens on the host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

D_MODEL, D_FF, R, K, LAYERS = 2304, 9216, 1152, 737, 26
HBM_PEAK_GBS = 8000.0
METRIC = "Spark-FFN decode tokens/s (2304×9216, k=8%) + achieved HBM GB/s vs peak"


def algorithmic_bytes(counts: np.ndarray) -> float:
    """Bytes one token must move from HBM: per layer the whole K1 (r x d_ff bf16),
    the selected neurons' K2 rows ((d_model - r) bf16) and V rows (d_model bf16),
    plus the fp32 input and output vectors."""
    k1 = R * D_FF * 2
    per_sel = (D_MODEL - R) * 2 + D_MODEL * 2
    vecs = 2 * D_MODEL * 4
    return float(LAYERS * (k1 + vecs) + per_sel * counts.sum())


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("ffn_decode.hip", "exchange.hpp", "common.hpp"):
        with open(os.path.join(ROOT, "attention_spark_ffn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per decode launch from rocprofv3 counters (profiles/), only if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(layers_np, budget_s: float = 12.0):
    import oracle

    oracle.build()
    # a bounded sample sized from a timed batch of 8 tokens (about budget_s of CPU work)
    q = np.random.default_rng(12345).standard_normal((8, D_MODEL)).astype(np.float32)
    oracle.decode_stack(q[:1], layers_np, R, K, 1e-6)  # first call: thread start-up
    t0 = time.perf_counter()
    oracle.decode_stack(q, layers_np, R, K, 1e-6)
    one = (time.perf_counter() - t0) / 8
    n = int(max(8, min(1600, budget_s / max(one, 1e-4))))
    qs = np.random.default_rng(54321).standard_normal((n, D_MODEL)).astype(np.float32)
    t0 = time.perf_counter()
    oracle.decode_stack(qs, layers_np, R, K, 1e-6)
    dt = time.perf_counter() - t0
    out = {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
           "sample": f"{n} tokens through the same 26-layer stack (fp64 C oracle, OpenMP), {dt:.1f} s"}
    # the same oracle computing one layer densely (every neuron's K2 dot and V
    # row, unselected neurons weighted by zero) against the sparse layer on the
    # same tokens: the CPU sparse-vs-dense ratio
    nq = 32
    ql = np.random.default_rng(777).standard_normal((nq, D_MODEL)).astype(np.float32)
    t0 = time.perf_counter()
    oracle.spark_ffn(ql, *layers_np[0], R, K)
    t_sparse = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.spark_ffn_dense(ql, *layers_np[0], R, K)
    t_dense = time.perf_counter() - t0
    out["dense_masked"] = {"sparse_layer_tokens_per_s": nq / t_sparse, "dense_layer_tokens_per_s": nq / t_dense,
                           "sparse_over_dense_speedup": t_dense / t_sparse,
                           "sample": f"{nq} tokens through layer 0, sparse and dense-masked oracle"}
    return out


def _time_ms(torch, fn, reps=20, warm=3):
    """Median time of fn() in ms, HIP events on the current stream."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def _time_b2b_ms(torch, fns, n=20, reps=5, warm=2):
    """Per-call time in ms on the GPU timeline: n calls issued back to back
    (cycling through fns) between two HIP events, median over reps.  Unlike
    _time_ms, the host-side setup of each call (argument marshalling, the
    first launch) overlaps the GPU work of the previous calls."""
    for i in range(warm):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fns[i % len(fns)]()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / n)
    return float(np.median(ts))


MFMA_BF16_PEAK_TFLOPS = 2500.0


def read_ceiling(torch, sf, dev, gib: int = 4, reps: int = 10) -> float:
    """HBM read ceiling on this device: GB/s of the library's streaming-read
    probe over a buffer far larger than the caches (median of reps)."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, device=dev)
    ms = _time_ms(torch, lambda: sf.hbm_read_probe(buf, sink), reps=reps)
    del buf
    torch.cuda.empty_cache()
    return (gib << 30) / ms / 1e6


def _oracle_rate(fn, n_units: int, unit: str, sample: str) -> dict:
    """Time fn() (one call of the fp64 oracle over a bounded sample of n_units)."""
    import oracle

    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": n_units / dt, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{sample}, {dt:.3f} s"}


def batched_decode(torch, sf, layers, qs):
    """The same 26-layer stack decoded B tokens at a time (one K1 read per
    layer for the batch; K2 and V rows read once per union of the selected
    sets), for B in 1, 2, 4, 8.  Algorithmic bytes per call: per layer K1, the
    union's K2 and V rows, the fp32 input and output vectors of the batch."""
    res = {}
    for B in (1, 2, 4, 8):
        q = qs[:B].contiguous()
        ms = _time_ms(torch, lambda: sf.spark_ffn_decode_batched(q, layers, K, R, check=False), reps=20)
        # 20 calls back to back in one timed region (the launch of one call
        # overlaps the end of the previous one)
        ms20 = _time_ms(torch, lambda: [sf.spark_ffn_decode_batched(q, layers, K, R, check=False)
                                        for _ in range(20)], reps=3, warm=1) / 20
        _, tr = sf.spark_ffn_decode_batched(q, layers, K, R, trace=True)
        idx, cnt = tr["idx"].cpu().numpy(), tr["counts"].cpu().numpy()
        union = [len(set().union(*[set(idx[b, l, :cnt[b, l]].tolist()) for b in range(B)])) for l in range(LAYERS)]
        moved = sum(R * D_FF * 2 + u * ((D_MODEL - R) * 2 + D_MODEL * 2) + 2 * B * D_MODEL * 4 for u in union)
        res[str(B)] = {"ms_per_call": ms, "tokens_per_s": B / ms * 1e3,
                       "ms_per_call_back_to_back": ms20, "tokens_per_s_back_to_back": B / ms20 * 1e3,
                       "mean_union_per_layer": float(np.mean(union)),
                       "algorithmic_bytes_per_call": float(moved),
                       "roofline": {"bound": "hbm", "achieved": moved / ms / 1e6, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": moved / ms / 1e6 / HBM_PEAK_GBS}}
    return {"workload": "spark_ffn_decode_batched: the 26-layer decode stack, B tokens per call", "batch": res}


def extra_workloads(torch, sf, synth, dev, seed, with_cpu):
    """The other workloads of the hot path, each timed on its own, with its
    roofline and (with_cpu) the oracle timed on a bounded sample."""
    res = {}
    if with_cpu:
        import oracle

        oracle.build()
    # standalone statistical top-k: 65536 rows x 9216, k 737, Gaussian rows
    # x = mu + s * e with mu ~ U(-1,1), s ~ U(0.5,2) (generated on the GPU)
    g = torch.Generator(device=dev).manual_seed(seed)
    rows, d, k = 65536, 9216, 737
    x = torch.randn((rows, d), generator=g, device=dev)
    x.mul_(torch.rand((rows, 1), generator=g, device=dev) * 1.5 + 0.5)
    x.add_(torch.rand((rows, 1), generator=g, device=dev) * 2 - 1)
    cap = 2 * k
    vals = torch.empty((rows, cap), device=dev)
    idx = torch.empty((rows, cap), dtype=torch.int32, device=dev)
    counts = torch.empty(rows, dtype=torch.int32, device=dev)
    theta = torch.empty(rows, device=dev)
    L = sf.lib()
    st = lambda: L.stat_topk(sf._p(x), rows, d, d, k, sf._p(vals), sf._p(idx), cap, sf._p(counts), sf._p(theta),
                             sf._stream(dev))
    ms = _time_ms(torch, st)
    nsel = float(counts.double().sum().item())
    moved = rows * d * 4 + nsel * 8 + rows * 8
    res["stat_topk"] = {"workload": "65536 x 9216 fp32 rows, k 737", "ms": ms, "rows_per_s": rows / ms * 1e3,
                        "mean_count": nsel / rows,
                        "roofline": {"bound": "hbm", "achieved": moved / ms / 1e6, "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": moved / ms / 1e6 / HBM_PEAK_GBS}}
    if with_cpu:
        xs = synth.stat_rows(seed, 2000, d)
        res["stat_topk"]["cpu_baseline"] = _oracle_rate(lambda: oracle.stat_topk(xs, k, cap), 2000, "rows/s",
                                                        "2000 rows of 9216 (same recipe, host-generated)")
    del vals, idx
    torch.cuda.empty_cache()
    # training side on the same rows: Huber-smoothed forward (read x, write y)
    # and its gradient (read x and dy, write dx)
    delta = 0.01
    y = torch.empty_like(x)
    dyt = torch.randn((rows, d), generator=g, device=dev)
    ms_f = _time_ms(torch, lambda: sf.stat_topk_huber(x, k, delta), reps=10)
    ms_b = _time_ms(torch, lambda: sf.stat_topk_huber_backward(x, dyt, k, delta), reps=10)
    bf_, bb_ = rows * d * 8 + rows * 4, rows * d * 12
    res["stat_topk_train"] = {
        "workload": "Huber-smoothed statistical top-k, 65536 x 9216 fp32 rows, k 737, delta 0.01",
        "forward_ms": ms_f, "backward_ms": ms_b,
        "roofline_forward": {"bound": "hbm", "achieved": bf_ / ms_f / 1e6, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": bf_ / ms_f / 1e6 / HBM_PEAK_GBS},
        "roofline_backward": {"bound": "hbm", "achieved": bb_ / ms_b / 1e6, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": bb_ / ms_b / 1e6 / HBM_PEAK_GBS}}
    if with_cpu:
        xs = synth.stat_rows(seed, 500, d)
        gs = np.random.default_rng(seed).standard_normal(xs.shape).astype(np.float32)
        res["stat_topk_train"]["cpu_baseline"] = _oracle_rate(
            lambda: (oracle.stat_topk_huber(xs, k, delta), oracle.stat_topk_huber_backward(xs, gs, k, delta)), 500,
            "rows/s", "forward and gradient of 500 rows of 9216 (same recipe, host-generated)")
    del x, y, dyt
    torch.cuda.empty_cache()
    # prefill: 4096 tokens through one 2304 x 9216 layer, bf16
    T = 4096
    lw = synth.ffn_layer(seed, 0, D_MODEL, D_FF, R, "bf16")
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    layer = tuple(bf(a) for a in lw)
    Q = bf(synth.queries(seed, T, D_MODEL, "bf16"))
    ms_one = _time_ms(torch, lambda: sf.spark_ffn_prefill(Q, layer, K, R), reps=10)
    # back to back (each call writes ~420 MB of workspace, which turns the
    # memory-side cache over by itself)
    ms = _time_b2b_ms(torch, [lambda: sf.spark_ffn_prefill(Q, layer, K, R)], n=10, reps=5)
    _, ptr = sf.spark_ffn_prefill(Q, layer, K, R, trace=True, cap=1)
    nsel = float(ptr["counts"].double().sum().item())
    flops = 2.0 * T * R * D_FF
    # the method's own work: the dense predictor product, and per token the
    # selected neurons' K2 dots and V rows
    method = flops + 2.0 * nsel * ((D_MODEL - R) + D_MODEL)
    # the gathered form (only the selected K2 and V rows read, per token)
    gath_ms = _time_ms(torch, lambda: sf.spark_ffn_prefill(Q, layer, K, R, gathered=True), reps=5)
    # the predictor product alone (its own entry point), HIP events
    pred_ms_one = _time_ms(torch, lambda: sf.spark_ffn_prefill_scores(Q, layer, R), reps=50)
    pred_ms = _time_b2b_ms(torch, [lambda: sf.spark_ffn_prefill_scores(Q, layer, R)], n=20, reps=5)
    Qr = Q[:, :R].contiguous()
    K1 = layer[0].t().contiguous()  # [r][d_ff]
    ref_ms = _time_ms(torch, lambda: torch.mm(Qr, K1), reps=10)
    del Qr, K1
    # the products as run: dense on the matrix cores (unselected neurons
    # contribute exact zeros): scores, gated K2 values, and C V
    dense = 2.0 * T * D_FF * (R + (D_MODEL - R) + D_MODEL)
    res["prefill"] = {"workload": "4096 tokens, one 2304 x 9216 layer (r 1152, k 737), bf16", "ms": ms,
                      "ms_one_call": ms_one,
                      "tokens_per_s": T / ms * 1e3, "us_per_token": ms * 1e3 / T, "mean_selected": nsel / T,
                      "method_gflop": method / 1e9, "dense_products_gflop": dense / 1e9,
                      "roofline": {"bound": "mfma", "achieved": method / ms / 1e9, "peak": MFMA_BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": method / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
                                   "note": "the method's FLOPs (2 T r d_ff + 2 sum_t |S_t| (d_model - r + d_model)) "
                                           "over the whole call (calls back to back; 'ms_one_call' is one call "
                                           "timed alone, host-side setup included)"},
                      "predictor_gemm": {"us": pred_ms * 1e3, "us_one_call": pred_ms_one * 1e3, "gflop": flops / 1e9,
                                         "roofline": {"bound": "mfma", "achieved": flops / pred_ms / 1e9,
                                                      "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                                      "frac": flops / pred_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}},
                      "gathered": {"ms": gath_ms, "achieved_tflops": method / gath_ms / 1e9,
                                   "gathered_row_bytes": nsel * ((D_MODEL - R) * 2 + D_MODEL * 2),
                                   "note": "spark_ffn_prefill_gathered: per token only the selected K2 and V rows"},
                      "hipblaslt_predictor_gemm_ms": ref_ms,
                      "hipblaslt_predictor_tflops": flops / ref_ms / 1e9}
    if with_cpu:
        Qs = synth.queries(seed, 64, D_MODEL, "bf16")
        res["prefill"]["cpu_baseline"] = _oracle_rate(lambda: oracle.spark_ffn(Qs, *lw, R, K), 64, "tokens/s",
                                                      "64 tokens of the same layer")
    del Q, layer
    torch.cuda.empty_cache()
    # attention decode: 8 query heads / 4 KV heads, hd 256, r 128, k_attn 256
    att = {}
    for n in (4096, 32768):
        qb, k1b, k2b, vb = synth.attn_inputs(seed, 8, 4, n, 256, 128)
        args = [bf(a) for a in (qb, k1b, k2b, vb)]
        out, cnt, _, _ = sf.spark_attn_decode(*args, 256)
        # the operator alone through the C ABI: outputs preallocated, no list
        need = ctypes.c_size_t(0)
        L.spark_attn_workspace_size(8, 4, n, 256, 128, 256, ctypes.byref(need))
        ws = torch.zeros(need.value, dtype=torch.uint8, device=dev)  # zero-filled before its first use
        o2 = torch.empty((8, 256), device=dev)
        c2 = torch.empty(8, dtype=torch.int32, device=dev)
        mk = lambda kv: (lambda: L.spark_attn_decode(*[sf._p(a) for a in [args[0]] + kv], 8, 4, n, 256, 128, 256,
                                                     sf._p(o2), sf._p(c2), None, 0, None, sf._p(ws), need.value,
                                                     sf._stream(dev)))
        ms = _time_ms(torch, mk(args[1:]), reps=50)
        # back to back over copies of the cache whose total (> 512 MB) exceeds
        # the memory-side cache, so every call reads its cache from HBM
        cache_bytes = sum(a.numel() * 2 for a in args[1:])
        ncopy = max(2, -(-(512 << 20) // cache_bytes))
        copies = [[a.clone() for a in args[1:]] for _ in range(ncopy)]
        ms_b2b = _time_b2b_ms(torch, [mk(kv) for kv in copies], n=max(20, 2 * ncopy), reps=7)
        del copies
        torch.cuda.empty_cache()
        c = cnt.double().sum().item()
        moved = 4 * n * 128 * 2 + c * (128 + 256) * 2 + 8 * 256 * 2
        att[str(n)] = {"us": ms * 1e3, "us_back_to_back_cold": ms_b2b * 1e3, "cache_copies": ncopy,
                       "mean_attended": c / 8, "algorithmic_bytes": moved,
                       "roofline": {"bound": "hbm", "achieved": moved / ms_b2b / 1e6, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": moved / ms_b2b / 1e6 / HBM_PEAK_GBS,
                                    "note": "calls back to back over cache copies that do not fit the memory-side "
                                            "cache; 'us' is one call timed alone, host-side setup included"}}
        if with_cpu:
            att[str(n)]["cpu_baseline"] = _oracle_rate(lambda: oracle.spark_attn_decode(qb, k1b, k2b, vb, 256), 1,
                                                       "steps/s", f"one decode step at n_ctx {n}")
    res["attention_decode"] = att
    # causal attention prefill over a 4096-position prompt, same heads
    Tp = 4096
    qp, k1p, k2p, vp = synth.attn_prefill_inputs(seed, Tp, 8, 4, 256, 128)
    pargs = [bf(a) for a in (qp, k1p, k2p, vp)]
    po, pc, _, _ = sf.spark_attn_prefill(*pargs, 256)
    ms_one = _time_ms(torch, lambda: sf.spark_attn_prefill(*pargs, 256), reps=10)
    # back to back over copies of the inputs (> 512 MB in all: none is found in
    # the memory-side cache)
    in_bytes = sum(a.numel() * 2 for a in pargs)
    ncopy = max(2, -(-(512 << 20) // in_bytes))
    pcopies = [[a.clone() for a in pargs] for _ in range(ncopy)]
    ms = _time_b2b_ms(torch, [(lambda c=c: sf.spark_attn_prefill(*c, 256)) for c in pcopies], n=2 * ncopy, reps=3)
    del pcopies
    torch.cuda.empty_cache()
    flops = 2.0 * 8 * (Tp * (Tp + 1) / 2) * (128 + 128 + 256)  # causal S, gated K2 scores, W V
    res["attention_prefill"] = {
        "workload": "4096-position prompt, Hq 8, Hkv 4, hd 256, r 128, k_attn 256, causal", "ms": ms,
        "ms_one_call": ms_one, "input_copies": ncopy,
        "positions_per_s": Tp / ms * 1e3, "mean_attended": float(pc.double().mean().item()),
        "roofline": {"bound": "mfma", "achieved": flops / ms / 1e9, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS,
                     "note": "algorithmic causal products (scores, gate products, weights x V) over the "
                             "whole call (calls back to back over input copies; 'ms_one_call' is one call timed "
                             "alone, host-side setup included); the moments pass recomputes the scores and is "
                             "not counted"}}
    if with_cpu:
        qs, k1s, k2s, vs = synth.attn_prefill_inputs(seed, 512, 8, 4, 256, 128)
        res["attention_prefill"]["cpu_baseline"] = _oracle_rate(
            lambda: oracle.spark_attn_prefill(qs, k1s, k2s, vs, 256), 512, "positions/s",
            "a 512-position prompt with the same heads")
    del pargs, po, pc
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads (stat top-k, prefill, attention)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (scale for HBM byte counters)")
    ap.add_argument("--predictor-gemm", type=int, default=0, metavar="N",
                    help="only run the prefill predictor product (4096 x 1152 x 9216, bf16) N times "
                         "(for matrix-core counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the decode path is a single-GPU kernel); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_spark_ffn_amd as sf
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        a = torch.ones(1 << 28, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4, "launches": 5}))
        return
    if args.predictor_gemm:
        bf = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        layer = tuple(bf(x) for x in synth.ffn_layer(args.seed, 0, D_MODEL, D_FF, R, "bf16"))
        Q = bf(synth.queries(args.seed, 4096, D_MODEL, "bf16"))
        ms = _time_b2b_ms(torch, [lambda: sf.spark_ffn_prefill_scores(Q, layer, R)], n=args.predictor_gemm, reps=1)
        flops = 2.0 * 4096 * R * D_FF
        print(json.dumps({"predictor_gemm_us": ms * 1e3, "calls": args.predictor_gemm + 2, "gflop_per_call": flops / 1e9,
                          "tflops": flops / ms / 1e9}))
        return
    t0 = time.perf_counter()
    layers_np = synth.ffn_stack(args.seed, LAYERS, D_MODEL, D_FF, R, "bf16", workers=16)

    def to_dev(a):
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)

    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    nq = args.warmup + args.steps
    qs = torch.from_numpy(synth.queries(args.seed, nq, D_MODEL)).to(dev)
    print(f"# setup {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        sf.spark_ffn_decode(qs[i:i + 1], layers, K, R, check=False)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        sf.spark_ffn_decode(qs[args.warmup + i:args.warmup + i + 1], layers, K, R, check=False)
        ev[i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per_launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    failed = sf.decode_workspace_failed(device=dev)

    # actual per-layer selected counts of the timed tokens (same inputs,
    # deterministic), one launch per token like the timed launches
    counts = []
    for i in range(args.steps):
        _, tr = sf.spark_ffn_decode(qs[args.warmup + i:args.warmup + i + 1], layers, K, R, trace=True, cap=1)
        counts.append(tr["counts"])
    counts = torch.cat(counts).cpu().numpy()
    bytes_per_token = np.array([algorithmic_bytes(c) for c in counts])
    avg_launch_s = per_launch_ms.mean() / 1e3
    achieved_gbs = bytes_per_token.mean() / avg_launch_s / 1e9
    traffic = load_traffic()
    probe_gbs = read_ceiling(torch, sf, dev)

    out = {
        "metric": METRIC,
        "value": args.steps / (total_ms / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "spark_ffn_decode: 26 layers x (d_model 2304, d_ff 9216, r 1152, k 737), "
                               "bf16 weights, fp32 q, batch 1",
                   "weights_dtype": "bf16", "layers": LAYERS, "d_model": D_MODEL, "d_ff": D_FF, "r": R, "k": K,
                   "global_batch": 1},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "spark::decode_kernel<bf16>",
                     "algorithmic_bytes_per_launch": float(bytes_per_token.mean()),
                     "avg_launch_us": avg_launch_s * 1e6,
                     "median_us": float(np.median(per_launch_ms) * 1e3),
                     "p10_us": float(np.percentile(per_launch_ms, 10) * 1e3),
                     "p90_us": float(np.percentile(per_launch_ms, 90) * 1e3),
                     "probe_read_gbs": probe_gbs, "frac_of_probe": achieved_gbs / probe_gbs,
                     "mean_selected_per_layer": float(counts.mean())},
        "cpu_baseline": None,
        "kernel_failed": bool(failed),
    }
    if not args.no_extra:
        bd = batched_decode(torch, sf, layers, qs)
        del layers, qs
        torch.cuda.empty_cache()
        out["extra"] = extra_workloads(torch, sf, synth, dev, args.seed, not args.no_cpu)
        out["extra"]["decode_batched"] = bd
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(layers_np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
