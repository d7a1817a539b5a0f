"""Pins of the fp64 oracle to facts fixed independently of it.

Each check raises AssertionError on failure.  They are run against the real
oracle (tests/test_oracle_pins.py) and against copies of oracle.c with planted
mistakes (tests/test_oracle_mutants.py), where at least one must fail.

Independent references used here: scipy's ndtri (Cephes algorithm, not
AS 241) and Python's NormalDist for the quantile; numpy mean/std/matmul/
argsort; torch fp64 gelu(tanh), softmax and softplus; scipy's Student-t
survival function; closed forms (quantile grid, power-of-two scaling,
constant rows); and the O(sqrt(log d / d)) count concentration the pages state
for Gaussian scores.
"""
from __future__ import annotations

import math
import os
from statistics import NormalDist

import numpy as np
import torch
from scipy import stats
from scipy.special import ndtri

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers
def np_stat_topk(x: np.ndarray, k: int):
    """Statistical top-k of one row with numpy's population mean/std and scipy's ndtri."""
    x = np.asarray(x, np.float64)
    th = x.mean() + x.std() * ndtri(1.0 - k / x.size)
    return th, np.nonzero(x > th)[0]


def gelu_t(v: np.ndarray) -> np.ndarray:
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(v, np.float64)), approximate="tanh").numpy()


def softplus_t(v: np.ndarray) -> np.ndarray:
    return torch.nn.functional.softplus(torch.from_numpy(np.asarray(v, np.float64))).numpy()


def dense_masked_ffn(q, k1t, k2t, v, r, k):
    """The Spark FFN written densely: every neuron is computed and the
    unselected ones are multiplied by GELU(0) = 0.  No index list, no gather."""
    q = np.asarray(q, np.float64)
    W1, W2, V = (np.asarray(a, np.float64) for a in (k1t, k2t, v))
    h = W1 @ q[:r]
    th, S = np_stat_topk(h, k)
    a = gelu_t(np.maximum(h - th, 0.0))
    g = W2 @ q[r:]
    return V.T @ (a * g), h, th, S


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- P1 quantile
def check_quantile():
    ps = np.concatenate([np.linspace(1e-6, 1 - 1e-6, 1001), np.logspace(-300, -1, 61),
                         1 - np.logspace(-15, -1, 29), [0.5, 0.425, 0.075, 0.925, 1 - 737 / 9216]])
    nd = NormalDist()
    for p in ps:
        a, b = oracle.norm_quantile(p), float(ndtri(p))
        assert abs(a - b) <= 4e-15 * max(1.0, abs(b)), (p, a, b)
        if 1e-300 < p < 1 - 1e-15:
            c = nd.inv_cdf(p)
            assert abs(a - c) <= 4e-15 * max(1.0, abs(c)), (p, a, c)
    assert oracle.norm_quantile(0.5) == 0.0
    for d, k in [(9216, 737), (1024, 82), (4096, 256), (32768, 256)]:
        assert abs(oracle.threshold_z(k, d) - ndtri(1 - k / d)) < 4e-15


# ---------------------------------------------------------------- P2 closed form
def check_threshold_closed_form():
    g = np.random.default_rng(7)
    x = (g.standard_normal((32, 777)) * g.uniform(0.1, 3, (32, 1)) + g.uniform(-2, 2, (32, 1))).astype(np.float32)
    for k in (1, 62, 388, 700, 776):
        res = oracle.stat_topk(x, k)
        xd = x.astype(np.float64)
        mu, sd = xd.mean(axis=1), xd.std(axis=1)
        assert np.allclose(res["mean"], mu, rtol=1e-13, atol=1e-13)
        assert np.allclose(res["std"], sd, rtol=1e-13, atol=0)
        th = mu + sd * ndtri(1 - k / 777)
        assert np.allclose(res["theta"], th, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- P3 / R9 special cases
def check_special_rows():
    g = np.random.default_rng(3)
    x = g.standard_normal((8, 1000)).astype(np.float32)
    res = oracle.stat_topk(x, 500)  # k = d/2: z = 0, theta = mean
    assert np.array_equal(res["theta"], res["mean"])
    for i in range(8):
        assert res["counts"][i] == int((x[i].astype(np.float64) > res["mean"][i]).sum())
    c = np.full((3, 64), 0.75, np.float32)  # constant row: std 0, theta = mean, nothing strictly above
    res = oracle.stat_topk(c, 5)
    assert np.all(res["counts"] == 0) and np.all(res["theta"] == 0.75)


# ---------------------------------------------------------------- P4 worked example (golden)
def check_quantile_grid():
    rows = [list(map(int, l.split())) for l in open(os.path.join(GOLDEN, "quantile_grid.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) >= 4
    for d, k, expected in rows:
        x = ndtri((np.arange(d) + 0.5) / d).astype(np.float32)
        res = oracle.stat_topk(x[None, :], k)
        n = int(res["counts"][0])
        assert n == expected, (d, k, n)
        assert np.array_equal(res["idx"][0, :n], np.arange(d - k, d))
        gap = np.min(np.abs(x.astype(np.float64) - res["theta"][0])) / res["std"][0]
        assert gap > 1e-4, (d, k, gap)


# ---------------------------------------------------------------- P5 invariants
def check_invariants():
    x = synth.stat_rows(11, 64, 2000)
    k = 160
    res = oracle.stat_topk(x, k, cap=2000)
    for i in range(x.shape[0]):
        xd = x[i].astype(np.float64)
        n = int(res["counts"][i])
        S = res["idx"][i, :n]
        th = res["theta"][i]
        assert n == int((xd > th).sum())
        assert np.all(np.diff(S) > 0)
        assert np.array_equal(res["vals"][i, :n], xd[S] - th)
        assert np.all(res["vals"][i, :n] > 0)
        mask = np.zeros(xd.size, bool)
        mask[S] = True
        assert xd[mask].min() > th >= xd[~mask].max()
    # capacity: the first cap entries of the same ascending list, true count kept
    res2 = oracle.stat_topk(x, k, cap=50)
    assert np.array_equal(res2["counts"], res["counts"])
    assert np.array_equal(res2["idx"], res["idx"][:, :50])


# ---------------------------------------------------------------- P6 scale invariance
def check_scale_invariance():
    x = synth.stat_rows(5, 16, 3000)
    a = oracle.stat_topk(x, 240)
    for j in (-3, 5):
        b = oracle.stat_topk(x * np.float32(2.0 ** j), 240)
        assert np.array_equal(a["counts"], b["counts"]) and np.array_equal(a["idx"], b["idx"])
        assert np.array_equal(a["theta"] * 2.0 ** j, b["theta"])
        assert np.array_equal(a["vals"] * 2.0 ** j, b["vals"])


# ---------------------------------------------------------------- P7 Theorem 3.1
def check_theorem31(rows: int = 256):
    for d, k in [(9216, 737), (1024, 82)]:
        x = synth.stat_rows(17, rows, d, "gauss")
        c = oracle.stat_topk(x, k, cap=1)["counts"].astype(np.float64)
        bound = math.sqrt(math.log(d) / d)
        assert np.all(np.abs(c - k) / d <= bound), (d, k, c.min(), c.max())
        # binomial-like spread around k: the mean sits within 5 standard errors
        se = math.sqrt(d * (k / d) * (1 - k / d)) / math.sqrt(rows)
        assert abs(c.mean() - k) <= 5 * se + 0.5, (d, k, c.mean(), se)


# ---------------------------------------------------------------- P8 Student-t rows
def check_student_t(rows: int = 1500):
    d, k = 9216, 737
    x = synth.stat_rows(19, rows, d, "t4")
    c = oracle.stat_topk(x, k, cap=1)["counts"].astype(np.float64)
    z = ndtri(1 - k / d)
    expected = d * stats.t.sf(math.sqrt(2.0) * z, 4)  # population std of t(4) is sqrt(2)
    assert abs(c.mean() - expected) <= 10.0, (c.mean(), expected)


# ---------------------------------------------------------------- P9 sparse == dense-masked
FFN_SHAPES = [(16, 64, 8, 6), (24, 40, 12, 3), (32, 96, 20, 9), (256, 1024, 128, 82)]


def check_ffn_dense_masked(shapes=FFN_SHAPES, seeds=(0, 1, 2)):
    for (dm, dff, r, k) in shapes:
        for s in seeds:
            k1t, k2t, v = synth.ffn_layer(s, 0, dm, dff, r, "f32")
            q = synth.queries(s, 3, dm)
            res = oracle.spark_ffn(q, k1t, k2t, v, r, k)
            for t in range(3):
                y, h, th, S = dense_masked_ffn(q[t], k1t, k2t, v, r, k)
                n = int(res["counts"][t])
                assert n == S.size and np.array_equal(res["idx"][t, :n], S), (dm, dff, s, t)
                assert rel(res["h"][t], h) < 1e-13
                assert abs(res["theta"][t] - th) <= 1e-13 * (1 + abs(th))
                assert np.allclose(res["m"][t, :n], h[S] - th, rtol=1e-12, atol=1e-13)
                assert rel(res["y"][t], y) < 1e-12, (dm, dff, s, t, rel(res["y"][t], y))


def check_ffn_bf16_widening():
    dm, dff, r, k = 48, 128, 16, 10
    k1t, k2t, v = synth.ffn_layer(4, 0, dm, dff, r, "bf16")
    qb = synth.queries(4, 2, dm, "bf16")
    a = oracle.spark_ffn(qb, k1t, k2t, v, r, k)
    w = synth.bf16_bits_to_f32
    b = oracle.spark_ffn(w(qb), w(k1t), w(k2t), w(v), r, k)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["counts"], b["counts"])
    # and the widened values drive the same result as the dense numpy form
    y, _, _, _ = dense_masked_ffn(w(qb)[0], w(k1t), w(k2t), w(v), r, k)
    assert rel(a["y"][0], y) < 1e-12


# ---------------------------------------------------------------- P10 "top-k" = largest
def check_topk_is_largest():
    x = synth.stat_rows(23, 32, 4096)
    res = oracle.stat_topk(x, 300)
    for i in range(32):
        n = int(res["counts"][i])
        top = np.sort(np.argsort(-x[i].astype(np.float64), kind="stable")[:n])
        assert np.array_equal(res["idx"][i, :n], top)


# ---------------------------------------------------------------- P11 GELU / softplus
def check_activations():
    pts = np.array([0.0, 1e-8, 0.1, 0.5, 1.0, 1.4, 2.0, 3.7, 8.0, -0.5, -2.0, -6.0])
    gt = gelu_t(pts)
    for p, e in zip(pts, gt):
        assert abs(oracle.gelu_tanh(p) - e) <= 4e-16 * max(1.0, abs(e)), (p, oracle.gelu_tanh(p), e)
    assert oracle.gelu_tanh(0.0) == 0.0
    sp_pts = np.array([-60.0, -5.0, -0.3, 0.0, 0.3, 5.0, 60.0, 700.0])
    for p in sp_pts:
        e = float(np.logaddexp(0.0, p))
        assert abs(oracle.softplus(p) - e) <= 4e-16 * max(1.0, abs(e)), (p, oracle.softplus(p), e)
    assert np.allclose([oracle.softplus(p) for p in sp_pts], softplus_t(sp_pts), rtol=1e-15, atol=0)


# ---------------------------------------------------------------- P12 attention
def _attn_ref(q, k1, k2, v, k_attn, sigma2=True):
    """Masked softmax attention written with torch fp64 (dense over all tokens, mask from numpy stat top-k)."""
    Hq, hd = q.shape
    Hkv, n, r = k1.shape
    grp = Hq // Hkv
    out = np.zeros((Hq, hd))
    cnt = np.zeros(Hq, int)
    for h in range(Hq):
        g = h // grp
        s = k1[g] @ q[h, :r]
        S = np.arange(n) if n <= k_attn else np_stat_topk(s, k_attn)[1]
        cnt[h] = S.size
        mask = torch.full((n,), -math.inf, dtype=torch.float64)
        mask[torch.from_numpy(S)] = 0.0
        w = torch.softmax(torch.from_numpy(s) + mask, dim=0).numpy()
        u = softplus_t(k2[g] @ q[h, r:]) if sigma2 else np.ones(n)
        out[h] = (w * u) @ v[g]
    return out, cnt


def check_attention():
    w = synth.bf16_bits_to_f32
    for (Hq, Hkv, n, hd, r, ka) in [(4, 2, 100, 32, 16, 256), (4, 2, 64, 32, 16, 64), (8, 4, 1500, 64, 32, 128),
                                    (2, 1, 3000, 16, 8, 200)]:
        qb, k1b, k2b, vb = synth.attn_inputs(31, Hq, Hkv, n, hd, r, scale=0.5)
        res = oracle.spark_attn_decode(qb, k1b, k2b, vb, ka)
        ref, cnt = _attn_ref(w(qb).astype(np.float64), w(k1b).astype(np.float64), w(k2b).astype(np.float64),
                             w(vb).astype(np.float64), ka)
        assert np.array_equal(res["counts"], cnt), (n, res["counts"], cnt)
        assert rel(res["out"], ref) < 1e-12, (n, rel(res["out"], ref))
        # with the compute-key half of q zeroed, sigma2 is the constant softplus(0) = ln 2
        q0 = qb.copy()
        q0[:, r:] = 0
        res0 = oracle.spark_attn_decode(q0, k1b, k2b, vb, ka)
        ref0, _ = _attn_ref(w(q0).astype(np.float64), w(k1b).astype(np.float64), w(k2b).astype(np.float64),
                            w(vb).astype(np.float64), ka, sigma2=False)
        assert rel(res0["out"], math.log(2.0) * ref0) < 1e-12
    # GQA grouping: query head h reads KV head h // (Hq/Hkv)
    qb, k1b, k2b, vb = synth.attn_inputs(37, 4, 2, 600, 32, 16)
    a = oracle.spark_attn_decode(qb, k1b, k2b, vb, 64)
    k1c, vc = k1b.copy(), vb.copy()
    k1c[1] = k1c[1][::-1]
    vc[1] = 0
    b = oracle.spark_attn_decode(qb, k1c, k2b, vc, 64)
    assert np.array_equal(a["out"][:2], b["out"][:2]) and not np.allclose(a["out"][2:], b["out"][2:])
    # constant scores: std 0, nothing strictly above theta, zero output
    k1z = np.zeros_like(k1b)
    z = oracle.spark_attn_decode(qb, k1z, k2b, vb, 64)
    assert np.all(z["counts"] == 0) and np.all(z["out"] == 0)


# ---------------------------------------------------------------- P15 causal attention prefill
def check_attention_prefill():
    """Each position against the masked-softmax reference on its own prefix
    (dense rows while t + 1 <= k_attn, statistical top-k after), and causality:
    keys and values after position t never change its output."""
    w = synth.bf16_bits_to_f32
    for (T, Hq, Hkv, hd, r, ka) in [(40, 4, 2, 32, 16, 8), (24, 2, 1, 16, 8, 64)]:
        qb, k1b, k2b, vb = synth.attn_prefill_inputs(41, T, Hq, Hkv, hd, r, scale=0.5)
        res = oracle.spark_attn_prefill(qb, k1b, k2b, vb, ka)
        q64, k164, k264, v64 = (w(a).astype(np.float64) for a in (qb, k1b, k2b, vb))
        for t in range(T):
            ref, cnt = _attn_ref(q64[t], k164[:, :t + 1], k264[:, :t + 1], v64[:, :t + 1], ka)
            assert np.array_equal(res["counts"][t], cnt), (t, res["counts"][t], cnt)
            assert rel(res["out"][t], ref) < 1e-12, (t, rel(res["out"][t], ref))
            assert np.all(np.isnan(res["theta"][t])) == (t + 1 <= ka)
        t0 = T // 2
        k1c, k2c, vc = k1b.copy(), k2b.copy(), vb.copy()
        k1c[:, t0:] = k1c[:, t0:][:, ::-1]
        k2c[:, t0:] = 0
        vc[:, t0:] = vc[:, t0:][:, ::-1]
        b = oracle.spark_attn_prefill(qb, k1c, k2c, vc, ka)
        assert np.array_equal(res["out"][:t0], b["out"][:t0]) and not np.allclose(res["out"][t0:], b["out"][t0:])


# ---------------------------------------------------------------- P13 continuity at theta
def check_continuity():
    dm, dff, r, k = 16, 64, 8, 6
    k1t, k2t, v = synth.ffn_layer(9, 0, dm, dff, r, "f32")
    g = np.random.default_rng(1)
    crossings = 0
    for trial in range(400):
        q = g.standard_normal(dm).astype(np.float32)
        u = g.standard_normal(dm).astype(np.float32)
        delta = 1e-2
        a = oracle.spark_ffn(q[None], k1t, k2t, v, r, k)
        b = oracle.spark_ffn((q + np.float32(delta) * u)[None], k1t, k2t, v, r, k)
        if not np.array_equal(a["idx"], b["idx"]):
            crossings += 1
        dy = np.linalg.norm(a["y"] - b["y"])
        assert dy <= 10.0 * delta, (trial, dy)
    assert crossings >= 10, crossings  # the perturbations did move entries across theta


# ---------------------------------------------------------------- P14 decode chain
def check_decode_chain():
    dm, dff, r, k, L = 32, 128, 16, 10, 4
    layers = [synth.ffn_layer(2, l, dm, dff, r, "f32") for l in range(L)]
    q0 = synth.queries(2, 2, dm)
    eps = 1e-6
    res = oracle.decode_stack(q0, layers, r, k, eps, trace=True)
    for t in range(2):
        q = q0[t].astype(np.float64)
        for l in range(L):
            assert np.allclose(res["q_trace"][t, l], q, rtol=1e-12, atol=1e-14)
            y, _, _, S = dense_masked_ffn(q, *layers[l], r, k)
            assert res["counts"][t, l] == S.size
            q = y / np.sqrt(np.mean(y * y) + eps)
        assert rel(res["y"][t], y) < 1e-12


# ---------------------------------------------------------------- P9b the dense form the bench times
def check_ffn_dense_form():
    """The oracle's dense-masked layer (every neuron used, the unselected ones
    weighted by zero) equals the sparse layer bit for bit (adding exact zeros in
    the same ascending order changes no fp64 sum), and the numpy dense form."""
    for (dm, dff, r, k, wd) in ((16, 64, 8, 6, "f32"), (256, 1024, 128, 82, "f32"), (64, 200, 24, 15, "bf16")):
        lw = synth.ffn_layer(3, 0, dm, dff, r, wd)
        q = synth.queries(3, 3, dm)
        dense = oracle.spark_ffn_dense(q, *lw, r, k)
        sparse = oracle.spark_ffn(q, *lw, r, k)["y"]
        assert np.array_equal(dense, sparse), (dm, dff)
        w = [synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a for a in lw]
        for t in range(q.shape[0]):
            ref, _, _, _ = dense_masked_ffn(q[t], *w, r, k)
            assert rel(dense[t], ref) < 1e-12


# ---------------------------------------------------------------- P15 training side (Huber smoothing)
def check_huber_function():
    """h(u) against numerical integration of its derivative clamp(t / delta, 0, 1)
    (scipy quad), h' against central differences of h, continuity at the joints,
    and the distance to max{u, 0} (at most delta / 2, reached for u >= delta)."""
    from scipy.integrate import quad

    for delta in (1e-3, 0.25, 2.0):
        for u in np.concatenate([np.linspace(-2 * delta, 3 * delta, 41), [delta, 0.0, 5.0, -5.0]]):
            val, _ = quad(lambda t: min(max(t / delta, 0.0), 1.0), 0.0, max(u, 0.0), points=[delta], limit=200)
            assert abs(oracle.huber_relu(u, delta) - val) <= 1e-12 * max(1.0, abs(val)), (u, delta)
            e = 1e-7 * delta
            fd = (oracle.huber_relu(u + e, delta) - oracle.huber_relu(u - e, delta)) / (2 * e)
            assert abs(oracle.huber_relu_grad(u, delta) - fd) <= 1e-5, (u, delta, fd)
            assert 0.0 <= max(u, 0.0) - oracle.huber_relu(u, delta) <= delta / 2 + 1e-15
        e = 1e-9 * delta
        for j in (0.0, delta):  # value and slope continuous at the joints
            l, r = oracle.huber_relu(j - e, delta), oracle.huber_relu(j + e, delta)
            assert abs(l - r) <= 4 * e
            assert abs(oracle.huber_relu_grad(j - e, delta) - oracle.huber_relu_grad(j + e, delta)) < 1e-8
        assert oracle.huber_relu(10 * delta, delta) == 10 * delta - delta / 2


def _quantised_rows(seed, rows, d, scale=1.0):
    """Rows of multiples of 1/256 (exact in fp32, as are x +- 2^-12)."""
    g = np.random.default_rng(seed)
    return (np.round(g.standard_normal((rows, d)) * scale * 256) / 256).astype(np.float32)


def check_huber_limit():
    """delta -> 0: the smoothed forward is the soft-threshold max{x - theta, 0} of the
    statistical top-k (the separately pinned unsmoothed operator)."""
    x = synth.stat_rows(5, 16, 300)
    base = oracle.stat_topk(x, 25)
    for delta in (1e-6, 1e-9):
        res = oracle.stat_topk_huber(x, 25, delta)
        assert np.allclose(res["theta"], base["theta"], rtol=0, atol=1e-13)
        for r in range(x.shape[0]):
            dense = np.zeros(x.shape[1])
            n = base["counts"][r]
            dense[base["idx"][r, :n]] = base["vals"][r, :n]
            assert np.abs(res["y"][r] - dense).max() <= delta / 2 + 1e-13, r


def check_huber_gradient_fd():
    """The backward against central differences of L(x) = sum_i dy_i y_i(x), the
    forward evaluated by the oracle itself, on inputs that keep every x_i - theta
    away from the joints 0 and delta by more than the step."""
    eps, delta = 2.0 ** -12, 0.25
    checked = 0
    for seed in range(40):
        for d, k in ((8, 2), (33, 5), (64, 9)):
            x = _quantised_rows(seed + 100 * d, 1, d)[0]
            th = oracle.stat_topk_huber(x, k, delta)["theta"][0]
            u = x.astype(np.float64) - th
            if np.min(np.abs(u)) < 4e-3 or np.min(np.abs(u - delta)) < 4e-3:
                continue
            dy = np.random.default_rng(seed).standard_normal(d).astype(np.float32)
            grad = oracle.stat_topk_huber_backward(x, dy, k, delta)[0]

            def loss(xx):
                return float(np.dot(dy.astype(np.float64), oracle.stat_topk_huber(xx, k, delta)["y"][0]))

            fd = np.zeros(d)
            for j in range(d):
                xp, xm = x.copy(), x.copy()
                xp[j] += np.float32(eps)
                xm[j] -= np.float32(eps)
                fd[j] = (loss(xp) - loss(xm)) / (2 * eps)
            assert np.abs(grad - fd).max() <= 1e-5 * max(1.0, np.abs(fd).max()), (seed, d, np.abs(grad - fd).max())
            checked += 1
    assert checked >= 40, checked


def check_huber_autograd():
    """The backward against torch autograd (fp64) of the same forward."""
    for seed, (rows, d, k, delta) in enumerate(((4, 50, 6, 0.3), (3, 1000, 80, 0.05), (2, 9216, 737, 0.01))):
        x = synth.stat_rows(seed + 40, rows, d)
        dy = np.random.default_rng(seed).standard_normal((rows, d)).astype(np.float32)
        got = oracle.stat_topk_huber_backward(x, dy, k, delta)
        xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
        th = xt.mean(1, keepdim=True) + xt.std(1, correction=0, keepdim=True) * float(ndtri(1 - k / d))
        u = xt - th
        h = torch.where(u <= 0, torch.zeros_like(u), torch.where(u < delta, u * u / (2 * delta), u - delta / 2))
        (h * torch.from_numpy(dy.astype(np.float64))).sum().backward()
        ref = xt.grad.numpy()
        assert rel(got, ref) < 1e-10, (seed, rel(got, ref))


def check_huber_invariances():
    """A common shift of a row moves theta with it and leaves y unchanged, so the
    gradient sums to zero along each row; a constant row gives y = 0 and dx = 0."""
    x = _quantised_rows(7, 5, 200)
    dy = np.random.default_rng(3).standard_normal(x.shape).astype(np.float32)
    a = oracle.stat_topk_huber(x, 20, 0.1)
    b = oracle.stat_topk_huber(x + np.float32(3.0), 20, 0.1)
    assert np.abs(a["y"] - b["y"]).max() < 1e-12 and np.allclose(b["theta"] - a["theta"], 3.0, atol=1e-12)
    g = oracle.stat_topk_huber_backward(x, dy, 20, 0.1)
    assert np.abs(g.sum(1)).max() < 1e-12 * max(1.0, np.abs(g).max() * x.shape[1])
    assert np.abs(g).max() > 0
    c = np.full((2, 64), 1.5, np.float32)
    assert np.all(oracle.stat_topk_huber(c, 6, 0.1)["y"] == 0)
    assert np.all(oracle.stat_topk_huber_backward(c, np.ones_like(c), 6, 0.1) == 0)


ALL_CHECKS = [check_quantile, check_threshold_closed_form, check_special_rows, check_quantile_grid,
              check_invariants, check_scale_invariance, check_theorem31, check_student_t, check_ffn_dense_masked,
              check_ffn_bf16_widening, check_topk_is_largest, check_activations, check_attention,
              check_attention_prefill, check_continuity, check_decode_chain, check_ffn_dense_form,
              check_huber_function,
              check_huber_limit, check_huber_gradient_fd, check_huber_autograd, check_huber_invariances]
