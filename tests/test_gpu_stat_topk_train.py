"""Training side of the statistical top-k on the GPU against the fp64 oracle:
the Huber-smoothed forward (dense y, theta) and its gradient.  The smoothed
operator is continuous in theta with a continuous slope, so no entry is
decided differently by the two sides: every value is held to the fp32 bar
(rel 1e-4 per row, normwise)."""
import numpy as np
import pytest
import torch

import attention_spark_ffn_amd as sf
import oracle
import synth
from parity import rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check(x, dy, k, delta, rows_to_check=None, x_dev=None, dy_dev=None):
    xt = torch.from_numpy(x).to(DEV) if x_dev is None else x_dev
    gt = torch.from_numpy(dy).to(DEV) if dy_dev is None else dy_dev
    y, theta = sf.stat_topk_huber(xt, k, delta)
    dx = sf.stat_topk_huber_backward(xt, gt, k, delta)
    torch.cuda.synchronize()
    sel = np.arange(x.shape[0]) if rows_to_check is None else np.asarray(rows_to_check)
    ref = oracle.stat_topk_huber(x[sel], k, delta)
    rdx = oracle.stat_topk_huber_backward(x[sel], dy[sel], k, delta)
    y, theta, dx = y.cpu().numpy(), theta.cpu().numpy(), dx.cpu().numpy()
    sd = x[sel].astype(np.float64).std(1)
    for j, row in enumerate(sel):
        assert abs(theta[row] - ref["theta"][j]) <= 2e-6 * (abs(ref["theta"][j]) + sd[j]), row
        assert rel_err(y[row], ref["y"][j]) <= 1e-4, (row, rel_err(y[row], ref["y"][j]))
        assert rel_err(dx[row], rdx[j]) <= 1e-4, (row, rel_err(dx[row], rdx[j]))
    return y, dx


@pytest.mark.parametrize("d,k,delta", [(1024, 82, 0.05), (9216, 737, 0.01), (777, 60, 0.2), (33, 5, 0.5),
                                       (2, 1, 0.1), (16384, 1000, 0.02), (20000, 1500, 0.01), (65536, 4000, 0.005),
                                       (4100, 300, 1e-4), (6000, 3000, 0.3)])
def test_huber_shapes(d, k, delta):
    x = synth.stat_rows(d + k + 1, 64, d)
    dy = np.random.default_rng(d).standard_normal(x.shape).astype(np.float32)
    check(x, dy, k, delta)


def test_huber_config_rows():
    """The statistical top-k workload's shape (65536 x 9216, k = 737) for the
    training pass: all rows on the GPU, 1000 sampled rows against the oracle,
    and on every row the gradient's sum (zero: a common shift of the row leaves
    y unchanged) and y >= 0."""
    d, k, rows, delta = 9216, 737, 65536, 0.01
    x = synth.stat_rows(0, rows, d)
    dy = np.random.default_rng(5).standard_normal(x.shape).astype(np.float32)
    xt, gt = torch.from_numpy(x).to(DEV), torch.from_numpy(dy).to(DEV)
    sample = np.sort(np.random.default_rng(2).choice(rows, 1000, replace=False))
    check(x, dy, k, delta, rows_to_check=sample, x_dev=xt, dy_dev=gt)
    y, _ = sf.stat_topk_huber(xt, k, delta)
    dx = sf.stat_topk_huber_backward(xt, gt, k, delta)
    assert bool((y >= 0).all())
    s = dx.double().sum(1).abs()
    scale = dx.double().abs().sum(1)
    assert bool((s <= 1e-5 * scale + 1e-30).all()), float((s / scale).max())


def test_huber_edge_cases():
    # constant rows: y = 0, dx = 0; an empty batch is a no-op
    x = np.full((4, 300), -1.25, np.float32)
    y, dx = check(x, np.ones_like(x), 10, 0.1)
    assert np.all(y == 0) and np.all(dx == 0)
    e = torch.empty((0, 300), device=DEV)
    assert sf.stat_topk_huber(e, 10, 0.1)[0].numel() == 0
    # a base pointer that is not 16-byte aligned (the scalar path)
    big = torch.from_numpy(synth.stat_rows(8, 1, 64 * 1024 + 1)).to(DEV)
    xt = big[0, 1:].view(64, 1024)
    gt = torch.from_numpy(np.random.default_rng(1).standard_normal((64, 1024)).astype(np.float32)).to(DEV)
    check(xt.cpu().numpy(), gt.cpu().numpy(), 80, 0.1, x_dev=xt, dy_dev=gt)
    # bad arguments are rejected before any launch
    with pytest.raises(RuntimeError):
        sf.stat_topk_huber(torch.zeros((2, 10), device=DEV), 10, 0.1)
    with pytest.raises(RuntimeError):
        sf.stat_topk_huber(torch.zeros((2, 10), device=DEV), 3, 0.0)


def test_huber_autograd_function_and_determinism():
    """The autograd function runs both kernels; its gradient matches the oracle,
    and repeated calls are bit-identical."""
    x = synth.stat_rows(31, 128, 9216)
    dy = np.random.default_rng(31).standard_normal(x.shape).astype(np.float32)
    xt = torch.from_numpy(x).to(DEV).requires_grad_(True)
    y = sf.StatTopkHuber.apply(xt, 737, 0.01)
    (y * torch.from_numpy(dy).to(DEV)).sum().backward()
    g1 = xt.grad.clone()
    ref = oracle.stat_topk_huber_backward(x, dy, 737, 0.01)
    for r in range(x.shape[0]):
        assert rel_err(g1[r].cpu().numpy(), ref[r]) <= 1e-4, r
    xt.grad = None
    y2 = sf.StatTopkHuber.apply(xt, 737, 0.01)
    (y2 * torch.from_numpy(dy).to(DEV)).sum().backward()
    assert torch.equal(y, y2) and torch.equal(xt.grad, g1)


def test_huber_small_delta_is_the_soft_threshold():
    """delta -> 0: the smoothed forward becomes the statistical top-k's
    soft-threshold values, listed by the forward kernel (within delta / 2)."""
    x = synth.stat_rows(17, 256, 9216)
    xt = torch.from_numpy(x).to(DEV)
    y, th = sf.stat_topk_huber(xt, 737, 1e-6)
    vals, idx, counts, th2 = sf.stat_topk(xt, 737)
    torch.cuda.synchronize()
    sd = torch.from_numpy(x.astype(np.float64).std(1)).to(DEV)
    dth = (th.double() - th2.double()).abs()
    assert bool((dth <= 1e-6 * (th2.double().abs() + sd)).all())
    dense = torch.zeros_like(y)
    for r in range(x.shape[0]):
        n = int(counts[r])
        dense[r, idx[r, :n].long()] = vals[r, :n]
    # delta / 2, the two thresholds' difference, and the rounding of x - theta
    assert float((y - dense).abs().max()) <= 1e-6 / 2 + float(dth.max()) + 1e-6
