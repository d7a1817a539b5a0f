"""Statistical top-k on the GPU against the fp64 oracle (standalone operator)."""
import numpy as np
import pytest
import torch
from scipy.special import ndtri

import attention_spark_ffn_amd as sf
import oracle
import synth
from parity import check_index_set, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_and_compare(x: np.ndarray, k: int, cap=None, rows_to_check=None, x_dev=None):
    xt = torch.from_numpy(x).to(DEV) if x_dev is None else x_dev
    vals, idx, counts, theta = sf.stat_topk(xt, k, cap)
    torch.cuda.synchronize()
    rows, d = x.shape
    cap = d if cap is None else cap
    sel = np.arange(rows) if rows_to_check is None else np.asarray(rows_to_check)
    ref = oracle.stat_topk(x[sel], k, cap=cap)
    vals, idx, counts, theta = (t.cpu().numpy() for t in (vals, idx, counts, theta))
    flips = 0
    for j, row in enumerate(sel):
        flips += check_index_set(idx[row], counts[row], cap, x[row], ref["theta"][j], ref["std"][j], f"row {row}")
        assert abs(theta[row] - ref["theta"][j]) <= 2e-6 * (abs(ref["theta"][j]) + ref["std"][j])
        # soft-threshold values on every entry both lists hold (tie-band flips
        # and truncation aside, that is the whole list)
        n, nr = min(int(counts[row]), cap), min(int(ref["counts"][j]), cap)
        common, ig, ir = np.intersect1d(idx[row, :n], ref["idx"][j, :nr], assume_unique=True, return_indices=True)
        assert common.size >= min(n, nr) - 3, (row, common.size, n, nr)
        if common.size:
            assert rel_err(vals[row, ig], ref["vals"][j, ir]) <= 1e-4, row
        assert np.all(vals[row, :n] > 0), row
    return flips, counts[sel], ref["counts"]


def check_all_rows_on_device(vals, idx, counts, cap):
    """Every row, on the device: min(count, cap) entries listed (the rest of the
    row untouched, -1), strictly ascending, each with a positive value."""
    valid = idx >= 0
    listed = valid.sum(1)
    assert torch.equal(listed, torch.clamp(counts.long(), max=cap)), "listed entries != min(count, cap)"
    # the listed entries are a prefix of the row
    assert torch.equal(valid, torch.arange(cap, device=idx.device)[None, :] < listed[:, None])
    assert bool(((idx[:, 1:] > idx[:, :-1]) | ~valid[:, 1:]).all()), "list not ascending"
    assert bool(((vals > 0) | ~valid).all()), "a listed value is not above the threshold"


@pytest.mark.parametrize("d,k", [(1024, 82), (9216, 737), (777, 60), (4100, 300), (33, 5), (2, 1), (16384, 1000),
                                 (20000, 1500), (65536, 4000), (1000, 999), (1000, 1), (6000, 3000)])
def test_stat_topk_shapes(d, k):
    x = synth.stat_rows(d + k, 96, d)
    run_and_compare(x, k)


@pytest.mark.parametrize("rows,d,k,cap", [(7001, 4096, 300, None), (6200, 8192, 650, 300), (6145, 9216, 737, 1474)])
def test_stat_topk_many_rows_every_row(rows, d, k, cap):
    """Thousands of rows whose length fills whole 16-byte lanes, every row
    against the oracle: row counts that are not a multiple of the resident
    workgroups, and a list capacity below the count (cap 300 at k 650)."""
    x = synth.stat_rows(rows + d, rows, d)
    _, got, want = run_and_compare(x, k, cap=cap)
    assert np.abs(got.astype(np.int64) - want.astype(np.int64)).max() <= 2


def test_stat_topk_config_rows_both_sets():
    """The statistical top-k workload (65536 x 9216, k = 737), Gaussian and
    Student-t rows: all rows on the GPU; 1500 sampled rows against the oracle
    (set, threshold, values); every row's list checked on the device against
    its count (length, order, positive values)."""
    d, k, rows = 9216, 737, 65536
    for kind in ("gauss", "t4"):
        x = synth.stat_rows(0, rows, d, kind)
        sample = np.random.default_rng(1).choice(rows, 1500, replace=False)
        xt = torch.from_numpy(x).to(DEV)
        run_and_compare(x, k, cap=2 * k, rows_to_check=np.sort(sample), x_dev=xt)
        vals, idx, counts, _ = sf.stat_topk(xt, k, 2 * k)
        check_all_rows_on_device(vals, idx, counts, 2 * k)
        del x, xt, vals, idx


def test_stat_topk_worked_example_grid():
    # quantile grid: exactly k selected, the top k grid points (golden fixture)
    for d, k in [(9216, 737), (1024, 82), (4096, 256), (32768, 256)]:
        x = ndtri((np.arange(d) + 0.5) / d).astype(np.float32)[None, :].repeat(3, axis=0)
        vals, idx, counts, theta = sf.stat_topk(torch.from_numpy(x).to(DEV), k)
        counts = counts.cpu().numpy()
        idx = idx.cpu().numpy()
        assert np.all(counts == k)
        assert np.array_equal(idx[0, :k], np.arange(d - k, d))


def test_stat_topk_edge_cases():
    # constant rows select nothing; an empty batch is a no-op
    x = np.full((5, 300), 2.5, np.float32)
    vals, idx, counts, theta = sf.stat_topk(torch.from_numpy(x).to(DEV), 10)
    assert np.all(counts.cpu().numpy() == 0)
    e = torch.empty((0, 300), device=DEV)
    _, _, c0, _ = sf.stat_topk(e, 10)
    assert c0.numel() == 0
    # capacity smaller than the count: true counts, first cap entries listed
    x = synth.stat_rows(3, 64, 2048)
    run_and_compare(x, 200, cap=50)
    # a strided view (row stride > d) and a base pointer that is not 16-byte aligned
    big = torch.from_numpy(synth.stat_rows(4, 64, 1030)).to(DEV)
    view = big[:, 1:1025]
    x = view.cpu().numpy()
    run_and_compare(np.ascontiguousarray(x), 80, x_dev=view)


def test_stat_topk_deterministic():
    x = torch.from_numpy(synth.stat_rows(9, 512, 9216)).to(DEV)
    a = sf.stat_topk(x, 737)
    b = sf.stat_topk(x, 737)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_stat_topk_theorem31_on_gpu():
    d, k = 9216, 737
    x = torch.from_numpy(synth.stat_rows(21, 4096, d, "gauss")).to(DEV)
    _, _, counts, _ = sf.stat_topk(x, k, cap=1)
    c = counts.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(c - k) / d <= np.sqrt(np.log(d) / d))
