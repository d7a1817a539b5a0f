"""Causal Spark attention prefill on the GPU against the fp64 oracle.

Every (position, head) row is checked: the threshold, the attended set
(positions listed by the library, compared with the oracle's set outside the
tie band of 1e-4 std around the oracle's threshold), its count, and the
output row (rel 2e-2 for the bf16 path).
"""
import numpy as np
import pytest
import torch

import attention_spark_ffn_amd as sf
import oracle
import synth
from parity import check_index_set, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def check_row(t, h, s, th_ref, out_row, out_ref, count, idx_row, cap, theta, ka, tol):
    """One row: s are the row's fp64 predictor scores over positions 0..t."""
    n = t + 1
    listed = idx_row[:min(int(count), cap)]
    if n <= ka:  # every position attended
        assert count == n and np.isnan(theta), (t, h, count, theta)
        assert np.array_equal(listed, np.arange(min(n, cap))), (t, h)
    else:
        sd = s.std()
        assert abs(theta - th_ref) <= 1e-5 * (abs(th_ref) + sd), (t, h, theta, th_ref)
        check_index_set(idx_row, count, cap, s, th_ref, sd, f"row t={t} h={h}")
    assert np.all(idx_row[min(int(count), cap):] == -1), (t, h)
    assert rel_err(out_row, out_ref) <= tol, (t, h, rel_err(out_row, out_ref))


def run_prefill(T, Hq, Hkv, hd, r, ka, seed, tol=2e-2, scale=None):
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(seed, T, Hq, Hkv, hd, r, scale=scale)
    cap = T
    out, counts, idx, theta = sf.spark_attn_prefill(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka, cap=cap)
    torch.cuda.synchronize()
    out, counts, idx, theta = (t.cpu().numpy() for t in (out, counts, idx, theta))
    ref = oracle.spark_attn_prefill(qb, k1b, k2b, vb, ka)
    w = synth.bf16_bits_to_f32
    q64, k164 = w(qb).astype(np.float64), w(k1b).astype(np.float64)
    grp = Hq // Hkv
    flips = 0
    for t in range(T):
        for h in range(Hq):
            s = k164[h // grp, :t + 1] @ q64[t, h, :r]
            check_row(t, h, s, ref["theta"][t, h], out[t, h], ref["out"][t, h], counts[t, h], idx[t, h], cap,
                      theta[t, h], ka, tol)
            flips += int(counts[t, h] != ref["counts"][t, h])
    return flips


@pytest.mark.parametrize("T,Hq,Hkv,hd,r,ka", [
    (40, 4, 2, 32, 16, 8),        # K shorter than one 64 step; dense rows then thresholded rows
    (300, 8, 4, 64, 32, 64),      # T not a multiple of 8 (padded rows of the scores and weights)
    (130, 2, 1, 128, 64, 200),    # every row dense (T <= k_attn)
    (1000, 8, 4, 256, 128, 256),
    (1, 1, 1, 16, 8, 4),          # one position
    (200, 4, 2, 96, 32, 32),      # r != hd - r: the materialised-scores path
    (150, 6, 2, 64, 32, 16),      # three heads per KV head: 64-query row sets of one head
    (257, 2, 2, 32, 16, 300),     # one head per KV head, every row dense
    (1100, 4, 2, 96, 32, 100),    # materialised-scores path past one 1024-score row chunk
])
def test_attn_prefill_shapes(T, Hq, Hkv, hd, r, ka):
    run_prefill(T, Hq, Hkv, hd, r, ka, seed=T + hd)


def test_attn_prefill_config():
    """The attention configuration (Hq 8, Hkv 4, hd 256, r 128, k_attn 256) over a
    2048-position prompt: every row's threshold, set and output."""
    run_prefill(2048, 8, 4, 256, 128, 256, seed=7)


def test_attn_prefill_list_capacity():
    """A list capacity below the counts: true counts, the first cap positions
    listed (ascending), and the same outputs as without lists."""
    T, Hq, Hkv, hd, r, ka, cap = 600, 8, 4, 128, 64, 128, 40
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(17, T, Hq, Hkv, hd, r)
    args = [to_dev(a) for a in (qb, k1b, k2b, vb)]
    out, counts, idx, theta = sf.spark_attn_prefill(*args, ka, cap=cap)
    out0, counts0, idx0, _ = sf.spark_attn_prefill(*args, ka)
    full = sf.spark_attn_prefill(*args, ka, cap=T)[2]
    torch.cuda.synchronize()
    assert idx0 is None and torch.equal(out, out0) and torch.equal(counts, counts0)
    counts, idx, full = counts.cpu().numpy(), idx.cpu().numpy(), full.cpu().numpy()
    for t in range(T):
        for h in range(Hq):
            c = int(counts[t, h])
            assert np.array_equal(idx[t, h, :min(c, cap)], full[t, h, :min(c, cap)])
            assert np.all(idx[t, h, min(c, cap):] == -1)


def test_attn_prefill_last_row_is_decode():
    """The last position of a prefill is a decode step over the whole cache."""
    T, Hq, Hkv, hd, r, ka = 700, 8, 4, 128, 64, 128
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(3, T, Hq, Hkv, hd, r)
    out, counts, _, _ = sf.spark_attn_prefill(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka)
    od, cd, _, _ = sf.spark_attn_decode(to_dev(np.ascontiguousarray(qb[T - 1])), to_dev(k1b), to_dev(k2b),
                                        to_dev(vb), ka)
    torch.cuda.synchronize()
    assert np.array_equal(counts[T - 1].cpu().numpy(), cd.cpu().numpy())
    for h in range(Hq):
        assert rel_err(out[T - 1, h].cpu().numpy(), od[h].cpu().numpy()) <= 1e-2


def test_attn_prefill_deterministic():
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(5, 513, 8, 4, 256, 128)
    args = [to_dev(a) for a in (qb, k1b, k2b, vb)]
    a = sf.spark_attn_prefill(*args, 256, cap=513)
    b = sf.spark_attn_prefill(*args, 256, cap=513)
    assert all(torch.equal(u, v) for u, v in zip(a[:3], b[:3]))
    assert torch.equal(torch.isnan(a[3]), torch.isnan(b[3]))  # NaN where every position is attended
    assert torch.equal(torch.nan_to_num(a[3]), torch.nan_to_num(b[3]))


def test_attn_prefill_bench_workload_sampled_rows():
    """The timed attention-prefill workload (a 4096-position prompt, Hq 8, Hkv 4,
    hd 256, r 128, k_attn 256, the bench's inputs): row t of a causal prefill
    is a decode step over positions 0..t, so sampled rows are checked one by
    one against the oracle's decode on that prefix, all heads: the first and
    last row of every 32-position query block, the dense-to-thresholded
    transition and rows in between."""
    T, Hq, Hkv, hd, r, ka, cap = 4096, 8, 4, 256, 128, 256, 1024
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(0, T, Hq, Hkv, hd, r)
    out, counts, idx, theta = sf.spark_attn_prefill(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka, cap=cap)
    torch.cuda.synchronize()
    out, counts, idx, theta = (t.cpu().numpy() for t in (out, counts, idx, theta))
    rows = set()
    for b in range(T // 32):
        rows |= {32 * b, 32 * b + 31}
    rows |= {37, 254, 255, 256, 257, 258, 1023, 1024, 2049, 3333, 4094}
    assert len(rows) >= 256
    for t in sorted(rows):
        n = t + 1
        ref = oracle.spark_attn_decode(np.ascontiguousarray(qb[t]), np.ascontiguousarray(k1b[:, :n]),
                                       np.ascontiguousarray(k2b[:, :n]), np.ascontiguousarray(vb[:, :n]), ka)
        for h in range(Hq):
            check_row(t, h, ref["scores"][h], ref["theta"][h], out[t, h], ref["out"][h], counts[t, h], idx[t, h],
                      cap, theta[t, h], ka, 2e-2)
