"""Causal Spark attention prefill on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import attention_spark_ffn_amd as sf
import oracle
import synth
from parity import TIE_BAND, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def run_prefill(T, Hq, Hkv, hd, r, ka, seed, tol=2e-2, scale=None):
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(seed, T, Hq, Hkv, hd, r, scale=scale)
    out, counts, theta = sf.spark_attn_prefill(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka)
    torch.cuda.synchronize()
    out, counts, theta = (t.cpu().numpy() for t in (out, counts, theta))
    ref = oracle.spark_attn_prefill(qb, k1b, k2b, vb, ka)
    w = synth.bf16_bits_to_f32
    q64, k164 = w(qb).astype(np.float64), w(k1b).astype(np.float64)
    grp = Hq // Hkv
    for t in range(T):
        for h in range(Hq):
            n = t + 1
            if n <= ka:  # every position attended
                assert counts[t, h] == n and np.isnan(theta[t, h]), (t, h)
            else:
                s = k164[h // grp, :n] @ q64[t, h, :r]
                sd = s.std()
                th = ref["theta"][t, h]
                assert abs(theta[t, h] - th) <= 1e-5 * (abs(th) + sd), (t, h, theta[t, h], th)
                if counts[t, h] != ref["counts"][t, h]:
                    # only entries inside the tie band of theta may be decided differently
                    near = int(np.sum(np.abs(s - th) <= TIE_BAND * sd))
                    assert abs(int(counts[t, h]) - int(ref["counts"][t, h])) <= near, (t, h)
            assert rel_err(out[t, h], ref["out"][t, h]) <= tol, (t, h, rel_err(out[t, h], ref["out"][t, h]))


@pytest.mark.parametrize("T,Hq,Hkv,hd,r,ka", [
    (40, 4, 2, 32, 16, 8),        # K shorter than one 64 step; dense rows then thresholded rows
    (300, 8, 4, 64, 32, 64),      # T not a multiple of 8 (padded rows of the scores and weights)
    (130, 2, 1, 128, 64, 200),    # every row dense (T <= k_attn)
    (1000, 8, 4, 256, 128, 256),
    (1, 1, 1, 16, 8, 4),          # one position
    (200, 4, 2, 96, 32, 32),      # r != hd - r: the materialised-scores path
    (150, 6, 2, 64, 32, 16),      # three heads per KV head: 64-query row sets of one head
    (257, 2, 2, 32, 16, 300),     # one head per KV head, every row dense
])
def test_attn_prefill_shapes(T, Hq, Hkv, hd, r, ka):
    run_prefill(T, Hq, Hkv, hd, r, ka, seed=T + hd)


def test_attn_prefill_config():
    """The attention configuration (Hq 8, Hkv 4, hd 256, r 128, k_attn 256) over a
    2048-position prompt: 16 tiles of 128 queries, causal tiles skipped."""
    run_prefill(2048, 8, 4, 256, 128, 256, seed=7)


def test_attn_prefill_last_row_is_decode():
    """The last position of a prefill is a decode step over the whole cache."""
    T, Hq, Hkv, hd, r, ka = 700, 8, 4, 128, 64, 128
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(3, T, Hq, Hkv, hd, r)
    out, counts, _ = sf.spark_attn_prefill(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka)
    od, cd, _, _ = sf.spark_attn_decode(to_dev(np.ascontiguousarray(qb[T - 1])), to_dev(k1b), to_dev(k2b),
                                        to_dev(vb), ka)
    torch.cuda.synchronize()
    assert np.array_equal(counts[T - 1].cpu().numpy(), cd.cpu().numpy())
    for h in range(Hq):
        assert rel_err(out[T - 1, h].cpu().numpy(), od[h].cpu().numpy()) <= 1e-2


def test_attn_prefill_deterministic():
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(5, 513, 8, 4, 256, 128)
    args = [to_dev(a) for a in (qb, k1b, k2b, vb)]
    a = sf.spark_attn_prefill(*args, 256)
    b = sf.spark_attn_prefill(*args, 256)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_attn_prefill_bench_workload_sampled_rows():
    """The timed attention-prefill workload (a 4096-position prompt, Hq 8, Hkv 4,
    hd 256, r 128, k_attn 256, the bench's inputs): row t of a causal prefill
    is a decode step over positions 0..t, so sampled rows are checked one by
    one against the oracle's decode on that prefix, all heads, including dense
    rows, the first thresholded row and the last."""
    T, Hq, Hkv, hd, r, ka = 4096, 8, 4, 256, 128, 256
    qb, k1b, k2b, vb = synth.attn_prefill_inputs(0, T, Hq, Hkv, hd, r)
    out, counts, theta = sf.spark_attn_prefill(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka)
    torch.cuda.synchronize()
    out, counts, theta = (t.cpu().numpy() for t in (out, counts, theta))
    for t in (0, 37, 255, 256, 257, 1023, 2048, 2049, 3333, 4094, 4095):
        n = t + 1
        ref = oracle.spark_attn_decode(np.ascontiguousarray(qb[t]), np.ascontiguousarray(k1b[:, :n]),
                                       np.ascontiguousarray(k2b[:, :n]), np.ascontiguousarray(vb[:, :n]), ka)
        for h in range(Hq):
            if n <= ka:
                assert counts[t, h] == n and np.isnan(theta[t, h]), (t, h)
            else:
                s = ref["scores"][h]
                sd = s.std()
                th = ref["theta"][h]
                assert abs(theta[t, h] - th) <= 1e-5 * (abs(th) + sd), (t, h, theta[t, h], th)
                if counts[t, h] != ref["counts"][h]:
                    near = int(np.sum(np.abs(s - th) <= TIE_BAND * sd))
                    assert abs(int(counts[t, h]) - int(ref["counts"][h])) <= near, (t, h)
            assert rel_err(out[t, h], ref["out"][h]) <= 2e-2, (t, h, rel_err(out[t, h], ref["out"][h]))
