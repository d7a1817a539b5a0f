"""Spark attention decode on the GPU against the fp64 oracle."""
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


def run_attn(Hq, Hkv, n, hd, r, ka, seed, tol=2e-2, scale=None):
    qb, k1b, k2b, vb = synth.attn_inputs(seed, Hq, Hkv, n, hd, r, scale=scale)
    cap = min(n, 4096)
    out, counts, idx, theta = sf.spark_attn_decode(to_dev(qb), to_dev(k1b), to_dev(k2b), to_dev(vb), ka, cap=cap)
    torch.cuda.synchronize()
    out, counts, idx, theta = (t.cpu().numpy() for t in (out, counts, idx, theta))
    ref = oracle.spark_attn_decode(qb, k1b, k2b, vb, ka)
    dense = n <= ka
    for h in range(Hq):
        s = ref["scores"][h]
        if dense:
            assert counts[h] == n and np.isnan(theta[h])
            assert np.array_equal(idx[h, :min(n, cap)], np.arange(min(n, cap)))
        else:
            sd = s.std()
            check_index_set(idx[h], counts[h], cap, s, ref["theta"][h], sd, f"head {h}")
            assert abs(theta[h] - ref["theta"][h]) <= 1e-5 * (abs(ref["theta"][h]) + sd)
        assert rel_err(out[h], ref["out"][h]) <= tol, (h, rel_err(out[h], ref["out"][h]))
    return counts


@pytest.mark.parametrize("n", [4096, 32768])
def test_attn_config(n):
    """The attention decode workload: 8 query heads on 4 KV heads, hd 256,
    r 128, k_attn 256, Q/K/V ~ N(0,1)/16 in bf16."""
    counts = run_attn(8, 4, n, 256, 128, 256, 0)
    assert np.all(np.abs(counts - 256) <= 256 * 0.5)


@pytest.mark.parametrize("Hq,Hkv,n,hd,r,ka", [
    (8, 4, 200, 256, 128, 256),     # dense: fewer tokens than k_attn
    (8, 4, 256, 256, 128, 256),     # dense at the boundary
    (8, 4, 257, 256, 128, 256),     # one past the boundary
    (4, 4, 1000, 128, 64, 100),     # no grouping, ragged
    (8, 2, 5000, 64, 32, 300),      # group of 4
    (8, 4, 10000, 256, 128, 256),   # 128-token chunks (79 of them, the last 16 tokens long)
    (2, 1, 70000, 256, 128, 512),   # long context, 256-token chunks (the last 112 tokens long)
    (1, 1, 33, 16, 8, 8),           # tiny
])
def test_attn_shapes(Hq, Hkv, n, hd, r, ka):
    run_attn(Hq, Hkv, n, hd, r, ka, n + hd, scale=0.5)


def test_attn_deterministic():
    qb, k1b, k2b, vb = synth.attn_inputs(4, 8, 4, 32768, 256, 128)
    args = [to_dev(a) for a in (qb, k1b, k2b, vb)]
    a = sf.spark_attn_decode(*args, 256)
    b = sf.spark_attn_decode(*args, 256)
    for u, w in zip(a, b):
        assert torch.equal(u, w)


@pytest.mark.parametrize("Hq,Hkv,n,hd,r,ka", [
    (16, 1, 3000, 128, 64, 200),     # 16 query heads per KV head (two register groups of 8)
    (2, 1, 150000, 64, 32, 256),     # 586 chunks of 256 tokens
    (2, 1, 3000, 512, 256, 4096),    # every token attended, more than one LDS batch, hd 512
    (4, 2, 20000, 320, 160, 4000),   # ~4000 selected: two LDS batches; hd 320
    (2, 2, 5000, 264, 128, 8000),    # every token attended, more than the list capacity of 4096
])
def test_attn_wide_groups_and_long_context(Hq, Hkv, n, hd, r, ka):
    run_attn(Hq, Hkv, n, hd, r, ka, n + Hq, scale=0.5)


def test_attn_repeated_calls():
    """Many calls in a row on changing inputs and one cached workspace: each
    matches the oracle's result for its own inputs."""
    for i in range(6):
        n = 4096 if i % 2 == 0 else 1500
        run_attn(8, 4, n, 256, 128, 256, 100 + i)
