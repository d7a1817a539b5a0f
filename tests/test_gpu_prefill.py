"""Spark FFN prefill on the GPU against the fp64 oracle."""
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
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def run_prefill(dm, dff, r, k, T, seed, sample=None, tol=2e-2, gathered=False):
    layer = synth.ffn_layer(seed, 0, dm, dff, r, "bf16")
    Q = synth.queries(seed, T, dm, "bf16")
    Y, tr = sf.spark_ffn_prefill(to_dev(Q), tuple(to_dev(a) for a in layer), k, r, trace=True, gathered=gathered)
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    tr = {key: v.cpu().numpy() for key, v in tr.items()}
    rows = np.arange(T) if sample is None else np.asarray(sample)
    ref = oracle.spark_ffn(Q[rows], *layer, r, k)
    flips = 0
    for i, t in enumerate(rows):
        flips += check_index_set(tr["idx"][t, 0], tr["counts"][t, 0], dff, ref["h"][i], ref["theta"][i],
                                 ref["std"][i], f"token {t}")
        assert abs(tr["theta"][t, 0] - ref["theta"][i]) <= 1e-5 * (abs(ref["theta"][i]) + ref["std"][i])
        assert rel_err(Y[t], ref["y"][i]) <= tol, (t, rel_err(Y[t], ref["y"][i]))
    return flips


def test_prefill_config():
    """The prefill workload: 4096 tokens through one 2304 x 9216 layer
    (r 1152, k 737), bf16; a sample of 96 tokens against the oracle, spread
    over every 128-row tile of the predictor GEMM."""
    T = 4096
    sample = np.sort(np.random.default_rng(0).choice(T, 96, replace=False))
    run_prefill(2304, 9216, 1152, 737, T, 0, sample)


@pytest.mark.parametrize("dm,dff,r,k,T", [
    (256, 1024, 128, 82, 300),      # ragged token count (not a multiple of 128)
    (512, 512, 192, 40, 130),
    (1024, 2048, 512, 160, 64),
    (136, 256, 64, 20, 1),          # one token
    (2304, 9216, 1152, 737, 257),
])
def test_prefill_shapes(dm, dff, r, k, T):
    run_prefill(dm, dff, r, k, T, dm + T)


def test_prefill_large_tiles_ragged():
    """Enough tokens for the 256 x 192 product tiles (ceil(3000/256) x
    ceil(4096/192) = 264 tiles, at least one per CU) with both edges ragged:
    the last tile row holds 184 tokens and the last tile column 64 neurons.
    A sample of tokens, every fourth of the last tile row included."""
    T = 3000
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([rng.choice(2816, 60, replace=False), np.arange(2816, T, 4), [T - 1]]))
    run_prefill(512, 4096, 256, 330, T, 11, sample)


def test_prefill_large_tiles_full_width_ragged():
    """The full-width layer (2304 x 9216, r 1152, k 737) over 2900 tokens: the
    scores and gate products on 256 x 192 tiles (12 x 48) and the C V product
    on 256 x 192 tiles in four K splits (12 x 12 x 4), the last tile row 84
    tokens deep.  A sample of tokens including the last tile row."""
    T = 2900
    rng = np.random.default_rng(6)
    sample = np.unique(np.concatenate([rng.choice(2816, 24, replace=False), np.arange(2816, T, 6), [T - 1]]))
    run_prefill(2304, 9216, 1152, 737, T, 12, sample)


def test_prefill_deterministic():
    layer = [to_dev(a) for a in synth.ffn_layer(3, 0, 2304, 9216, 1152, "bf16")]
    Q = to_dev(synth.queries(3, 512, 2304, "bf16"))
    a = sf.spark_ffn_prefill(Q, layer, 737, 1152)
    b = sf.spark_ffn_prefill(Q, layer, 737, 1152)
    assert torch.equal(a, b)


@pytest.mark.parametrize("T", [4096, 300])
def test_prefill_traced_and_untraced_agree(T):
    """The timed call (no trace) and the traced call select with the same
    thresholds, so their outputs are identical; the trace's counts are those of
    its lists."""
    layer = [to_dev(a) for a in synth.ffn_layer(4, 0, 2304, 9216, 1152, "bf16")]
    Q = to_dev(synth.queries(4, T, 2304, "bf16"))
    a = sf.spark_ffn_prefill(Q, layer, 737, 1152)
    b, tr = sf.spark_ffn_prefill(Q, layer, 737, 1152, trace=True)
    c, tr2 = sf.spark_ffn_prefill(Q, layer, 737, 1152, trace=True, cap=1)
    assert torch.equal(a, b) and torch.equal(a, c)
    assert torch.equal(tr["counts"], tr2["counts"]) and torch.equal(tr["theta"], tr2["theta"])
    assert torch.equal((tr["idx"][:, 0] >= 0).sum(1).int(), tr["counts"][:, 0])


def test_prefill_matches_decode_per_token():
    # the same layer through the prefill path and the decode path (bf16 q)
    dm, dff, r, k = 512, 1024, 256, 80
    layer_np = synth.ffn_layer(8, 0, dm, dff, r, "bf16")
    Qb = synth.queries(8, 16, dm, "bf16")
    layer = tuple(to_dev(a) for a in layer_np)
    Y = sf.spark_ffn_prefill(to_dev(Qb), layer, k, r).cpu().numpy()
    q32 = torch.from_numpy(synth.bf16_bits_to_f32(Qb)).to(DEV)
    Yd = sf.spark_ffn_decode(q32, [layer], k, r).cpu().numpy()
    # prefill feeds the gated values to the V product on the matrix cores as
    # bf16 (relative rounding 2^-9 each); decode keeps them fp32.  The rounding
    # errors of the ~80 terms add at random, far inside 2^-8 of the norm.
    for t in range(16):
        assert rel_err(Y[t], Yd[t]) <= 2.0 ** -8


# ---------------------------------------------------------------- the gathered form
def test_prefill_gathered_config():
    """spark_ffn_prefill_gathered on the prefill workload (4096 tokens, 2304 x
    9216, r 1152, k 737): 96 sampled tokens against the oracle."""
    T = 4096
    sample = np.sort(np.random.default_rng(1).choice(T, 96, replace=False))
    run_prefill(2304, 9216, 1152, 737, T, 0, sample, gathered=True)


@pytest.mark.parametrize("dm,dff,r,k,T", [
    (256, 1024, 128, 82, 300),
    (136, 256, 64, 20, 1),
    (512, 4096, 256, 330, 700),
])
def test_prefill_gathered_shapes(dm, dff, r, k, T):
    run_prefill(dm, dff, r, k, T, dm + T + 1, gathered=True)


def test_prefill_gathered_matches_dense_and_is_deterministic():
    """The gathered and the dense forms select with the same thresholds (the
    same scores and statistics), so their lists are identical; their outputs
    differ only by the dense form's bf16 rounding of the gated values."""
    layer = [to_dev(a) for a in synth.ffn_layer(9, 0, 2304, 9216, 1152, "bf16")]
    Q = to_dev(synth.queries(9, 1000, 2304, "bf16"))
    yd, trd = sf.spark_ffn_prefill(Q, layer, 737, 1152, trace=True)
    yg, trg = sf.spark_ffn_prefill(Q, layer, 737, 1152, trace=True, gathered=True)
    yg2 = sf.spark_ffn_prefill(Q, layer, 737, 1152, gathered=True)
    torch.cuda.synchronize()
    assert torch.equal(trd["idx"], trg["idx"]) and torch.equal(trd["counts"], trg["counts"])
    assert torch.equal(yg, yg2)
    yd, yg = yd.cpu().numpy(), yg.cpu().numpy()
    for t in range(0, 1000, 7):
        assert rel_err(yd[t], yg[t]) <= 2.0 ** -8, t
