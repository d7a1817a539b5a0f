"""Batched Spark FFN decode (B tokens layer by layer, one K1 read per layer,
K2/V rows read once per union of the selected sets) on the GPU against the
fp64 oracle, and against the token-by-token decode."""
import numpy as np
import pytest
import torch

import attention_spark_ffn_amd as sf
import synth
from parity import rel_err
from test_gpu_decode import DEV, run_stack, to_dev

pytestmark = pytest.mark.gpu


def test_batched_tiny_fp32_config():
    """The tiny fp32 layer (d_model 256, d_ff 1024, r 128, k 82), 8 tokens, 3 layers."""
    layers = [synth.ffn_layer(0, l, 256, 1024, 128, "f32") for l in range(3)]
    q0 = synth.queries(0, 8, 256)
    run_stack(layers, q0, 128, 82, tol=1e-4, fn=sf.spark_ffn_decode_batched)


@pytest.mark.parametrize("dm,dff,r,k,L,B,dt", [
    (64, 256, 32, 20, 3, 2, "f32"),       # tiny, several layers
    (2304, 9216, 1152, 737, 3, 8, "bf16"),
    (512, 1000, 256, 80, 2, 5, "bf16"),   # d_ff not a multiple of the 32-neuron blocks, odd batch
    (1024, 4096, 512, 300, 4, 4, "f32"),
    (136, 300, 64, 29, 2, 3, "bf16"),     # ragged everywhere
    (2304, 9216, 1152, 737, 2, 1, "bf16"),  # a batch of one (the single-token V kernel)
    (2304, 9216, 1152, 737, 2, 2, "bf16"),  # the smallest batch of the sliced V product
])
def test_batched_shapes(dm, dff, r, k, L, B, dt):
    layers = [synth.ffn_layer(dm + dff + 1, l, dm, dff, r, dt) for l in range(L)]
    q0 = synth.queries(dm + 1, B, dm)
    run_stack(layers, q0, r, k, tol=1e-4 if dt == "f32" else 2e-2, fn=sf.spark_ffn_decode_batched)


def test_batched_full_stack_config():
    """The 26-layer decode workload (2304 x 9216, r 1152, k 737, bf16), 8 tokens:
    every layer teacher-forced against the oracle, and the whole chain."""
    layers = synth.ffn_stack(0, 26, 2304, 9216, 1152, "bf16")
    q0 = synth.queries(0, 8, 2304)
    run_stack(layers, q0, 1152, 737, tol=2e-2, fn=sf.spark_ffn_decode_batched)


def test_batched_clustered_selection():
    """Planted blocks of active neurons (see the token-by-token test): a
    neuron block selected by every token, or by one token only."""
    dm, dff, r, k = 2304, 9216, 1152, 737
    q0 = synth.queries(11, 2, dm)
    blocks = [(0, 0, 64, 0.1), (1, 4000, 4100, 0.1), (0, 3600, 3612, 0.1), (0, 3612, 3636, -0.1)]
    layers = [synth.ffn_layer_planted(11, 0, dm, dff, r, q0, blocks, "bf16"),
              synth.ffn_layer(11, 1, dm, dff, r, "bf16")]
    y, tr = run_stack(layers, q0, r, k, tol=2e-2, fn=sf.spark_ffn_decode_batched)
    idx0 = set(tr["idx"][0, 0][: tr["counts"][0, 0]].tolist())
    assert set(range(64)) | set(range(3600, 3612)) <= idx0 and not idx0 & set(range(3612, 3636))
    idx1 = set(tr["idx"][1, 0][: tr["counts"][1, 0]].tolist())
    assert set(range(4000, 4100)) <= idx1


def test_batched_matches_token_by_token_decode():
    """Same layers and tokens through both entry points: outputs agree to the
    fp32 rounding of the two summation orders (bf16 weights, 4 layers)."""
    layers_np = [synth.ffn_layer(21, l, 2304, 9216, 1152, "bf16") for l in range(4)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(21, 6, 2304)).to(DEV)
    ya, ta = sf.spark_ffn_decode(q, layers, 737, 1152, trace=True)
    yb, tb = sf.spark_ffn_decode_batched(q, layers, 737, 1152, trace=True)
    torch.cuda.synchronize()
    for t in range(6):
        assert rel_err(yb[t].cpu().numpy(), ya[t].cpu().numpy()) <= 1e-3, t
    # the selected counts agree up to near-threshold flips
    assert (ta["counts"] - tb["counts"]).abs().max().item() <= 3


def test_batched_deterministic():
    layers_np = [synth.ffn_layer(7, l, 2304, 9216, 1152, "bf16") for l in range(3)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(7, 8, 2304)).to(DEV)
    a = sf.spark_ffn_decode_batched(q, layers, 737, 1152)
    b = sf.spark_ffn_decode_batched(q, layers, 737, 1152)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
