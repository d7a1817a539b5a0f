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
    (2304, 9216, 1152, 737, 2, 1, "bf16"),  # a batch of one (the single-token persistent kernel)
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


# ---------------------------------------------------------------- more shapes, deep stacks, shared blocks
@pytest.mark.parametrize("dm,dff,r,k,L,B", [
    (1024, 3000, 512, 240, 3, 7),    # 11-12 neurons per workgroup, an odd batch
    (256, 256, 128, 30, 2, 4),       # one neuron per workgroup
    (2304, 9216, 1152, 737, 2, 3),   # three tokens in four slots
    (640, 9216, 320, 737, 2, 2),     # a narrow layer over the full neuron count
])
def test_batched_more_shapes(dm, dff, r, k, L, B):
    layers = [synth.ffn_layer(dm + dff + 3, l, dm, dff, r, "bf16") for l in range(L)]
    q0 = synth.queries(dm + 3, B, dm)
    run_stack(layers, q0, r, k, tol=2e-2, fn=sf.spark_ffn_decode_batched)


def test_batched_many_layers():
    """34 layers of a small bf16 layer, five tokens; the first, middle and
    last layers teacher-forced against the oracle, and the whole chain."""
    layers = [synth.ffn_layer(31, l, 256, 1024, 128, "bf16") for l in range(34)]
    q0 = synth.queries(31, 5, 256)
    run_stack(layers, q0, 128, 82, tol=2e-2, fn=sf.spark_ffn_decode_batched, check_layers=[0, 1, 31, 32, 33])


def test_batched_block_selected_by_every_token():
    """Planted keys that every token selects: the first 36 neurons (one
    workgroup's range) are selected by all eight tokens, and a block by tokens
    1 and 6 only; sets and outputs against the oracle."""
    dm, dff, r, k = 2304, 9216, 1152, 737
    q0 = synth.queries(17, 8, dm)
    blocks = [(tuple(range(8)), 0, 36, 0.3), ((1, 6), 5000, 5040, 0.2)]
    layers = [synth.ffn_layer_planted(17, 0, dm, dff, r, q0, blocks, "bf16"),
              synth.ffn_layer(17, 1, dm, dff, r, "bf16")]
    y, tr = run_stack(layers, q0, r, k, tol=2e-2, fn=sf.spark_ffn_decode_batched)
    for t in range(8):
        idx = set(tr["idx"][t, 0][: tr["counts"][t, 0]].tolist())
        assert set(range(36)) <= idx, t
        assert (set(range(5000, 5040)) <= idx) == (t in (1, 6)), t


def test_batched_one_token_failure_path_and_recovery():
    """A batch of one runs the single-token persistent kernel on the batched
    workspace: its failure path driven from the host through the workspace's
    test hook (every wait one polling round) ends with every kernel exiting,
    counts one failed call, leaves NaN in y and raises in the checked wrapper;
    with the hook cleared the next calls on the same workspace match a fresh
    workspace bit for bit."""
    layers_np = [synth.ffn_layer(19, l, 2304, 9216, 1152, "bf16") for l in range(3)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(19, 1, 2304)).to(DEV)
    nbytes = 1 << 24
    good = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=torch.zeros(nbytes, dtype=torch.uint8, device=DEV))
    ws = sf.TaggedWorkspace(torch.zeros(nbytes, dtype=torch.uint8, device=DEV))
    first = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, good) and ws.failures() == 0
    ws.buf[24:32].view(torch.int64).fill_(1)
    with pytest.raises(RuntimeError, match="timed out"):
        sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws)
    assert ws.failures() == 1
    y = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws, check=False)
    torch.cuda.synchronize()
    assert ws.new_failures() == 1 and ws.failures() == 2 and bool(torch.isnan(y).any())
    ws.buf[24:32].view(torch.int64).fill_(0)
    for _ in range(2):
        again = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, good)
    assert ws.failures() == 2


def test_batched_fused_failure_path_and_recovery():
    """Four tokens on bf16 weights run the fused predictor-and-gate kernel,
    whose workgroups exchange their score statistics while they run: its
    failure path driven from the host through the workspace's test hook ends
    with every kernel exiting, counts one failed call for three failed layers,
    leaves NaN in y and raises in the checked wrapper; with the hook cleared
    the next calls on the same workspace match a fresh workspace bit for bit."""
    layers_np = [synth.ffn_layer(31, l, 2304, 9216, 1152, "bf16") for l in range(3)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(31, 4, 2304)).to(DEV)
    nbytes = 1 << 24
    good = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=torch.zeros(nbytes, dtype=torch.uint8, device=DEV))
    ws = sf.TaggedWorkspace(torch.zeros(nbytes, dtype=torch.uint8, device=DEV))
    first = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, good) and ws.failures() == 0
    ws.buf[24:32].view(torch.int64).fill_(1)
    with pytest.raises(RuntimeError, match="timed out"):
        sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws)
    assert ws.failures() == 1
    y = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws, check=False)
    torch.cuda.synchronize()
    assert ws.new_failures() == 1 and ws.failures() == 2 and bool(torch.isnan(y).all())
    ws.buf[24:32].view(torch.int64).fill_(0)
    for _ in range(2):
        again = sf.spark_ffn_decode_batched(q, layers, 737, 1152, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, good)
    assert ws.failures() == 2


def test_batched_repeated_calls_share_workspace():
    """Calls with different batch sizes on the one cached workspace (a batch of
    one carries exchange tags in it, the others only use the space after its
    header) give the results of fresh workspaces, bit for bit."""
    layers_np = [synth.ffn_layer(23, l, 2304, 9216, 1152, "bf16") for l in range(2)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(23, 8, 2304)).to(DEV)
    for B in (8, 3, 1, 8, 1, 2):
        fresh = sf.spark_ffn_decode_batched(q[:B], layers, 737, 1152,
                                            ws=torch.zeros(1 << 24, dtype=torch.uint8, device=DEV))
        cached = sf.spark_ffn_decode_batched(q[:B], layers, 737, 1152)
        torch.cuda.synchronize()
        assert torch.equal(fresh, cached), B


def test_batched_one_token_matches_decode():
    """A batch of one and spark_ffn_decode run the same kernel: equal outputs
    bit for bit."""
    layers_np = [synth.ffn_layer(29, l, 2304, 9216, 1152, "bf16") for l in range(3)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(29, 1, 2304)).to(DEV)
    a = sf.spark_ffn_decode_batched(q, layers, 737, 1152)
    b = sf.spark_ffn_decode(q, layers, 737, 1152)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
