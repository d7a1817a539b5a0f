"""Spark FFN decode on the GPU against the fp64 oracle."""
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
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def layer_parity(q_in, lw, r, k, gpu_idx, gpu_count, gpu_theta, y_next_gpu, eps, tol, cap, what):
    """Teacher-forced check of one layer: the oracle runs the layer on the GPU's
    own input q_in; compare the selected set and the layer output."""
    ref = oracle.spark_ffn(q_in[None, :].astype(np.float32), *lw, r, k)
    h, th, sd = ref["h"][0], ref["theta"][0], ref["std"][0]
    flips = check_index_set(gpu_idx, gpu_count, cap, h, th, sd, what)
    assert abs(gpu_theta - th) <= 1e-5 * (abs(th) + sd), (what, gpu_theta, th)
    y = ref["y"][0]
    if y_next_gpu is not None:  # compare normalised outputs
        yn = y / np.sqrt(np.mean(y * y) + eps)
        assert rel_err(y_next_gpu, yn) <= tol, (what, rel_err(y_next_gpu, yn))
    return flips, y


def run_stack(layers_np, q0, r, k, eps=1e-6, tol=1e-4, check_layers=None, fn=None):
    """fn: the decode entry point under test (spark_ffn_decode by default)."""
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(q0).to(DEV)
    d_ff = layers_np[0][2].shape[0]
    y, tr = (fn or sf.spark_ffn_decode)(q, layers, k, r, eps, trace=True)
    torch.cuda.synchronize()
    if fn is None:
        assert not sf.decode_workspace_failed(device=torch.device(DEV))
    y = y.cpu().numpy()
    tr = {key: v.cpu().numpy() for key, v in tr.items()}
    T, L = tr["counts"].shape
    # per layer, teacher-forced on the GPU's own layer inputs
    for t in range(T):
        for l in (range(L) if check_layers is None else check_layers):
            y_next = tr["q_in"][t, l + 1] if l + 1 < L else None
            _, y_ref = layer_parity(tr["q_in"][t, l], layers_np[l], r, k, tr["idx"][t, l], tr["counts"][t, l],
                                    tr["theta"][t, l], y_next, eps, tol, d_ff, f"token {t} layer {l}")
            if l == L - 1:
                assert rel_err(y[t], y_ref) <= tol, (t, rel_err(y[t], y_ref))
    # The whole chain against the oracle's own chain.  A stack of random layers
    # with RMS normalisation is chaotic (the oracle alone amplifies a 1e-7 input
    # perturbation about 1.8x per layer), so the chain is held to the oracle's
    # own conditioning: at every layer the GPU may drift from the oracle at most
    # 100x as far as the oracle drifts from itself when its input is perturbed at
    # fp32 rounding level, or by tol, whichever is larger.  After the first few
    # layers that bound is loose (the oracle's own drift reaches O(1) by layer
    # 26 of the 2304 x 9216 stack), so parity rests on the per-layer,
    # teacher-forced checks above; this one catches a wrong chain (a missing
    # normalisation, a layer applied twice) in the early layers.
    ref = oracle.decode_stack(q0, layers_np, r, k, eps, trace=True)
    g = np.random.default_rng(99)
    qp = (q0.astype(np.float64) * (1 + 2.0 ** -24 * g.standard_normal(q0.shape))).astype(np.float32)
    pert = oracle.decode_stack(qp, layers_np, r, k, eps, trace=True)
    for t in range(T):
        for l in range(L):
            d_gpu = rel_err(tr["q_in"][t, l], ref["q_trace"][t, l])
            d_self = rel_err(pert["q_trace"][t, l], ref["q_trace"][t, l])
            assert d_gpu <= max(tol, 100 * d_self), (t, l, d_gpu, d_self)
        d_gpu = rel_err(y[t], ref["y"][t])
        d_self = rel_err(pert["y"][t], ref["y"][t])
        assert d_gpu <= max(tol, 100 * d_self), (t, "y", d_gpu, d_self)
    return y, tr


def test_decode_tiny_fp32_config():
    """The tiny Spark FFN layer: d_model 256, d_ff 1024, r 128, k 82, fp32, 16 tokens."""
    layers = [synth.ffn_layer(0, 0, 256, 1024, 128, "f32")]
    q0 = synth.queries(0, 16, 256)
    run_stack(layers, q0, 128, 82, tol=1e-4)


@pytest.mark.parametrize("dm,dff,r,k,L,T,dt", [
    (64, 256, 32, 20, 3, 2, "f32"),       # tiny, several layers
    (2304, 9216, 1152, 737, 2, 1, "bf16"),
    (512, 1000, 256, 80, 2, 3, "bf16"),   # d_ff not a multiple of the grid
    (1024, 4096, 512, 300, 4, 2, "f32"),
    (136, 300, 64, 29, 2, 2, "bf16"),     # ragged everywhere
])
def test_decode_shapes(dm, dff, r, k, L, T, dt):
    layers = [synth.ffn_layer(dm + dff, l, dm, dff, r, dt) for l in range(L)]
    q0 = synth.queries(dm, T, dm)
    run_stack(layers, q0, r, k, tol=1e-4 if dt == "f32" else 2e-2)


def test_decode_full_stack_config():
    """The decode workload: 26 layers of 2304 x 9216, r 1152, k 737, bf16
    weights, fp32 q, RMS normalisation between layers; 2 tokens, every layer
    teacher-forced against the oracle, and the whole chain."""
    L = 26
    layers = synth.ffn_stack(0, L, 2304, 9216, 1152, "bf16")
    q0 = synth.queries(0, 2, 2304)
    run_stack(layers, q0, 1152, 737, tol=2e-2)


def test_decode_clustered_selection():
    """Workgroups whose neurons are nearly all selected.  Layer 0 plants blocks
    of predictor keys along each token's query: token 0 gets 64 contiguous
    neurons far above theta (more than a workgroup publishes as candidates
    with 256 workgroups of 36 neurons), token 1 a block of 100; neurons
    3600..3611 are far above theta and 3612..3635 far below for token 0 (with
    256 workgroups: exactly the candidates selected, none beyond).  Any grid
    must give the oracle's result."""
    dm, dff, r, k = 2304, 9216, 1152, 737
    q0 = synth.queries(11, 2, dm)
    blocks = [(0, 0, 64, 0.1), (1, 4000, 4100, 0.1), (0, 3600, 3612, 0.1), (0, 3612, 3636, -0.1)]
    layers = [synth.ffn_layer_planted(11, 0, dm, dff, r, q0, blocks, "bf16"),
              synth.ffn_layer(11, 1, dm, dff, r, "bf16")]
    y, tr = run_stack(layers, q0, r, k, tol=2e-2)
    idx0 = set(tr["idx"][0, 0][: tr["counts"][0, 0]].tolist())
    assert set(range(64)) | set(range(3600, 3612)) <= idx0 and not idx0 & set(range(3612, 3636))
    idx1 = set(tr["idx"][1, 0][: tr["counts"][1, 0]].tolist())
    assert set(range(4000, 4100)) <= idx1


def test_decode_many_layers_segments():
    # more layers than one launch holds: the stack is split across launches
    L = 40
    layers = [synth.ffn_layer(5, l, 64, 256, 32, "f32") for l in range(L)]
    q0 = synth.queries(5, 2, 64)
    run_stack(layers, q0, 32, 20, tol=1e-4, check_layers=[0, 31, 32, 39])


def test_decode_deterministic_and_reusable_workspace():
    layers_np = [synth.ffn_layer(7, l, 2304, 9216, 1152, "bf16") for l in range(3)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(7, 3, 2304)).to(DEV)
    a = sf.spark_ffn_decode(q, layers, 737, 1152)
    b = sf.spark_ffn_decode(q, layers, 737, 1152)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)  # a fresh caller-owned workspace
    c = sf.spark_ffn_decode(q, layers, 737, 1152, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
    assert not sf.decode_workspace_failed(ws)


def test_decode_failure_path_and_recovery():
    """The failure path, driven from the host: a wait bound of one polling round
    (the workspace's test hook) makes the exchanges time out; the call must
    end with every kernel exiting normally, count one failed call, leave NaN
    in the output, and raise in the checked wrapper.  With the hook cleared,
    the next calls on the same workspace match a fresh workspace bit for bit
    (the failed call's words cannot satisfy their waits)."""
    layers_np = [synth.ffn_layer(13, l, 2304, 9216, 1152, "bf16") for l in range(3)]
    layers = [tuple(to_dev(a) for a in lw) for lw in layers_np]
    q = torch.from_numpy(synth.queries(13, 2, 2304)).to(DEV)
    good = sf.spark_ffn_decode(q, layers, 737, 1152, ws=torch.zeros(1 << 22, dtype=torch.uint8, device=DEV))
    ws = sf.DecodeWorkspace(torch.zeros(1 << 22, dtype=torch.uint8, device=DEV))
    first = sf.spark_ffn_decode(q, layers, 737, 1152, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, good) and ws.failures() == 0
    ws.buf[24:32].view(torch.int64).fill_(1)  # every wait: one polling round
    with pytest.raises(RuntimeError, match="timed out"):
        sf.spark_ffn_decode(q, layers, 737, 1152, ws=ws)
    assert ws.failures() == 1
    y = sf.spark_ffn_decode(q, layers, 737, 1152, ws=ws, check=False)
    torch.cuda.synchronize()
    assert ws.new_failures() == 1 and ws.failures() == 2 and bool(torch.isnan(y).any())
    ws.buf[24:32].view(torch.int64).fill_(0)
    for _ in range(2):
        again = sf.spark_ffn_decode(q, layers, 737, 1152, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, good)
    assert ws.failures() == 2
