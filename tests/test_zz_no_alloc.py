"""spark_ffn_decode_noalloc -- the decode entry point for callers that cannot
allocate device memory -- against spark_ffn_decode on the same inputs, two
calls in a row, the second smaller: the same kernel on the library's
per-device scratch array must give the same results bit for bit (output,
selected sets, counts, thresholds, layer inputs)."""
import numpy as np
import pytest
import torch

import attention_spark_ffn_amd as sf
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def compare(q, layers, k, r):
    ref, tr_ref = sf.spark_ffn_decode(q, layers, k, r, trace=True)
    got, tr = sf.spark_ffn_decode_noalloc(q, layers, k, r, trace=True)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for key in ("counts", "idx", "theta", "q_in"):
        assert torch.equal(tr[key], tr_ref[key]), key


def test_noalloc_matches_decode_two_calls():
    dm, dff, r, k = 2304, 9216, 1152, 737
    layers = [tuple(to_dev(a) for a in synth.ffn_layer(21, l, dm, dff, r, "bf16")) for l in range(3)]
    q = torch.from_numpy(synth.queries(21, 3, dm)).to(DEV)
    print("noalloc: 3 layers x 3 tokens, then 2 layers x 1 token", flush=True)
    compare(q, layers, k, r)
    compare(q[:1].contiguous(), layers[:2], k, r)


def test_noalloc_fp32_tiny_and_repeat():
    layers = [tuple(to_dev(a) for a in synth.ffn_layer(0, 0, 256, 1024, 128, "f32"))]
    q = torch.from_numpy(synth.queries(0, 16, 256)).to(DEV)
    print("noalloc: tiny fp32 layer, 16 tokens then 4", flush=True)
    compare(q, layers, 82, 128)
    compare(q[:4].contiguous(), layers, 82, 128)
    a = sf.spark_ffn_decode_noalloc(q, layers, 82, 128)
    b = sf.spark_ffn_decode_noalloc(q, layers, 82, 128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_rejects_sizes_beyond_scratch():
    dm, dff, r = 512, 1024, 256
    layers = [tuple(to_dev(a) for a in synth.ffn_layer(3, 0, dm, dff, r, "f32"))] * 40
    T = sf.lib().spark_ffn_decode_noalloc_max_bytes() // (8 * dm) + 1
    q = torch.zeros((T, dm), device=DEV)
    with pytest.raises(RuntimeError, match="unsupported"):
        sf.spark_ffn_decode_noalloc(q, layers, 80, r)
