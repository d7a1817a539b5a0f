"""The predictor step of the prefill on its own (spark_ffn_prefill_scores):
H = Q[:, :r] K1 in fp32 against the oracle's scores (the oracle reads the same
bf16 values in fp64), and against the scores the whole prefill thresholds."""
import numpy as np
import pytest
import torch

import attention_spark_ffn_amd as sf
import oracle
import synth
from parity import rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("T,dm,dff,r", [(4096, 2304, 9216, 1152), (100, 512, 1024, 256), (1, 256, 256, 128)])
def test_prefill_scores(T, dm, dff, r):
    lw = synth.ffn_layer(T, 0, dm, dff, r, "bf16")
    Qb = synth.queries(T, T, dm, "bf16")
    H = sf.spark_ffn_prefill_scores(bf(Qb), tuple(bf(a) for a in lw), r).cpu().numpy()
    rows = np.unique(np.linspace(0, T - 1, min(T, 64)).astype(int))
    ref = oracle.spark_ffn(Qb[rows], *lw, r, max(1, dff // 12))["h"]
    for j, t in enumerate(rows):
        # fp32 accumulation of bf16 products over r terms
        assert rel_err(H[t], ref[j]) <= 1e-5, (t, rel_err(H[t], ref[j]))
