"""Comparison rules between the HIP path and the fp64 oracle.

Index sets: the selected set of the GPU and of the oracle may differ only in
entries whose oracle score lies within 1e-4 * std of the oracle threshold
(the tie band); everything else must match exactly, lists must be ascending.
Values: normwise relative error ||a - b|| / ||b|| within the stated tolerance.
"""
from __future__ import annotations

import numpy as np

TIE_BAND = 1e-4


def rel_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def check_index_set(gpu_list, gpu_count, cap, x_ref, theta_ref, std_ref, what=""):
    """Check one row's GPU index list against the oracle's scores/threshold.

    Returns the number of tie-band flips (entries selected by exactly one side)."""
    x_ref = np.asarray(x_ref, np.float64)
    gpu_count = int(gpu_count)
    listed = np.asarray(gpu_list[:min(gpu_count, cap)], np.int64)
    assert np.all(np.diff(listed) > 0), f"{what}: GPU list not strictly ascending"
    assert listed.size == 0 or (listed.min() >= 0 and listed.max() < x_ref.size), f"{what}: index out of range"
    ref = np.nonzero(x_ref > theta_ref)[0]
    band = np.abs(x_ref - theta_ref) <= TIE_BAND * std_ref
    if gpu_count <= cap:
        sym = np.setxor1d(listed, ref)
        assert np.all(band[sym]), f"{what}: {int((~band[sym]).sum())} set differences outside the tie band"
        assert abs(gpu_count - ref.size) <= int(band.sum()), f"{what}: count {gpu_count} vs {ref.size}"
        return int(sym.size)
    # truncated list: the first `cap` entries of the GPU's set
    ref_prefix = ref[:cap]
    sym = np.setxor1d(listed, ref_prefix)
    # a tie flip below the cap shifts the prefix; accept differences that are band entries or shifted tails
    assert np.all(band[sym] | (sym >= min(listed.max(initial=0), ref_prefix.max(initial=0)))), what
    return int(sym.size)
