"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before touching the
device."""
import ctypes
import os
import re

import numpy as np
import pytest
from scipy.special import ndtri

import attention_spark_ffn_amd as sf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spark_ffn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|size_t|double|const char \*)\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["stat_topk", "spark_ffn_decode", "spark_ffn_decode_batched", "spark_ffn_prefill", "spark_attn_decode",
              "spark_ffn_decode_noalloc", "spark_ffn_decode_noalloc_max_bytes", "spark_ffn_decode_tags",
              "spark_ffn_decode_workspace_size", "spark_ffn_decode_batched_workspace_size",
              "spark_ffn_prefill_workspace_size", "spark_attn_workspace_size",
              "spark_attn_prefill", "spark_attn_prefill_workspace_size", "spark_status_string", "spark_threshold_z"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = sf.lib()
    for n in declared_functions():
        assert hasattr(L, n), f"missing export {n}"


def test_status_strings():
    for st in (sf.SPARK_OK, sf.SPARK_EINVAL, sf.SPARK_EUNSUPPORTED, sf.SPARK_EHIP, sf.SPARK_EWORKSPACE):
        assert sf.status_string(st) and sf.status_string(st) != "unknown status"
    assert sf.status_string(12345) == "unknown status"


@pytest.mark.parametrize("k,d", [(737, 9216), (82, 1024), (256, 4096), (256, 32768), (1, 2), (5000, 9216),
                                 (512, 1024), (1, 1 << 20), (99999, 100000)])
def test_library_threshold_constant(k, d):
    # the library's own quantile (bisection + Newton on erfc) against a
    # 40-digit evaluation, Q(1 - k/d) = -sqrt(2) erfinv(2k/d - 1)
    import mpmath
    with mpmath.workdps(40):
        ref = float(-mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(k) / d - 1))
    assert abs(sf.threshold_z(k, d) - ref) <= 4e-15 * max(1.0, abs(ref))
    assert abs(sf.threshold_z(k, d) + ndtri(k / d)) < 1e-11  # and scipy, to its own accuracy
    assert np.isnan(sf.threshold_z(0, 10)) and np.isnan(sf.threshold_z(10, 10))


def test_stat_topk_rejects_bad_arguments():
    L = sf.lib()
    vp = ctypes.c_void_p(16)
    cases = [dict(rows=-1), dict(d=0), dict(ldx=5, d=10), dict(k=0), dict(k=10, d=10), dict(cap=-1)]
    for c in cases:
        a = dict(rows=4, d=10, ldx=10, k=3, cap=10)
        a.update(c)
        st = L.stat_topk(vp, a["rows"], a["d"], a["ldx"], a["k"], vp, vp, a["cap"], vp, None, None)
        assert st == sf.SPARK_EINVAL, (c, st)
    assert L.stat_topk(vp, 4, 70000, 70000, 3, vp, vp, 1, vp, None, None) == sf.SPARK_EUNSUPPORTED
    assert L.stat_topk(None, 4, 10, 10, 3, vp, vp, 1, vp, None, None) == sf.SPARK_EINVAL  # null x
    assert L.stat_topk(vp, 4, 10, 10, 3, vp, vp, 1, None, None, None) == sf.SPARK_EINVAL  # null counts
    assert L.stat_topk(None, 0, 10, 10, 3, None, None, 0, None, None, None) == sf.SPARK_OK  # empty: nothing to do


def _shape(**kw):
    a = dict(d_model=256, d_ff=1024, r=128, k=82, wdtype=sf.SPARK_F32)
    a.update(kw)
    return sf.ShapeC(a["d_model"], a["d_ff"], a["r"], a["k"], a["wdtype"])


@pytest.mark.parametrize("bad", [dict(r=0), dict(r=256), dict(k=0), dict(k=1024), dict(d_model=0), dict(d_ff=0),
                                 dict(r=130), dict(wdtype=sf.SPARK_BF16, r=124)])
def test_decode_rejects_bad_shapes(bad):
    L = sf.lib()
    s = _shape(**bad)
    w = (sf.WeightsC * 1)(sf.WeightsC(256, 256, 256))
    st = L.spark_ffn_decode(ctypes.byref(s), w, 1, ctypes.c_void_p(256), 1, ctypes.c_void_p(256), 1e-6, None,
                            ctypes.c_void_p(256), 1 << 30, None)
    assert st == sf.SPARK_EINVAL
    n = ctypes.c_size_t(0)
    assert L.spark_ffn_decode_workspace_size(ctypes.byref(s), 1, 1, ctypes.byref(n)) == sf.SPARK_EINVAL


def test_decode_rejects_bad_arguments():
    L = sf.lib()
    s = _shape()
    w = (sf.WeightsC * 1)(sf.WeightsC(256, 256, 256))
    good = dict(n=1, T=1, eps=1e-6)
    for bad in (dict(n=0), dict(T=-1), dict(eps=-1.0), dict(eps=float("nan"))):
        a = dict(good)
        a.update(bad)
        st = L.spark_ffn_decode(ctypes.byref(s), w, a["n"], ctypes.c_void_p(256), a["T"], ctypes.c_void_p(256),
                                a["eps"], None, ctypes.c_void_p(256), 1 << 30, None)
        assert st == sf.SPARK_EINVAL, bad
    assert L.spark_ffn_decode(None, w, 1, None, 1, None, 1e-6, None, None, 0, None) == sf.SPARK_EINVAL
    assert L.spark_ffn_decode(ctypes.byref(_shape(wdtype=7)), w, 1, None, 1, None, 1e-6, None, None, 0,
                              None) == sf.SPARK_EUNSUPPORTED


def test_batched_decode_rejects_bad_arguments():
    L = sf.lib()
    n = ctypes.c_size_t(0)
    W = L.spark_ffn_decode_batched_workspace_size
    assert W(ctypes.byref(_shape()), 4, ctypes.byref(n)) == sf.SPARK_OK and n.value > 0
    assert W(ctypes.byref(_shape()), -1, ctypes.byref(n)) == sf.SPARK_EINVAL
    assert W(ctypes.byref(_shape()), 9, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED  # more than 8 tokens
    big = _shape(d_model=8192, r=4096)
    assert W(ctypes.byref(big), 8, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED  # q slices beyond the LDS budget
    assert W(ctypes.byref(_shape(r=0)), 1, ctypes.byref(n)) == sf.SPARK_EINVAL
    s = _shape()
    w = (sf.WeightsC * 1)(sf.WeightsC(256, 256, 256))
    D = L.spark_ffn_decode_batched
    ws = ctypes.c_void_p(256)
    assert D(ctypes.byref(s), w, 0, ctypes.c_void_p(256), 1, ctypes.c_void_p(256), 1e-6, None, ws, 1 << 30,
             None) == sf.SPARK_EINVAL  # no layers
    assert D(ctypes.byref(s), w, 1, ctypes.c_void_p(260), 1, ctypes.c_void_p(256), 1e-6, None, ws, 1 << 30,
             None) == sf.SPARK_EINVAL  # q not 16-byte aligned
    assert D(ctypes.byref(s), w, 1, None, 1, ctypes.c_void_p(256), 1e-6, None, ws, 1 << 30,
             None) == sf.SPARK_EINVAL  # no q
    assert D(ctypes.byref(s), w, 1, ctypes.c_void_p(256), 1, ctypes.c_void_p(256), 1e-6, None, ws, 16,
             None) == sf.SPARK_EWORKSPACE
    assert D(ctypes.byref(s), w, 1, ctypes.c_void_p(256), 0, ctypes.c_void_p(256), 1e-6, None, ws, 1 << 30,
             None) == sf.SPARK_OK  # empty batch: nothing enqueued


def test_prefill_and_attention_reject_bad_arguments():
    L = sf.lib()
    n = ctypes.c_size_t(0)
    s = _shape(wdtype=sf.SPARK_F32)
    assert L.spark_ffn_prefill_workspace_size(ctypes.byref(s), 16, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED
    s = _shape(wdtype=sf.SPARK_BF16, d_ff=1000)
    assert L.spark_ffn_prefill_workspace_size(ctypes.byref(s), 16, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED
    s = _shape(wdtype=sf.SPARK_BF16, k=0)
    assert L.spark_ffn_prefill_workspace_size(ctypes.byref(s), 16, ctypes.byref(n)) == sf.SPARK_EINVAL
    A = L.spark_attn_workspace_size
    assert A(8, 3, 100, 256, 128, 256, ctypes.byref(n)) == sf.SPARK_EINVAL  # Hq % Hkv
    assert A(8, 4, 100, 256, 0, 256, ctypes.byref(n)) == sf.SPARK_EINVAL  # r
    assert A(8, 4, 100, 256, 256, 256, ctypes.byref(n)) == sf.SPARK_EINVAL  # r == hd
    assert A(8, 4, 0, 256, 128, 256, ctypes.byref(n)) == sf.SPARK_EINVAL  # empty context
    assert A(8, 4, 100, 256, 128, 0, ctypes.byref(n)) == sf.SPARK_EINVAL  # k_attn
    assert A(8, 4, 100, 1024, 512, 256, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED  # hd > 512
    assert A(8, 4, 100, 256, 128, 256, ctypes.byref(n)) == sf.SPARK_OK
    vp = ctypes.c_void_p(256)
    st = L.spark_attn_decode(None, vp, vp, vp, 8, 4, 100, 256, 128, 256, vp, None, None, 0, None, vp, 1 << 30, None)
    assert st == sf.SPARK_EINVAL
    st = L.spark_attn_decode(vp, vp, vp, vp, 8, 4, 100, 256, 128, 256, vp, None, None, 0, None, None, 0, None)
    assert st == sf.SPARK_EWORKSPACE


def test_attention_prefill_rejects_bad_arguments():
    L = sf.lib()
    n = ctypes.c_size_t(0)
    P = L.spark_attn_prefill_workspace_size
    assert P(64, 8, 3, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_EINVAL  # Hq % Hkv
    assert P(64, 8, 4, 256, 0, 256, 0, ctypes.byref(n)) == sf.SPARK_EINVAL  # r
    assert P(64, 8, 4, 256, 100, 256, 0, ctypes.byref(n)) == sf.SPARK_EINVAL  # r % 8
    assert P(0, 8, 4, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_EINVAL  # T
    assert P(1 << 15, 8, 4, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED  # T too long
    assert P(64, 8, 4, 1024, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED  # hd
    # r = hd - r: the fused kernels need only V^T and the threshold table
    assert P(64, 8, 4, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_OK
    assert 4 * 256 * 64 * 2 <= n.value < 64 * 64 * 8 * 6
    # other head splits materialise fp32 scores and bf16 weights
    assert P(64, 8, 4, 96, 32, 16, 0, ctypes.byref(n)) == sf.SPARK_OK and n.value > 64 * 64 * 8 * 6
    ws = ctypes.create_string_buffer(16)
    assert L.spark_attn_prefill(None, None, None, None, 64, 8, 4, 256, 128, 256, None, None, None, 0, None, ws, 16,
                                None) == sf.SPARK_EINVAL
    vp = ctypes.c_void_p(256)
    assert P(64, 8, 4, 256, 128, 256, -1, ctypes.byref(n)) == sf.SPARK_EINVAL  # negative list capacity
    assert L.spark_attn_prefill(vp, vp, vp, vp, 64, 8, 4, 256, 128, 256, vp, None, vp, -1, None, vp, 1 << 30,
                                None) == sf.SPARK_EINVAL
    # lists need the bitmask region: a workspace sized without it is too small
    assert P(64, 8, 4, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_OK
    small = n.value
    assert P(64, 8, 4, 256, 128, 256, 16, ctypes.byref(n)) == sf.SPARK_OK
    assert n.value >= small + 64 * 8 * 2 * 4
    assert L.spark_attn_prefill(vp, vp, vp, vp, 64, 8, 4, 256, 128, 256, vp, None, vp, 16, None, vp, small,
                                None) == sf.SPARK_EWORKSPACE


def test_empty_prefills():
    """A prefill of no tokens is a no-op that enqueues nothing (T >= 0); an
    attention prefill needs at least one position (1 <= T <= 16384)."""
    L = sf.lib()
    vp = ctypes.c_void_p(256)
    s = _shape(d_model=512, d_ff=1024, r=256, k=80, wdtype=sf.SPARK_BF16)
    w = sf.WeightsC(256, 256, 256)
    n = ctypes.c_size_t(0)
    assert L.spark_ffn_prefill_workspace_size(ctypes.byref(s), 0, ctypes.byref(n)) == sf.SPARK_OK
    assert L.spark_ffn_prefill(ctypes.byref(s), ctypes.byref(w), vp, 0, vp, None, vp, 1 << 30, None) == sf.SPARK_OK
    assert L.spark_ffn_prefill(ctypes.byref(s), ctypes.byref(w), vp, -1, vp, None, vp, 1 << 30, None) == sf.SPARK_EINVAL
    P = L.spark_attn_prefill_workspace_size
    assert P(0, 8, 4, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_EINVAL
    assert P(16385, 8, 4, 256, 128, 256, 0, ctypes.byref(n)) == sf.SPARK_EUNSUPPORTED
    assert L.spark_attn_prefill(vp, vp, vp, vp, 0, 8, 4, 256, 128, 256, vp, None, None, 0, None, vp, 1 << 30,
                                None) == sf.SPARK_EINVAL
