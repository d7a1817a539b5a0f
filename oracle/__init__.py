"""fp64 CPU oracle for the Spark FFN hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding in ``attention_spark_ffn_amd``) never imports, links or
calls anything here, and this package imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, plain loops, built with
gcc).  This module is argument marshalling over ctypes plus numpy containers.
bf16 arrays are passed as their raw 16-bit patterns (numpy ``uint16``).

What is computed, and from which passage, is stated in ``oracle.c``.  Every
function there is pinned by ``tests/test_oracle_pins.py`` to facts fixed
independently of it (library quantiles, closed forms, brute force, the
concentration result of the statistical top-k).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared", "-fopenmp",
                               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Lib:
    """ctypes view of one build of oracle.c (the default build, or a test's mutant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i64, ci, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_norm_quantile.restype = d
        lib.oracle_norm_quantile.argtypes = [d]
        lib.oracle_threshold_z.restype = d
        lib.oracle_threshold_z.argtypes = [i64, i64]
        lib.oracle_gelu_tanh.restype = d
        lib.oracle_gelu_tanh.argtypes = [d]
        lib.oracle_softplus.restype = d
        lib.oracle_softplus.argtypes = [d]
        lib.oracle_num_threads.restype = ci
        lib.oracle_stat_topk.restype = ci
        lib.oracle_stat_topk.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_spark_ffn.restype = ci
        lib.oracle_spark_ffn.argtypes = [i64, i64, i64, i64, ci, vp, vp, vp, ci, vp, i64, vp, vp, vp, vp, vp,
                                         i64, vp, vp, vp]
        lib.oracle_decode_stack.restype = ci
        lib.oracle_decode_stack.argtypes = [i64, i64, i64, i64, ci, ci, vp, vp, vp, vp, i64, d, vp, vp, vp]
        lib.oracle_spark_attn_decode.restype = ci
        lib.oracle_spark_attn_decode.argtypes = [ci, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, vp,
                                                 vp]
        lib.oracle_spark_attn_prefill.restype = ci
        lib.oracle_spark_attn_prefill.argtypes = [ci, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, vp]
        lib.oracle_spark_ffn_dense.restype = ci
        lib.oracle_spark_ffn_dense.argtypes = [i64, i64, i64, i64, ci, vp, vp, vp, ci, vp, i64, vp]
        lib.oracle_huber_relu.restype = d
        lib.oracle_huber_relu.argtypes = [d, d]
        lib.oracle_huber_relu_grad.restype = d
        lib.oracle_huber_relu_grad.argtypes = [d, d]
        lib.oracle_stat_topk_huber_forward.restype = ci
        lib.oracle_stat_topk_huber_forward.argtypes = [vp, i64, i64, i64, d, vp, vp]
        lib.oracle_stat_topk_huber_backward.restype = ci
        lib.oracle_stat_topk_huber_backward.argtypes = [vp, vp, i64, i64, i64, d, vp]
        self.c = lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _Lib(_LIB_PATH)
    return _lib.c


class use_build:
    """Context manager: route every call in this module through another build of
    oracle.c (the mutation test uses it to run the pins against planted mistakes)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _Lib(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def compile_variant(src_text: str, out_path: str) -> str:
    """Compile a (modified) copy of oracle.c to out_path with the same flags."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-D_DEFAULT_SOURCE", "-fPIC", "-shared", "-fopenmp",
                           "-ffp-contract=off", "-fno-fast-math", "-w", "-o", out_path, src, "-lm"])
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def num_threads() -> int:
    return _load().oracle_num_threads()


def norm_quantile(p: float) -> float:
    return _load().oracle_norm_quantile(float(p))


def threshold_z(k: int, d: int) -> float:
    return _load().oracle_threshold_z(int(k), int(d))


def gelu_tanh(v: float) -> float:
    return _load().oracle_gelu_tanh(float(v))


def softplus(v: float) -> float:
    return _load().oracle_softplus(float(v))


def stat_topk(x: np.ndarray, k: int, cap: int | None = None) -> dict:
    """Statistical top-k of each row of the fp32 matrix x [rows][d].

    Returns theta/mean/std [rows] (fp64), counts [rows] (true counts), and
    idx [rows][cap] int32 / vals [rows][cap] fp64 holding the first
    min(count, cap) selected entries in ascending index order (rest: -1 / 0).
    """
    x = _c(np.asarray(x, dtype=np.float32))
    if x.ndim == 1:
        x = x[None, :]
    rows, d = x.shape
    cap = d if cap is None else int(cap)
    vals = np.zeros((rows, cap), np.float64)
    idx = np.full((rows, cap), -1, np.int32)
    counts = np.zeros(rows, np.int32)
    theta, mean, sd = (np.zeros(rows, np.float64) for _ in range(3))
    rc = _load().oracle_stat_topk(_ptr(x), rows, d, d, int(k), cap, _ptr(vals), _ptr(idx), _ptr(counts),
                                  _ptr(theta), _ptr(mean), _ptr(sd))
    if rc != 0:
        raise ValueError("oracle_stat_topk: bad arguments")
    return dict(theta=theta, mean=mean, std=sd, counts=counts, idx=idx, vals=vals)


def spark_ffn(q: np.ndarray, k1t: np.ndarray, k2t: np.ndarray, v: np.ndarray, r: int, k: int) -> dict:
    """Spark FFN of one layer on T independent tokens.

    q [T][d_model] (fp32 or bf16 bits); k1t [d_ff][r], k2t [d_ff][d_model-r],
    v [d_ff][d_model] (all fp32, or all bf16 bits).  Returns y [T][d_model]
    fp64, counts, h [T][d_ff], idx/m [T][d_ff] (padded with -1 / 0), theta,
    mean, std.
    """
    q = _c(q)
    if q.ndim == 1:
        q = q[None, :]
    k1t, k2t, v = _c(k1t), _c(k2t), _c(v)
    T, d_model = q.shape
    d_ff = v.shape[0]
    wd = _dtype_code(k1t)
    assert _dtype_code(k2t) == wd and _dtype_code(v) == wd
    assert k1t.shape == (d_ff, r) and k2t.shape == (d_ff, d_model - r) and v.shape == (d_ff, d_model)
    y = np.zeros((T, d_model), np.float64)
    counts = np.zeros(T, np.int32)
    h = np.zeros((T, d_ff), np.float64)
    idx = np.full((T, d_ff), -1, np.int32)
    m = np.zeros((T, d_ff), np.float64)
    theta, mean, sd = (np.zeros(T, np.float64) for _ in range(3))
    rc = _load().oracle_spark_ffn(d_model, d_ff, int(r), int(k), wd, _ptr(k1t), _ptr(k2t), _ptr(v),
                                  _dtype_code(q), _ptr(q), T, _ptr(y), _ptr(counts), _ptr(h), _ptr(idx), _ptr(m),
                                  d_ff, _ptr(theta), _ptr(mean), _ptr(sd))
    if rc != 0:
        raise ValueError("oracle_spark_ffn: bad arguments")
    return dict(y=y, counts=counts, h=h, idx=idx, m=m, theta=theta, mean=mean, std=sd)


def decode_stack(q0: np.ndarray, layers, r: int, k: int, eps: float = 1e-6, trace: bool = False) -> dict:
    """Chain of Spark FFN layers with RMS normalisation in between.

    q0 [T][d_model] fp32; layers = list of (k1t, k2t, v) arrays.  Returns
    y [T][d_model] (last layer, before normalisation), counts [T][L] and,
    with trace=True, q_trace [T][L][d_model] (each layer's input).
    """
    q0 = _c(np.asarray(q0, dtype=np.float32))
    if q0.ndim == 1:
        q0 = q0[None, :]
    T, d_model = q0.shape
    L = len(layers)
    layers = [tuple(_c(a) for a in lw) for lw in layers]
    d_ff = layers[0][2].shape[0]
    wd = _dtype_code(layers[0][0])
    arr = ctypes.c_void_p * L
    p1 = arr(*[a[0].ctypes.data for a in layers])
    p2 = arr(*[a[1].ctypes.data for a in layers])
    p3 = arr(*[a[2].ctypes.data for a in layers])
    y = np.zeros((T, d_model), np.float64)
    counts = np.zeros((T, L), np.int32)
    qt = np.zeros((T, L, d_model), np.float64) if trace else None
    rc = _load().oracle_decode_stack(d_model, d_ff, int(r), int(k), wd, L, p1, p2, p3, _ptr(q0), T, float(eps),
                                     _ptr(y), _ptr(counts), _ptr(qt))
    if rc != 0:
        raise ValueError("oracle_decode_stack: bad arguments")
    return dict(y=y, counts=counts, q_trace=qt)


def spark_attn_decode(q: np.ndarray, k1: np.ndarray, k2: np.ndarray, v: np.ndarray, k_attn: int) -> dict:
    """Spark attention decode.  q [Hq][hd]; k1 [Hkv][n][r]; k2 [Hkv][n][hd-r];
    v [Hkv][n][hd]; one dtype for all (fp32 or bf16 bits).  Returns out
    [Hq][hd] fp64, counts [Hq], theta [Hq] (NaN when dense), scores
    [Hq][n]."""
    q, k1, k2, v = _c(q), _c(k1), _c(k2), _c(v)
    dt = _dtype_code(q)
    assert all(_dtype_code(a) == dt for a in (k1, k2, v))
    Hq, hd = q.shape
    Hkv, n, r = k1.shape
    assert k2.shape == (Hkv, n, hd - r) and v.shape == (Hkv, n, hd)
    out = np.zeros((Hq, hd), np.float64)
    counts = np.zeros(Hq, np.int32)
    theta = np.zeros(Hq, np.float64)
    scores = np.zeros((Hq, n), np.float64)
    rc = _load().oracle_spark_attn_decode(dt, _ptr(q), _ptr(k1), _ptr(k2), _ptr(v), Hq, Hkv, n, hd, r,
                                          int(k_attn), _ptr(out), _ptr(counts), _ptr(theta), _ptr(scores))
    if rc != 0:
        raise ValueError("oracle_spark_attn_decode: bad arguments")
    return dict(out=out, counts=counts, theta=theta, scores=scores)


def spark_attn_prefill(q: np.ndarray, k1: np.ndarray, k2: np.ndarray, v: np.ndarray, k_attn: int) -> dict:
    """Spark attention over a whole prompt, causal: the query of position t
    attends over positions 0..t with its own statistical top-k.  q [T][Hq][hd];
    k1 [Hkv][T][r]; k2 [Hkv][T][hd-r]; v [Hkv][T][hd]; one dtype for all.
    Returns out [T][Hq][hd] fp64, counts [T][Hq], theta [T][Hq] (NaN where
    t + 1 <= k_attn)."""
    q, k1, k2, v = _c(q), _c(k1), _c(k2), _c(v)
    dt = _dtype_code(q)
    assert all(_dtype_code(a) == dt for a in (k1, k2, v))
    T, Hq, hd = q.shape
    Hkv, n, r = k1.shape
    assert n == T and k2.shape == (Hkv, T, hd - r) and v.shape == (Hkv, T, hd)
    out = np.zeros((T, Hq, hd), np.float64)
    counts = np.zeros((T, Hq), np.int32)
    theta = np.zeros((T, Hq), np.float64)
    rc = _load().oracle_spark_attn_prefill(dt, _ptr(q), _ptr(k1), _ptr(k2), _ptr(v), T, Hq, Hkv, hd, r,
                                           int(k_attn), _ptr(out), _ptr(counts), _ptr(theta))
    if rc != 0:
        raise ValueError("oracle_spark_attn_prefill: bad arguments")
    return dict(out=out, counts=counts, theta=theta)


def huber_relu(u: float, delta: float) -> float:
    return _load().oracle_huber_relu(float(u), float(delta))


def huber_relu_grad(u: float, delta: float) -> float:
    return _load().oracle_huber_relu_grad(float(u), float(delta))


def stat_topk_huber(x: np.ndarray, k: int, delta: float) -> dict:
    """Huber-smoothed statistical top-k of each fp32 row of x [rows][d]:
    y [rows][d] fp64 (dense) and theta [rows]."""
    x = _c(np.asarray(x, dtype=np.float32))
    if x.ndim == 1:
        x = x[None, :]
    rows, d = x.shape
    y = np.zeros((rows, d), np.float64)
    theta = np.zeros(rows, np.float64)
    rc = _load().oracle_stat_topk_huber_forward(_ptr(x), rows, d, int(k), float(delta), _ptr(y), _ptr(theta))
    if rc != 0:
        raise ValueError("oracle_stat_topk_huber_forward: bad arguments")
    return dict(y=y, theta=theta)


def stat_topk_huber_backward(x: np.ndarray, dy: np.ndarray, k: int, delta: float) -> np.ndarray:
    """dL/dx [rows][d] fp64 of the Huber-smoothed statistical top-k, given
    dy = dL/dy (fp32 [rows][d]) at the fp32 input x."""
    x = _c(np.asarray(x, dtype=np.float32))
    dy = _c(np.asarray(dy, dtype=np.float32))
    if x.ndim == 1:
        x, dy = x[None, :], dy[None, :]
    assert dy.shape == x.shape
    rows, d = x.shape
    dx = np.zeros((rows, d), np.float64)
    rc = _load().oracle_stat_topk_huber_backward(_ptr(x), _ptr(dy), rows, d, int(k), float(delta), _ptr(dx))
    if rc != 0:
        raise ValueError("oracle_stat_topk_huber_backward: bad arguments")
    return dx


def spark_ffn_dense(q: np.ndarray, k1t: np.ndarray, k2t: np.ndarray, v: np.ndarray, r: int, k: int) -> np.ndarray:
    """The layer computed densely (every neuron's K2 dot and V row, unselected
    neurons weighted by zero): y [T][d_model] fp64, equal to spark_ffn's y."""
    q = _c(q)
    if q.ndim == 1:
        q = q[None, :]
    k1t, k2t, v = _c(k1t), _c(k2t), _c(v)
    T, d_model = q.shape
    d_ff = v.shape[0]
    wd = _dtype_code(k1t)
    y = np.zeros((T, d_model), np.float64)
    rc = _load().oracle_spark_ffn_dense(d_model, d_ff, int(r), int(k), wd, _ptr(k1t), _ptr(k2t), _ptr(v),
                                        _dtype_code(q), _ptr(q), T, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_spark_ffn_dense: bad arguments")
    return y
