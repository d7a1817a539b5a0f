"""Seeded synthetic inputs for the Spark FFN / statistical top-k / Spark attention workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  It is the one piece that both the oracle side and the
HIP side of the tests and the bench consume, so the two always see the same
host arrays.

Conventions:
  * numpy ``default_rng(SeedSequence([seed, layer, tensor_id]))`` per tensor;
  * weights ~ N(0, 1/fan_in) with fan_in the contraction length (r for K1,
    d_model - r for K2, d_ff for V), drawn directly in the stored layout:
    K1 transposed [d_ff][r], K2 transposed [d_ff][d_model - r], V [d_ff][d_model]
    (entries are i.i.d., so the draw orientation does not change the law);
  * bf16 tensors are the round-to-nearest-even rounding of the fp32 draw and
    are carried as raw 16-bit patterns (numpy ``uint16``).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

K1_ID, K2_ID, V_ID, Q_ID, ROWS_ID, ATTN_ID = 1, 2, 3, 4, 5, 6


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(g: np.random.Generator, shape, scale: float) -> np.ndarray:
    a = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def ffn_layer(seed: int, layer: int, d_model: int, d_ff: int, r: int, dtype: str = "bf16"):
    """One Spark FFN layer's weights (k1t, k2t, v) in the stored layouts."""
    k1t = _normal(rng(seed, layer, K1_ID), (d_ff, r), 1.0 / np.sqrt(r))
    k2t = _normal(rng(seed, layer, K2_ID), (d_ff, d_model - r), 1.0 / np.sqrt(d_model - r))
    v = _normal(rng(seed, layer, V_ID), (d_ff, d_model), 1.0 / np.sqrt(d_ff))
    if dtype == "bf16":
        return f32_to_bf16_bits(k1t), f32_to_bf16_bits(k2t), f32_to_bf16_bits(v)
    if dtype == "f32":
        return k1t, k2t, v
    raise ValueError(dtype)


def ffn_stack(seed: int, n_layers: int, d_model: int, d_ff: int, r: int, dtype: str = "bf16", workers: int = 8):
    """n_layers independent layers, drawn in parallel threads (numpy releases the GIL)."""
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        return list(ex.map(lambda l: ffn_layer(seed, l, d_model, d_ff, r, dtype), range(n_layers)))


def ffn_layer_planted(seed: int, layer: int, d_model: int, d_ff: int, r: int, q: np.ndarray, blocks,
                      dtype: str = "bf16"):
    """ffn_layer with planted blocks of predictor keys: for each (t, lo, hi, s)
    in `blocks`, K1 rows lo..hi-1 become s times the unit direction of
    q[t, :r] plus N(0, (0.02 s)^2 / r) noise, so their scores for token t are
    about s * |q[t, :r]| (far above or below the rest for |s| ~ 0.1).  t may
    also be a tuple of tokens: the direction is then the normalised sum of
    their unit directions (about 1/sqrt(len(t)) of the score for each)."""
    k1t, k2t, v = ffn_layer(seed, layer, d_model, d_ff, r, "f32")
    g = rng(seed, layer, K1_ID, 1)
    for t, lo, hi, s in blocks:
        ts = t if isinstance(t, tuple) else (t,)
        u = np.zeros(r)
        for tt in ts:
            qt = q[tt, :r].astype(np.float64)
            u += qt / np.linalg.norm(qt)
        u = (u / np.linalg.norm(u)).astype(np.float32)
        k1t[lo:hi] = np.float32(s) * u + _normal(g, (hi - lo, r), 0.02 * abs(s) / np.sqrt(r))
    if dtype == "bf16":
        return f32_to_bf16_bits(k1t), f32_to_bf16_bits(k2t), f32_to_bf16_bits(v)
    if dtype == "f32":
        return k1t, k2t, v
    raise ValueError(dtype)


def queries(seed: int, T: int, d_model: int, dtype: str = "f32", stream: int = 0) -> np.ndarray:
    """T query vectors ~ N(0, 1)."""
    q = _normal(rng(seed, stream, Q_ID), (T, d_model), 1.0)
    return f32_to_bf16_bits(q) if dtype == "bf16" else q


def stat_rows(seed: int, rows: int, d: int, kind: str = "gauss") -> np.ndarray:
    """Rows x_ij = mu_i + s_i * e_ij with mu_i ~ U(-1,1), s_i ~ U(0.5,2) and
    e ~ N(0,1) (kind='gauss') or Student-t with 4 degrees of freedom
    (kind='t4'); the same (mu_i, s_i) for both kinds."""
    g = rng(seed, 0, ROWS_ID)
    mu = g.uniform(-1.0, 1.0, size=(rows, 1)).astype(np.float32)
    s = g.uniform(0.5, 2.0, size=(rows, 1)).astype(np.float32)
    ge = rng(seed, 1 if kind == "gauss" else 2, ROWS_ID)
    if kind == "gauss":
        e = ge.standard_normal(size=(rows, d), dtype=np.float32)
    elif kind == "t4":
        e = ge.standard_t(4, size=(rows, d)).astype(np.float32)
    else:
        raise ValueError(kind)
    e *= s
    e += mu
    return e


def attn_inputs(seed: int, Hq: int, Hkv: int, n_ctx: int, hd: int, r: int, scale: float | None = None):
    """Spark attention decode inputs, bf16 bits: q [Hq][hd] and the split KV
    cache k1 [Hkv][n][r], k2 [Hkv][n][hd-r], v [Hkv][n][hd], all ~ N(0,1)*scale
    with scale = 1/sqrt(hd) by default."""
    sc = (1.0 / np.sqrt(hd)) if scale is None else scale
    q = _normal(rng(seed, 0, ATTN_ID), (Hq, hd), sc)
    k = _normal(rng(seed, 1, ATTN_ID), (Hkv, n_ctx, hd), sc)
    v = _normal(rng(seed, 2, ATTN_ID), (Hkv, n_ctx, hd), sc)
    b = f32_to_bf16_bits
    return b(q), b(np.ascontiguousarray(k[:, :, :r])), b(np.ascontiguousarray(k[:, :, r:])), b(v)


def attn_prefill_inputs(seed: int, T: int, Hq: int, Hkv: int, hd: int, r: int, scale: float | None = None):
    """Spark attention prefill inputs, bf16 bits: queries q [T][Hq][hd] and the
    split cache of the same T positions k1 [Hkv][T][r], k2 [Hkv][T][hd-r],
    v [Hkv][T][hd], all ~ N(0,1)*scale with scale = 1/sqrt(hd) by default."""
    sc = (1.0 / np.sqrt(hd)) if scale is None else scale
    q = _normal(rng(seed, 3, ATTN_ID), (T, Hq, hd), sc)
    k = _normal(rng(seed, 4, ATTN_ID), (Hkv, T, hd), sc)
    v = _normal(rng(seed, 5, ATTN_ID), (Hkv, T, hd), sc)
    b = f32_to_bf16_bits
    return b(q), b(np.ascontiguousarray(k[:, :, :r])), b(np.ascontiguousarray(k[:, :, r:])), b(v)
