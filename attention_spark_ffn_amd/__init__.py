"""Python binding of libspark_ffn.so, the MI355X (gfx950) Spark FFN library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/spark_ffn.h.  PyTorch supplies
device memory (tensors' data pointers) and the current HIP stream.  There is no
fallback: if the library is not built, or a call returns an error status, a
RuntimeError is raised.

Entry points (same names as the C ABI):
  stat_topk(x, k, cap=None)                         -> (vals, idx, counts, theta)
  stat_topk_huber(x, k, delta)                      -> (y, theta)   Huber-smoothed, dense
  stat_topk_huber_backward(x, dy, k, delta)         -> dx
  StatTopkHuber.apply(x, k, delta)                  -> y, as a torch.autograd.Function
  spark_ffn_decode(q, layers, k, r, eps, ...)       -> y  (and a trace dict)
  spark_ffn_decode_noalloc(q, layers, k, r, eps, ...)  -> the same, no device allocation by the library
  spark_ffn_decode_batched(q, layers, k, r, eps, ...)  -> the same, B <= 8 tokens layer by layer
  spark_ffn_prefill(Q, layer, k, r, ...)            -> Y  (and a trace dict)
  spark_attn_decode(q, k1, k2, v, k_attn, cap=None) -> (out, counts, idx, theta)
  spark_attn_prefill(q, k1, k2, v, k_attn, cap=0)   -> (out, counts, idx, theta)

Workspaces are cached per (kind, device, stream), so calls on different
streams never share one.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspark_ffn.so")

SPARK_OK, SPARK_EINVAL, SPARK_EUNSUPPORTED, SPARK_EHIP, SPARK_EWORKSPACE = 0, -1, -2, -3, -4
SPARK_F32, SPARK_BF16 = 0, 1

_vp, _i64, _ci, _f, _d, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double,
                               ctypes.c_size_t)


class ShapeC(ctypes.Structure):
    _fields_ = [("d_model", _i64), ("d_ff", _i64), ("r", _i64), ("k", _i64), ("wdtype", _ci)]


class WeightsC(ctypes.Structure):
    _fields_ = [("k1t", _vp), ("k2t", _vp), ("v", _vp)]


class TraceC(ctypes.Structure):
    _fields_ = [("counts", _vp), ("idx", _vp), ("theta", _vp), ("q_in", _vp), ("cap", _i64)]


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libspark_ffn.so (after torch, so that it binds to torch's HIP runtime)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is not built: run `python -m attention_spark_ffn_amd.build`")
                L = ctypes.CDLL(LIB_PATH)
                L.spark_status_string.restype = ctypes.c_char_p
                L.spark_status_string.argtypes = [_ci]
                L.spark_threshold_z.restype = _d
                L.spark_threshold_z.argtypes = [_i64, _i64]
                L.stat_topk_huber_forward.restype = _ci
                L.stat_topk_huber_forward.argtypes = [_vp, _i64, _i64, _i64, _f, _vp, _vp, _vp]
                L.stat_topk_huber_backward.restype = _ci
                L.stat_topk_huber_backward.argtypes = [_vp, _vp, _i64, _i64, _i64, _f, _vp, _vp]
                L.stat_topk.restype = _ci
                L.stat_topk.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp]
                L.spark_ffn_decode.restype = _ci
                L.spark_ffn_decode.argtypes = [ctypes.POINTER(ShapeC), ctypes.POINTER(WeightsC), _ci, _vp, _i64, _vp,
                                               _f, ctypes.POINTER(TraceC), _vp, _sz, _vp]
                L.spark_ffn_decode_batched.restype = _ci
                L.spark_ffn_decode_batched.argtypes = [ctypes.POINTER(ShapeC), ctypes.POINTER(WeightsC), _ci, _vp,
                                                       _i64, _vp, _f, ctypes.POINTER(TraceC), _vp, _sz, _vp]
                L.spark_ffn_decode_batched_workspace_size.restype = _ci
                L.spark_ffn_decode_batched_workspace_size.argtypes = [ctypes.POINTER(ShapeC), _i64,
                                                                      ctypes.POINTER(_sz)]
                L.spark_ffn_prefill.restype = _ci
                L.spark_ffn_prefill.argtypes = [ctypes.POINTER(ShapeC), ctypes.POINTER(WeightsC), _vp, _i64, _vp,
                                                ctypes.POINTER(TraceC), _vp, _sz, _vp]
                L.spark_ffn_prefill_gathered.restype = _ci
                L.spark_ffn_prefill_gathered.argtypes = [ctypes.POINTER(ShapeC), ctypes.POINTER(WeightsC), _vp,
                                                         _i64, _vp, ctypes.POINTER(TraceC), _vp, _sz, _vp]
                L.spark_ffn_prefill_gathered_workspace_size.restype = _ci
                L.spark_ffn_prefill_gathered_workspace_size.argtypes = [ctypes.POINTER(ShapeC), _i64,
                                                                        ctypes.POINTER(_sz)]
                L.spark_ffn_prefill_scores.restype = _ci
                L.spark_ffn_prefill_scores.argtypes = [ctypes.POINTER(ShapeC), ctypes.POINTER(WeightsC), _vp, _i64,
                                                       _vp, _vp]
                L.spark_hbm_read_probe.restype = _ci
                L.spark_hbm_read_probe.argtypes = [_vp, _sz, _vp, _vp]
                L.spark_attn_decode.restype = _ci
                L.spark_attn_decode.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp,
                                                _vp, _i64, _vp, _vp, _sz, _vp]
                L.spark_ffn_decode_noalloc.restype = _ci
                L.spark_ffn_decode_noalloc.argtypes = [ctypes.POINTER(ShapeC), ctypes.POINTER(WeightsC), _ci, _vp,
                                                       _i64, _vp, _f, ctypes.POINTER(TraceC), _vp]
                L.spark_ffn_decode_noalloc_max_bytes.restype = _sz
                L.spark_ffn_decode_noalloc_max_bytes.argtypes = []
                L.spark_ffn_decode_tags.restype = _i64
                L.spark_ffn_decode_tags.argtypes = [_ci, _i64]
                L.spark_ffn_decode_workspace_size.restype = _ci
                L.spark_ffn_decode_workspace_size.argtypes = [ctypes.POINTER(ShapeC), _ci, _i64,
                                                              ctypes.POINTER(_sz)]
                L.spark_ffn_prefill_workspace_size.restype = _ci
                L.spark_ffn_prefill_workspace_size.argtypes = [ctypes.POINTER(ShapeC), _i64, ctypes.POINTER(_sz)]
                L.spark_attn_workspace_size.restype = _ci
                L.spark_attn_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, ctypes.POINTER(_sz)]
                L.spark_attn_prefill.restype = _ci
                L.spark_attn_prefill.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp,
                                                 _vp, _i64, _vp, _vp, _sz, _vp]
                L.spark_attn_prefill_workspace_size.restype = _ci
                L.spark_attn_prefill_workspace_size.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                                                ctypes.POINTER(_sz)]
                _lib = L
    return _lib


def status_string(st: int) -> str:
    return lib().spark_status_string(st).decode()


def _check(st: int, what: str):
    if st != SPARK_OK:
        raise RuntimeError(f"{what}: {status_string(st)} (status {st})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _wdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SPARK_BF16
    if t.dtype == torch.float32:
        return SPARK_F32
    raise TypeError(f"weights must be bf16 or fp32, got {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on a HIP device")


def threshold_z(k: int, d: int) -> float:
    """The library's Q(1 - k/d) (host fp64)."""
    return lib().spark_threshold_z(int(k), int(d))


# ---------------------------------------------------------------------------- stat_topk
def stat_topk(x: torch.Tensor, k: int, cap: int | None = None):
    """Statistical top-k of each row of fp32 x [rows][d] (row stride taken from x).

    Returns vals [rows][cap] fp32, idx [rows][cap] int32 (first min(count, cap)
    selected entries, ascending; the rest of each row untouched: zeros / -1),
    counts [rows] int32 (true counts) and theta [rows] fp32.
    """
    if x.dim() != 2 or x.dtype != torch.float32 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a 2-D fp32 HIP tensor with unit column stride")
    rows, d = x.shape
    cap = d if cap is None else int(cap)
    dev = x.device
    vals = torch.zeros((rows, cap), dtype=torch.float32, device=dev)
    idx = torch.full((rows, cap), -1, dtype=torch.int32, device=dev)
    counts = torch.empty(rows, dtype=torch.int32, device=dev)
    theta = torch.empty(rows, dtype=torch.float32, device=dev)
    st = lib().stat_topk(_p(x), rows, d, x.stride(0) if rows > 0 else d, int(k), _p(vals), _p(idx), cap, _p(counts),
                         _p(theta), _stream(dev))
    _check(st, "stat_topk")
    return vals, idx, counts, theta


# ---------------------------------------------------------------------------- training side
def _rows_f32(*ts):
    for t in ts:
        if t.dim() != 2 or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("expected contiguous 2-D fp32 HIP tensors")


def stat_topk_huber(x: torch.Tensor, k: int, delta: float):
    """Huber-smoothed statistical top-k of each row of fp32 x [rows][d]: the
    dense y [rows][d] = h(x - theta) and theta [rows]."""
    _rows_f32(x)
    rows, d = x.shape
    y = torch.empty_like(x)
    theta = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib().stat_topk_huber_forward(_p(x), rows, d, int(k), float(delta), _p(y), _p(theta), _stream(x.device)),
           "stat_topk_huber_forward")
    return y, theta


def stat_topk_huber_backward(x: torch.Tensor, dy: torch.Tensor, k: int, delta: float) -> torch.Tensor:
    """dL/dx of the Huber-smoothed statistical top-k at input x, given dy = dL/dy."""
    _rows_f32(x, dy)
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    rows, d = x.shape
    dx = torch.empty_like(x)
    _check(lib().stat_topk_huber_backward(_p(x), _p(dy), rows, d, int(k), float(delta), _p(dx), _stream(x.device)),
           "stat_topk_huber_backward")
    return dx


class StatTopkHuber(torch.autograd.Function):
    """y = StatTopkHuber.apply(x, k, delta): the smoothed operator as an
    autograd function (forward and backward both run in the HIP kernels)."""

    @staticmethod
    def forward(ctx, x, k, delta):
        x = x.contiguous()
        y, _ = stat_topk_huber(x, k, delta)
        ctx.save_for_backward(x)
        ctx.k, ctx.delta = int(k), float(delta)
        return y

    @staticmethod
    def backward(ctx, dy):
        (x,) = ctx.saved_tensors
        return stat_topk_huber_backward(x, dy.contiguous(), ctx.k, ctx.delta), None, None


# ---------------------------------------------------------------------------- workspaces
_ws_cache: dict = {}

TAG_LIMIT = (1 << 32) - 1  # exchange tags are 32-bit; tag 0 is what a zeroed workspace holds


def _ws_key(kind: str, device):
    return (kind, device, torch.cuda.current_stream(device).cuda_stream)


def _cached_workspace(kind: str, device, nbytes: int) -> torch.Tensor:
    """Workspace for one (kind, device, stream), zero-filled when created."""
    key = _ws_key(kind, device)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


class TaggedWorkspace:
    """A workspace whose kernels exchange tagged words between workgroups
    (the decode kernel), with its host-side bookkeeping: the exchange
    tags the calls on it have used since it was last zeroed (it is zeroed
    again, on its stream, before they would pass 2^32 - 1), and the
    failed-call count the host last saw (the kernels count failed calls in the
    8-byte word at byte offset 16)."""

    def __init__(self, buf: torch.Tensor):
        self.buf = buf
        self.tags_used = 0
        self.failures_seen = 0

    def reserve(self, tags: int) -> bool:
        """Account for a call that uses `tags` tags; returns True when the
        workspace must be zeroed first (the count then restarts)."""
        reset = self.tags_used + tags > TAG_LIMIT
        if reset:
            self.tags_used = 0
        self.tags_used += tags
        return reset

    def failures(self) -> int:
        """Failed calls recorded in the workspace (reads it: synchronises)."""
        return int(self.buf[16:24].view(torch.int64).item())

    def new_failures(self) -> int:
        """Failed calls recorded since this was last asked (synchronises)."""
        n = self.failures()
        d, self.failures_seen = n - self.failures_seen, n
        return d


def decode_tags(n_layers: int, T: int) -> int:
    """Exchange tags one spark_ffn_decode call uses (the library's count)."""
    return int(lib().spark_ffn_decode_tags(int(n_layers), int(T)))


DecodeWorkspace = TaggedWorkspace


def _tagged_workspace(kind: str, device, nbytes: int) -> TaggedWorkspace:
    key = _ws_key(kind, device)
    dw = _ws_cache.get(key)
    if dw is None or dw.buf.numel() < nbytes:
        dw = TaggedWorkspace(torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device))
        _ws_cache[key] = dw
    return dw


def _decode_workspace(device, nbytes: int) -> TaggedWorkspace:
    return _tagged_workspace("decode", device, nbytes)


# ---------------------------------------------------------------------------- decode


def _shape(d_model, d_ff, r, k, wd) -> ShapeC:
    return ShapeC(int(d_model), int(d_ff), int(r), int(k), int(wd))


def _stack_args(q: torch.Tensor, layers, k: int, r: int):
    """Shape checks of a layer stack; the C shape and weight-table structs."""
    _need_cuda(q)
    T, d_model = q.shape
    L = len(layers)
    k1t0, k2t0, v0 = layers[0]
    d_ff = v0.shape[0]
    wd = _wdtype(k1t0)
    for lw in layers:
        _need_cuda(*lw)
        if any(_wdtype(a) != wd for a in lw):
            raise TypeError("all weights must share one dtype")
        if lw[0].shape != (d_ff, r) or lw[1].shape != (d_ff, d_model - r) or lw[2].shape != (d_ff, d_model):
            raise ValueError("weight shapes do not match q / r")
    shape = _shape(d_model, d_ff, r, k, wd)
    wts = (WeightsC * L)(*[WeightsC(a.data_ptr(), b.data_ptr(), c.data_ptr()) for (a, b, c) in layers])
    return T, d_model, L, d_ff, shape, wts


def _trace_buffers(T: int, L: int, d_ff: int, d_model: int, cap, dev):
    cap = d_ff if cap is None else int(cap)
    tr = dict(counts=torch.zeros((T, L), dtype=torch.int32, device=dev),
              idx=torch.full((T, L, cap), -1, dtype=torch.int32, device=dev),
              theta=torch.zeros((T, L), dtype=torch.float32, device=dev),
              q_in=torch.zeros((T, L, d_model), dtype=torch.float32, device=dev))
    trc = TraceC(tr["counts"].data_ptr(), tr["idx"].data_ptr(), tr["theta"].data_ptr(), tr["q_in"].data_ptr(), cap)
    return tr, trc


def spark_ffn_decode(q: torch.Tensor, layers, k: int, r: int, eps: float = 1e-6, trace: bool = False,
                     cap: int | None = None, ws: torch.Tensor | DecodeWorkspace | None = None, check: bool = True):
    """Run the stack of Spark FFN layers on T independent tokens.

    q [T][d_model] fp32; layers: list of (k1t [d_ff][r], k2t [d_ff][d_model-r],
    v [d_ff][d_model]) tensors, all bf16 or all fp32.  Returns y [T][d_model]
    fp32 (last layer, before normalisation).  With trace=True also returns a
    dict with counts [T][L], idx [T][L][cap], theta [T][L], q_in [T][L][d_model].
    ws: optional workspace to use (and carry) instead of the cached one of
    this device and stream: a DecodeWorkspace, or a zero-filled uint8 tensor
    (the caller then keeps its tag count below 2^32; see decode_tags).
    check: synchronise after the call and raise if the kernel recorded a
    failed exchange (a grid that could not make progress) since the
    workspace's count was last read; with check=False the caller reads
    DecodeWorkspace.new_failures() itself.
    """
    T, d_model, L, d_ff, shape, wts = _stack_args(q, layers, k, r)
    need = ctypes.c_size_t(0)
    _check(lib().spark_ffn_decode_workspace_size(ctypes.byref(shape), L, T, ctypes.byref(need)),
           "spark_ffn_decode_workspace_size")
    dev = q.device
    if ws is None:
        ws = _decode_workspace(dev, need.value)
    elif isinstance(ws, torch.Tensor):
        ws = DecodeWorkspace(ws)
    if ws.reserve(decode_tags(L, T)):
        ws.buf.zero_()
        ws.failures_seen = 0
    y = torch.empty((T, d_model), dtype=torch.float32, device=dev)
    tr = None
    trc = None
    if trace:
        tr, trc = _trace_buffers(T, L, d_ff, d_model, cap, dev)
    st = lib().spark_ffn_decode(ctypes.byref(shape), wts, L, _p(q), T, _p(y), float(eps),
                                ctypes.byref(trc) if trc is not None else None, _p(ws.buf), ws.buf.numel(),
                                _stream(dev))
    _check(st, "spark_ffn_decode")
    if check and ws.new_failures():
        raise RuntimeError("spark_ffn_decode: a grid-wide exchange timed out (the device could not keep the "
                           "whole grid running); the output holds NaN")
    return (y, tr) if trace else y


def spark_ffn_decode_noalloc(q: torch.Tensor, layers, k: int, r: int, eps: float = 1e-6, trace: bool = False,
                             cap: int | None = None):
    """spark_ffn_decode through the entry point that allocates nothing on the
    device: the library's own per-device scratch array replaces the workspace
    (calls on one device must not overlap).  Same arguments and results as
    spark_ffn_decode; this wrapper allocates only the outputs."""
    T, d_model, L, d_ff, shape, wts = _stack_args(q, layers, k, r)
    dev = q.device
    y = torch.empty((T, d_model), dtype=torch.float32, device=dev)
    tr, trc = _trace_buffers(T, L, d_ff, d_model, cap, dev) if trace else (None, None)
    st = lib().spark_ffn_decode_noalloc(ctypes.byref(shape), wts, L, _p(q), T, _p(y), float(eps),
                                        ctypes.byref(trc) if trc is not None else None, _stream(dev))
    _check(st, "spark_ffn_decode_noalloc")
    return (y, tr) if trace else y


def spark_ffn_decode_batched(q: torch.Tensor, layers, k: int, r: int, eps: float = 1e-6, trace: bool = False,
                             cap: int | None = None, ws: torch.Tensor | TaggedWorkspace | None = None,
                             check: bool = True):
    """The computation of spark_ffn_decode for a batch of B <= 8 tokens, run
    layer by layer for the whole batch (one K1 read per layer, K2 and V rows
    read once for all the tokens that select them).  Same arguments, results
    and trace as spark_ffn_decode with T = B.  ws: optional workspace to use
    (and carry) instead of the cached one of this device and stream (a
    TaggedWorkspace or a zero-filled uint8 tensor).  check: synchronise and
    raise if a grid-wide exchange timed out."""
    B, d_model, L, d_ff, shape, wts = _stack_args(q, layers, k, r)
    need = ctypes.c_size_t(0)
    _check(lib().spark_ffn_decode_batched_workspace_size(ctypes.byref(shape), B, ctypes.byref(need)),
           "spark_ffn_decode_batched_workspace_size")
    dev = q.device
    if ws is None:
        ws = _tagged_workspace("decode_batched", dev, need.value)
    elif isinstance(ws, torch.Tensor):
        ws = TaggedWorkspace(ws)
    # a batched call uses the exchange tags of one single-token call
    if ws.reserve(decode_tags(L, 1)):
        ws.buf.zero_()
        ws.failures_seen = 0
    y = torch.empty((B, d_model), dtype=torch.float32, device=dev)
    tr, trc = _trace_buffers(B, L, d_ff, d_model, cap, dev) if trace else (None, None)
    st = lib().spark_ffn_decode_batched(ctypes.byref(shape), wts, L, _p(q), B, _p(y), float(eps),
                                        ctypes.byref(trc) if trc is not None else None, _p(ws.buf), ws.buf.numel(),
                                        _stream(dev))
    _check(st, "spark_ffn_decode_batched")
    if check and ws.new_failures():
        raise RuntimeError("spark_ffn_decode_batched: a grid-wide exchange timed out (the device could not keep "
                           "the whole grid running); the output holds NaN")
    return (y, tr) if trace else y


def decode_workspace_failed(ws: torch.Tensor | DecodeWorkspace | None = None, device=None) -> bool:
    """True if a decode kernel that used this workspace (by default the cached
    one of the device and its current stream) recorded a failed call (reads
    the workspace header; synchronises)."""
    if ws is None:
        ws = _ws_cache.get(_ws_key("decode", device or torch.device("cuda", torch.cuda.current_device())))
        if ws is None:
            return False
    buf = ws.buf if isinstance(ws, DecodeWorkspace) else ws
    return int(buf[16:24].view(torch.int64).item()) != 0


# ---------------------------------------------------------------------------- prefill
def spark_ffn_prefill(Q: torch.Tensor, layer, k: int, r: int, trace: bool = False, cap: int | None = None,
                      gathered: bool = False):
    """One Spark FFN layer on T tokens at once.  Q [T][d_model] bf16; layer =
    (k1t, k2t, v) bf16.  Returns Y [T][d_model] fp32 (and with trace=True a dict
    with counts [T], idx [T][cap], theta [T]).  gathered=True runs
    spark_ffn_prefill_gathered (only the selected K2 and V rows are read)."""
    _need_cuda(Q, *layer)
    if Q.dim() != 2:
        raise ValueError("Q must be [T][d_model]")
    T, d_model = Q.shape
    k1t, k2t, v = layer
    d_ff = v.shape[0]
    wd = _wdtype(k1t)
    if Q.dtype != k1t.dtype or any(a.dtype != k1t.dtype for a in layer):
        raise TypeError("Q and the weights must share one dtype")
    if k1t.shape != (d_ff, r) or k2t.shape != (d_ff, d_model - r) or v.shape != (d_ff, d_model):
        raise ValueError("weight shapes do not match Q / r: need k1t [d_ff][r], k2t [d_ff][d_model-r], "
                         "v [d_ff][d_model]")
    shape = _shape(d_model, d_ff, r, k, wd)
    w = WeightsC(k1t.data_ptr(), k2t.data_ptr(), v.data_ptr())
    need = ctypes.c_size_t(0)
    size_fn = lib().spark_ffn_prefill_gathered_workspace_size if gathered else lib().spark_ffn_prefill_workspace_size
    _check(size_fn(ctypes.byref(shape), T, ctypes.byref(need)), "prefill workspace size")
    dev = Q.device
    ws = _cached_workspace("prefill_gathered" if gathered else "prefill", dev, need.value)
    Y = torch.empty((T, d_model), dtype=torch.float32, device=dev)
    tr = None
    trc = None
    if trace:
        cap = d_ff if cap is None else int(cap)
        tr = dict(counts=torch.zeros((T, 1), dtype=torch.int32, device=dev),
                  idx=torch.full((T, 1, cap), -1, dtype=torch.int32, device=dev),
                  theta=torch.zeros((T, 1), dtype=torch.float32, device=dev))
        trc = TraceC(tr["counts"].data_ptr(), tr["idx"].data_ptr(), tr["theta"].data_ptr(), None, cap)
    fn = lib().spark_ffn_prefill_gathered if gathered else lib().spark_ffn_prefill
    st = fn(ctypes.byref(shape), ctypes.byref(w), _p(Q), T, _p(Y), ctypes.byref(trc) if trc is not None else None,
            _p(ws), ws.numel(), _stream(dev))
    _check(st, "spark_ffn_prefill_gathered" if gathered else "spark_ffn_prefill")
    return (Y, tr) if trace else Y


def spark_ffn_prefill_scores(Q: torch.Tensor, layer, r: int) -> torch.Tensor:
    """The predictor step of the prefill alone: H [T][d_ff] fp32 = Q[:, :r] K1."""
    _need_cuda(Q, *layer)
    T, d_model = Q.shape
    k1t = layer[0]
    d_ff = k1t.shape[0]
    if k1t.shape != (d_ff, r) or Q.dtype != torch.bfloat16 or k1t.dtype != torch.bfloat16:
        raise ValueError("need bf16 Q [T][d_model] and k1t [d_ff][r]")
    shape = _shape(d_model, d_ff, r, 1, SPARK_BF16)
    w = WeightsC(k1t.data_ptr(), layer[1].data_ptr(), layer[2].data_ptr())
    H = torch.empty((T, d_ff), dtype=torch.float32, device=Q.device)
    _check(lib().spark_ffn_prefill_scores(ctypes.byref(shape), ctypes.byref(w), _p(Q), T, _p(H), _stream(Q.device)),
           "spark_ffn_prefill_scores")
    return H


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream every byte of buf (a measurement helper; see the header)."""
    _check(lib().spark_hbm_read_probe(_p(buf), buf.numel() * buf.element_size(), _p(sink), _stream(buf.device)),
           "spark_hbm_read_probe")


# ---------------------------------------------------------------------------- attention
def spark_attn_decode(q: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor, v: torch.Tensor, k_attn: int,
                      cap: int | None = None):
    """Spark attention decode.  q [Hq][hd] bf16; k1 [Hkv][n][r], k2 [Hkv][n][hd-r],
    v [Hkv][n][hd] bf16.  Returns out [Hq][hd] fp32, counts [Hq], idx [Hq][cap]
    (ascending selected tokens; -1 padded) and theta [Hq] (NaN when dense)."""
    _need_cuda(q, k1, k2, v)
    for t in (q, k1, k2, v):
        if t.dtype != torch.bfloat16:
            raise TypeError("attention inputs must be bf16")
    if q.dim() != 2 or k1.dim() != 3:
        raise ValueError("q must be [Hq][hd] and k1 [Hkv][n_ctx][r]")
    Hq, hd = q.shape
    Hkv, n, r = k1.shape
    if k2.shape != (Hkv, n, hd - r) or v.shape != (Hkv, n, hd):
        raise ValueError("cache shapes do not match: need k2 [Hkv][n_ctx][hd-r], v [Hkv][n_ctx][hd]")
    cap = min(n, 4096) if cap is None else int(cap)
    need = ctypes.c_size_t(0)
    _check(lib().spark_attn_workspace_size(Hq, Hkv, n, hd, r, int(k_attn), ctypes.byref(need)),
           "spark_attn_workspace_size")
    dev = q.device
    ws = _cached_workspace("attn", dev, need.value)
    out = torch.empty((Hq, hd), dtype=torch.float32, device=dev)
    counts = torch.empty(Hq, dtype=torch.int32, device=dev)
    idx = torch.full((Hq, max(cap, 1)), -1, dtype=torch.int32, device=dev)
    theta = torch.empty(Hq, dtype=torch.float32, device=dev)
    st = lib().spark_attn_decode(_p(q), _p(k1), _p(k2), _p(v), Hq, Hkv, n, hd, r, int(k_attn), _p(out), _p(counts),
                                 _p(idx), cap, _p(theta), _p(ws), ws.numel(), _stream(dev))
    _check(st, "spark_attn_decode")
    return out, counts, idx, theta


def spark_attn_prefill(q: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor, v: torch.Tensor, k_attn: int,
                       cap: int = 0):
    """Causal Spark attention over a prompt.  q [T][Hq][hd] bf16; k1 [Hkv][T][r],
    k2 [Hkv][T][hd-r], v [Hkv][T][hd] bf16.  Returns out [T][Hq][hd] fp32,
    counts [T][Hq], idx [T][Hq][cap] (the attended positions of each row,
    ascending, -1 padded; None when cap = 0) and theta [T][Hq] (NaN where
    t + 1 <= k_attn)."""
    _need_cuda(q, k1, k2, v)
    for t in (q, k1, k2, v):
        if t.dtype != torch.bfloat16:
            raise TypeError("attention inputs must be bf16")
    if q.dim() != 3 or k1.dim() != 3:
        raise ValueError("q must be [T][Hq][hd] and k1 [Hkv][T][r]")
    T, Hq, hd = q.shape
    Hkv, n, r = k1.shape
    if n != T:
        raise ValueError("the cache must hold the T prompt positions")
    if k2.shape != (Hkv, T, hd - r) or v.shape != (Hkv, T, hd):
        raise ValueError("cache shapes do not match: need k2 [Hkv][T][hd-r], v [Hkv][T][hd]")
    cap = int(cap)
    need = ctypes.c_size_t(0)
    _check(lib().spark_attn_prefill_workspace_size(T, Hq, Hkv, hd, r, int(k_attn), cap, ctypes.byref(need)),
           "spark_attn_prefill_workspace_size")
    dev = q.device
    ws = _cached_workspace("attn_prefill", dev, need.value)
    out = torch.empty((T, Hq, hd), dtype=torch.float32, device=dev)
    counts = torch.empty((T, Hq), dtype=torch.int32, device=dev)
    theta = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((T, Hq, cap), dtype=torch.int32, device=dev) if cap > 0 else None
    st = lib().spark_attn_prefill(_p(q), _p(k1), _p(k2), _p(v), T, Hq, Hkv, hd, r, int(k_attn), _p(out), _p(counts),
                                  _p(idx), cap, _p(theta), _p(ws), ws.numel(), _stream(dev))
    _check(st, "spark_attn_prefill")
    return out, counts, idx, theta
