"""Python binding of ``libglahybrid.so`` (C ABI in ``include/glahybrid.h``).

Argument marshalling only: each function checks its tensors (shapes, element
types, dense row-major layout, one device: the C boundary sees only
addresses and could not), reads the sizes into the ``glah_desc`` descriptor,
passes raw device pointers and the current HIP stream, and raises
:class:`GlahError` on a non-zero status.  Every step of the
layer runs in the library's HIP kernels; torch only provides device memory
(outputs and workspace are allocated with ``torch.empty`` when not given) and
the stream.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libglahybrid.so")

GLAH_OK, GLAH_EINVAL, GLAH_ENOTSUP, GLAH_EWORKSPACE, GLAH_EHIP = range(5)
GLAH_BF16, GLAH_F32 = 0, 1
GLAH_GATE_LOGITS, GLAH_GATE_LOG = 0, 1
GLAH_GATE_LOG_TOKEN, GLAH_GATE_LOG_HEAD = 2, 3  # scalar log-gates: [B,H,L] per token, [H] per head

EXPORTS = ("glah_status_str", "glah_version", "glah_workspace_bytes", "gla_prefill",
           "swa_meta_attn", "hybrid_layer_fwd", "gla_decode_step", "glah_bwd_workspace_bytes",
           "hybrid_layer_bwd", "gdn_prefill", "gdn_decode_step", "hybrid_layer_fwd_cont",
           "glah_output_gate", "hybrid_layer_fwd_noalloc", "gdn_workspace_bytes")


class GlahError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


class GlahDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("f", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("window", ctypes.c_int32), ("n_meta", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("gate_kind", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def load(path: str = LIBRARY):
    """Load the HIP library (raises when it is missing: there is no fallback)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                raise RuntimeError("libglahybrid.so is not built (run __graft_entry__.build() or "
                                   "python -m gated_linear_attention_hybrid_amd.build_lib)")
            lib = ctypes.CDLL(path)
            vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
            dp = ctypes.POINTER(GlahDesc)
            lib.glah_status_str.argtypes = [i32]
            lib.glah_status_str.restype = ctypes.c_char_p
            lib.glah_version.restype = i32
            lib.glah_workspace_bytes.argtypes = [dp]
            lib.glah_workspace_bytes.restype = sz
            lib.gla_prefill.argtypes = [dp] + [vp] * 9 + [vp, sz, vp]
            lib.gla_prefill.restype = i32
            lib.swa_meta_attn.argtypes = [dp] + [vp] * 5 + [vp]
            lib.swa_meta_attn.restype = i32
            lib.hybrid_layer_fwd.argtypes = [dp] + [vp] * 12 + [vp, sz, vp]
            lib.hybrid_layer_fwd.restype = i32
            lib.hybrid_layer_fwd_noalloc.argtypes = [dp] + [vp] * 12 + [vp]
            lib.hybrid_layer_fwd_noalloc.restype = i32
            lib.gla_decode_step.argtypes = [dp] + [vp] * 12 + [vp]
            lib.gla_decode_step.restype = i32
            lib.glah_bwd_workspace_bytes.argtypes = [dp]
            lib.glah_bwd_workspace_bytes.restype = sz
            lib.glah_bwd_workspace_bytes_whole.argtypes = [dp]
            lib.glah_bwd_workspace_bytes_whole.restype = sz
            lib.hybrid_layer_bwd.argtypes = [dp] + [vp] * 18 + [vp, sz, vp]
            lib.hybrid_layer_bwd.restype = i32
            lib.hybrid_layer_fwd_cont.argtypes = [dp, ctypes.c_int32] + [vp] * 15 + [sz, vp]
            lib.hybrid_layer_fwd_cont.restype = i32
            lib.glah_output_gate.argtypes = [dp, vp, vp, vp]
            lib.glah_output_gate.restype = i32
            lib.gdn_prefill.argtypes = [dp] + [vp] * 8 + [vp, sz, vp]
            lib.gdn_workspace_bytes.argtypes = [dp]
            lib.gdn_workspace_bytes.restype = sz
            lib.gdn_prefill.restype = i32
            lib.gdn_decode_step.argtypes = [dp] + [vp] * 7 + [vp]
            lib.gdn_decode_step.restype = i32
            _lib = lib
    return _lib


def _check(fn, status):
    if status != GLAH_OK:
        raise GlahError(fn, status, load().glah_status_str(status).decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class _Checked:
    """Checks of the tensor arguments of one call before their pointers cross
    the C boundary, which sees only addresses: each tensor's shape, element
    type and dense row-major layout as it is named (``need``), then, once all
    of those hold, that every tensor is on the same GPU (``on_device``).
    Raises TypeError / ValueError."""

    def __init__(self):
        self.seen = []

    def need(self, name, t, shape, dtype, optional=False):
        if t is None:
            if optional:
                return None
            raise ValueError("%s is required" % name)
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor, got %s" % (name, type(t).__name__))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
        if t.dtype != dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous (dense row-major)" % name)
        self.seen.append((name, t))
        return t

    def on_device(self, device):
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError("%s must be a GPU tensor, got device %s" % (name, t.device))
            if t.device != device:
                raise ValueError("%s is on %s, the other arguments on %s" % (name, t.device, device))


def _gate_shape(kind, B, H, L, f):
    """Shape of the gate tensor for gate layout ``kind`` (L = None: decode)."""
    tok = (B, H) if L is None else (B, H, L)
    if kind in (GLAH_GATE_LOGITS, GLAH_GATE_LOG):
        return tok + (f,)
    if kind == GLAH_GATE_LOG_TOKEN:
        return tok
    if kind == GLAH_GATE_LOG_HEAD:
        return (H,)
    raise ValueError("unknown gate kind %r" % (kind,))


def _kind(gate_is_log, gate_kind):
    return gate_kind if gate_kind is not None else (GLAH_GATE_LOG if gate_is_log else GLAH_GATE_LOGITS)


def _layer_args(ck, q, k, v, wq, wk, meta, gate=None, kind=GLAH_GATE_LOGITS, with_gla=True):
    """Check the inputs shared by the layer entry points (into ``ck``);
    returns (B, H, L, d, dv, f, n_meta)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a [B, H, L, d] tensor")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32, got %s" % q.dtype)
    B, H, L, d = q.shape
    dt = q.dtype
    ck.need("q", q, (B, H, L, d), dt)
    ck.need("k", k, (B, H, L, d), dt)
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a [B, H, L, d_v] tensor")
    dv = v.shape[-1]
    ck.need("v", v, (B, H, L, dv), dt)
    f = 0
    if with_gla:
        if not isinstance(wq, torch.Tensor) or wq.dim() != 3:
            raise ValueError("wq must be a [H, d, f/2] tensor")
        f = 2 * wq.shape[-1]
        ck.need("wq", wq, (H, d, f // 2), dt)
        ck.need("wk", wk, (H, d, f // 2), dt)
        ck.need("gate", gate, _gate_shape(kind, B, H, L, f), dt)
    n_meta = _meta(ck, meta, H)
    return B, H, L, d, dv, f, n_meta


def _meta(ck, meta, H):
    """Check the optional [H, n_meta] fp32 sink logits; returns n_meta."""
    if meta is None:
        return 0
    if not isinstance(meta, torch.Tensor) or meta.dim() != 2:
        raise ValueError("meta must be a [H, n_meta] tensor")
    ck.need("meta", meta, (H, meta.shape[-1]), torch.float32)
    return meta.shape[-1]


def _rings(ck, q, B, H, window, d, dv, **named):
    """Window ring tensors (optional) [B,H,window,d|dv] in q's dtype."""
    for name, t in named.items():
        width = d if name.startswith("k") else dv
        ck.need(name, t, (B, H, max(int(window), 0), width), q.dtype, optional=True)


def _states(ck, shape, **named):
    """fp32 state tensors (optional) of the given shape."""
    for name, t in named.items():
        ck.need(name, t, shape, torch.float32, optional=True)


def _out(ck, name, t, shape, like, dtype=None):
    """An output tensor: checked like an input when given (allocated by the
    caller of this after the device check when None)."""
    dtype = like.dtype if dtype is None else dtype
    if t is not None:
        ck.need(name, t, shape, dtype)
    return t


def _alloc(t, shape, like, dtype=None):
    return torch.empty(shape, dtype=like.dtype if dtype is None else dtype, device=like.device) if t is None else t


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return GLAH_BF16
    if t.dtype == torch.float32:
        return GLAH_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def make_desc(B, H, L, d, dv, f, *, window=0, n_meta=0, chunk=0, scale=0.0, dtype=GLAH_BF16,
              gate_is_log=False, gate_kind=None) -> GlahDesc:
    return GlahDesc(B, H, L, d, dv, f, chunk, window, n_meta, float(scale or 0.0), dtype,
                    gate_kind if gate_kind is not None else
                    (GLAH_GATE_LOG if gate_is_log else GLAH_GATE_LOGITS))


def workspace_bytes(desc: GlahDesc) -> int:
    n = load().glah_workspace_bytes(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise GlahError("glah_workspace_bytes", GLAH_EINVAL, "invalid argument")
    return n


def _workspace(desc, ws, device, need=None):
    n = workspace_bytes(desc) if need is None else need
    if ws is None and n:
        ws = torch.empty(n, dtype=torch.uint8, device=device)
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or not ws.is_contiguous() or ws.device != device:
            raise ValueError("ws must be a contiguous tensor on %s" % device)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def gla_prefill(q, k, v, gate, wq, wk, *, chunk=0, gate_is_log=False, gate_kind=None, state_in=None,
                state_out=None, o=None, ws=None, stream=None):
    """Gated linear attention prefill; returns o [B,H,L,dv]."""
    ck, kind = _Checked(), _kind(gate_is_log, gate_kind)
    B, H, L, d, dv, f, _ = _layer_args(ck, q, k, v, wq, wk, None, gate, kind)
    _states(ck, (B, H, f, dv), state_in=state_in, state_out=state_out)
    _out(ck, "o", o, (B, H, L, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, f, chunk=chunk, dtype=_dtype_code(q), gate_kind=kind)
    o = _alloc(o, (B, H, L, dv), q)
    ws, nbytes = _workspace(desc, ws, q.device)
    st = load().gla_prefill(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(gate), _p(wq), _p(wk),
                            _p(state_in), _p(state_out), _p(o), _p(ws), nbytes, _stream(stream))
    _check("gla_prefill", st)
    return o


def swa_meta_attn(q, k, v, meta, *, window, scale=0.0, o=None, stream=None):
    """Sliding-window attention with meta-memory sinks; returns o [B,H,L,dv]."""
    ck = _Checked()
    B, H, L, d, dv, _, n_meta = _layer_args(ck, q, k, v, None, None, meta, with_gla=False)
    _out(ck, "o", o, (B, H, L, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, 2, window=window, n_meta=n_meta, scale=scale,
                     dtype=_dtype_code(q))
    o = _alloc(o, (B, H, L, dv), q)
    st = load().swa_meta_attn(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(meta), _p(o),
                              _stream(stream))
    _check("swa_meta_attn", st)
    return o


def hybrid_layer_fwd(q, k, v, gate, wq, wk, meta, *, window, chunk=0, scale=0.0,
                     gate_is_log=False, gate_kind=None, state_in=None, state_out=None, kcache_out=None,
                     vcache_out=None, o=None, ws=None, stream=None):
    """Whole hybrid layer (gated linear + window attention); returns o [B,H,L,dv]."""
    ck, kind = _Checked(), _kind(gate_is_log, gate_kind)
    B, H, L, d, dv, f, n_meta = _layer_args(ck, q, k, v, wq, wk, meta, gate, kind)
    _states(ck, (B, H, f, dv), state_in=state_in, state_out=state_out)
    _rings(ck, q, B, H, window, d, dv, kcache_out=kcache_out, vcache_out=vcache_out)
    _out(ck, "o", o, (B, H, L, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, f, window=window, n_meta=n_meta, chunk=chunk, scale=scale,
                     dtype=_dtype_code(q), gate_kind=kind)
    o = _alloc(o, (B, H, L, dv), q)
    ws, nbytes = _workspace(desc, ws, q.device)
    st = load().hybrid_layer_fwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(gate), _p(wq),
                                 _p(wk), _p(meta), _p(state_in), _p(state_out), _p(kcache_out),
                                 _p(vcache_out), _p(o), _p(ws), nbytes, _stream(stream))
    _check("hybrid_layer_fwd", st)
    return o


def hybrid_layer_fwd_noalloc(q, k, v, gate, wq, wk, meta, o, *, window, chunk=0, scale=0.0,
                             gate_is_log=False, gate_kind=None, state_in=None, state_out=None,
                             kcache_out=None, vcache_out=None, stream=None):
    """hybrid_layer_fwd without a workspace (the library's per-device scratch
    array holds the segment states): the caller passes the output ``o``
    [B,H,L,dv], so neither this function nor the library allocates.  Calls that
    overlap on one device race on the scratch array; returns o."""
    ck, kind = _Checked(), _kind(gate_is_log, gate_kind)
    B, H, L, d, dv, f, n_meta = _layer_args(ck, q, k, v, wq, wk, meta, gate, kind)
    _states(ck, (B, H, f, dv), state_in=state_in, state_out=state_out)
    _rings(ck, q, B, H, window, d, dv, kcache_out=kcache_out, vcache_out=vcache_out)
    ck.need("o", o, (B, H, L, dv), q.dtype)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, f, window=window, n_meta=n_meta, chunk=chunk, scale=scale,
                     dtype=_dtype_code(q), gate_kind=kind)
    st = load().hybrid_layer_fwd_noalloc(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(gate), _p(wq), _p(wk),
                                         _p(meta), _p(state_in), _p(state_out), _p(kcache_out),
                                         _p(vcache_out), _p(o), _stream(stream))
    _check("hybrid_layer_fwd_noalloc", st)
    return o


def hybrid_layer_fwd_cont(q, k, v, gate, wq, wk, meta, *, window, start, state_in=None, kcache_in=None,
                          vcache_in=None, state_out=None, kcache_out=None, vcache_out=None, chunk=0, scale=0.0,
                          gate_is_log=False, gate_kind=None, o=None, ws=None, stream=None):
    """Hybrid layer over tokens start .. start+L-1 of sequences that already
    consumed ``start`` tokens (state and window ring of the previous call in,
    optionally the new ones out); returns o [B,H,L,dv]."""
    ck, kind = _Checked(), _kind(gate_is_log, gate_kind)
    B, H, L, d, dv, f, n_meta = _layer_args(ck, q, k, v, wq, wk, meta, gate, kind)
    _states(ck, (B, H, f, dv), state_in=state_in, state_out=state_out)
    _rings(ck, q, B, H, window, d, dv, kcache_in=kcache_in, vcache_in=vcache_in, kcache_out=kcache_out,
           vcache_out=vcache_out)
    _out(ck, "o", o, (B, H, L, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, f, window=window, n_meta=n_meta, chunk=chunk, scale=scale,
                     dtype=_dtype_code(q), gate_kind=kind)
    o = _alloc(o, (B, H, L, dv), q)
    ws, nbytes = _workspace(desc, ws, q.device)
    st = load().hybrid_layer_fwd_cont(ctypes.byref(desc), int(start), _p(q), _p(k), _p(v), _p(gate), _p(wq),
                                      _p(wk), _p(meta), _p(state_in), _p(kcache_in), _p(vcache_in),
                                      _p(state_out), _p(kcache_out), _p(vcache_out), _p(o), _p(ws), nbytes,
                                      _stream(stream))
    _check("hybrid_layer_fwd_cont", st)
    return o


def output_gate(o, g, *, stream=None):
    """o <- o * sigmoid(g) in place (o, g [B,H,L,dv], the same dtype); returns o."""
    if not isinstance(o, torch.Tensor) or o.dim() != 4:
        raise ValueError("o must be a [B, H, L, d_v] tensor")
    dtype = _dtype_code(o)
    B, H, L, dv = o.shape
    ck = _Checked()
    ck.need("o", o, (B, H, L, dv), o.dtype)
    ck.need("g", g, (B, H, L, dv), o.dtype)
    ck.on_device(o.device)
    desc = make_desc(B, H, L, 1, dv, 2, dtype=dtype)
    st = load().glah_output_gate(ctypes.byref(desc), _p(o), _p(g), _stream(stream))
    _check("glah_output_gate", st)
    return o


def _token_args(ck, q, k, v):
    """Check the one-token q, k [B,H,d] and v [B,H,dv]; returns (B, H, d, dv)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B, H, d] tensor")
    if not isinstance(v, torch.Tensor) or v.dim() != 3:
        raise ValueError("v must be a [B, H, d_v] tensor")
    _dtype_code(q)
    B, H, d = q.shape
    dv = v.shape[-1]
    ck.need("q", q, (B, H, d), q.dtype)
    ck.need("k", k, (B, H, d), q.dtype)
    ck.need("v", v, (B, H, dv), q.dtype)
    return B, H, d, dv


def gla_decode_step(q, k, v, gate, wq, wk, meta, state, kcache, vcache, pos, *, window,
                    scale=0.0, gate_is_log=False, gate_kind=None, o=None, stream=None):
    """One decode step (state and ring updated in place); returns o [B,H,dv].
    ``pos`` is a device int32 tensor [B] of tokens already consumed."""
    ck, kind = _Checked(), _kind(gate_is_log, gate_kind)
    B, H, d, dv = _token_args(ck, q, k, v)
    if not isinstance(wq, torch.Tensor) or wq.dim() != 3:
        raise ValueError("wq must be a [H, d, f/2] tensor")
    f = 2 * wq.shape[-1]
    ck.need("gate", gate, _gate_shape(kind, B, H, None, f), q.dtype)
    ck.need("wq", wq, (H, d, f // 2), q.dtype)
    ck.need("wk", wk, (H, d, f // 2), q.dtype)
    n_meta = _meta(ck, meta, H)
    ck.need("state", state, (B, H, f, dv), torch.float32)
    _rings(ck, q, B, H, window, d, dv, kcache=kcache, vcache=vcache)
    ck.need("pos", pos, (B,), torch.int32)
    _out(ck, "o", o, (B, H, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, 1, d, dv, f, window=window, n_meta=n_meta, scale=scale,
                     dtype=_dtype_code(q), gate_kind=kind)
    o = _alloc(o, (B, H, dv), q)
    st = load().gla_decode_step(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(gate), _p(wq), _p(wk),
                                _p(meta), _p(state), _p(kcache), _p(vcache), _p(pos), _p(o),
                                _stream(stream))
    _check("gla_decode_step", st)
    return o


def bwd_workspace_bytes(desc: GlahDesc) -> int:
    n = load().glah_bwd_workspace_bytes(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise GlahError("glah_bwd_workspace_bytes", GLAH_EINVAL, "invalid argument")
    return n


def bwd_workspace_bytes_whole(desc: GlahDesc) -> int:
    """Workspace with which hybrid_layer_bwd runs the whole call at once."""
    n = load().glah_bwd_workspace_bytes_whole(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise GlahError("glah_bwd_workspace_bytes_whole", GLAH_EINVAL, "invalid argument")
    return n


def hybrid_layer_bwd(q, k, v, gate, wq, wk, meta, d_o, *, window, scale=0.0, gate_is_log=False,
                     gate_kind=None, state_in=None, dstate_out=None, need_dstate_in=False, ws=None,
                     stream=None):
    """Gradient of hybrid_layer_fwd for the loss sum(o * d_o) + sum(S_final * dstate_out).

    Returns a dict with the gradients named as the forward's inputs: q, k, v,
    gate (the gate's layout and dtype), wq, wk ([H,d,f/2] fp32), meta ([H,M]
    fp32, None without sinks) and state_in ([B,H,f,dv] fp32, when
    ``need_dstate_in``)."""
    ck, kind = _Checked(), _kind(gate_is_log, gate_kind)
    B, H, L, d, dv, f, n_meta = _layer_args(ck, q, k, v, wq, wk, meta, gate, kind)
    ck.need("d_o", d_o, (B, H, L, dv), q.dtype)
    _states(ck, (B, H, f, dv), state_in=state_in, dstate_out=dstate_out)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, f, window=window, n_meta=n_meta, scale=scale,
                     dtype=_dtype_code(q), gate_kind=kind)
    dev = q.device
    out = dict(q=torch.empty_like(q), k=torch.empty_like(k), v=torch.empty_like(v),
               gate=torch.empty_like(gate),
               wq=torch.empty(wq.shape, dtype=torch.float32, device=dev),
               wk=torch.empty(wk.shape, dtype=torch.float32, device=dev),
               meta=None if meta is None else torch.empty(meta.shape, dtype=torch.float32, device=dev),
               state_in=(torch.empty((B, H, f, dv), dtype=torch.float32, device=dev)
                         if need_dstate_in else None))
    ws, nbytes = _workspace(desc, ws, dev, need=bwd_workspace_bytes(desc))
    st = load().hybrid_layer_bwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(gate), _p(wq), _p(wk),
                                 _p(meta), _p(state_in), _p(d_o), _p(dstate_out), _p(out["q"]),
                                 _p(out["k"]), _p(out["v"]), _p(out["gate"]), _p(out["wq"]),
                                 _p(out["wk"]), _p(out["meta"]), _p(out["state_in"]), _p(ws), nbytes,
                                 _stream(stream))
    _check("hybrid_layer_bwd", st)
    return out


def gdn_workspace_bytes(desc: GlahDesc) -> int:
    n = load().gdn_workspace_bytes(ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise GlahError("gdn_workspace_bytes", GLAH_EINVAL, "invalid argument")
    return n


def gdn_prefill(q, k, v, log_alpha, beta, *, state_in=None, state_out=None, o=None, ws=None, stream=None):
    """Gated delta rule over whole sequences; returns o [B,H,L,dv].  q, k
    [B,H,L,d], v [B,H,L,dv], log_alpha and beta [B,H,L] (the dtype of q); states
    [B,H,dv,d] fp32; ws a uint8 device buffer of at least gdn_workspace_bytes
    (allocated here when None)."""
    ck = _Checked()
    B, H, L, d, dv, _, _ = _layer_args(ck, q, k, v, None, None, None, with_gla=False)
    ck.need("log_alpha", log_alpha, (B, H, L), q.dtype)
    ck.need("beta", beta, (B, H, L), q.dtype)
    _states(ck, (B, H, dv, d), state_in=state_in, state_out=state_out)
    _out(ck, "o", o, (B, H, L, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, L, d, dv, d, dtype=_dtype_code(q))
    ws, nbytes = _workspace(desc, ws, q.device, need=gdn_workspace_bytes(desc))
    o = _alloc(o, (B, H, L, dv), q)
    st = load().gdn_prefill(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(log_alpha), _p(beta),
                            _p(state_in), _p(state_out), _p(o), _p(ws), nbytes, _stream(stream))
    _check("gdn_prefill", st)
    return o


def gdn_decode_step(q, k, v, log_alpha, beta, state, *, o=None, stream=None):
    """One gated delta rule token (state [B,H,dv,d] fp32 updated in place);
    returns o [B,H,dv]."""
    ck = _Checked()
    B, H, d, dv = _token_args(ck, q, k, v)
    ck.need("log_alpha", log_alpha, (B, H), q.dtype)
    ck.need("beta", beta, (B, H), q.dtype)
    ck.need("state", state, (B, H, dv, d), torch.float32)
    _out(ck, "o", o, (B, H, dv), q)
    ck.on_device(q.device)
    desc = make_desc(B, H, 1, d, dv, d, dtype=_dtype_code(q))
    o = _alloc(o, (B, H, dv), q)
    st = load().gdn_decode_step(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(log_alpha), _p(beta),
                                _p(state), _p(o), _stream(stream))
    _check("gdn_decode_step", st)
    return o
