"""ctypes binding of ``libgdn_stream.so`` (C ABI in include/gdn_stream.h and include/gdn_attn.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  The
functions carry the C names; ``Stream`` is a small convenience wrapper.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libgdn_stream.so")

GDN_OK = 0
GDN_E_INVAL, GDN_E_SHAPE, GDN_E_DTYPE, GDN_E_NOMEM, GDN_E_HIP = -1, -2, -3, -4, -5
GDN_BF16, GDN_F32 = 0, 1
GDN_L2NORM_QK = 1 << 0
GDN_GATE_IS_LOG = 1 << 1
GDN_POISON_WS = 1 << 2
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20
GDN_NO_COMMIT = 1 << 0
GDN_SEQUENTIAL = 1 << 1
GDN_KERNEL_PREP, GDN_KERNEL_SCAN, GDN_KERNEL_SEQ, GDN_KERNEL_BWD, GDN_KERNEL_COUNT = 0, 1, 2, 3, 4
KERNEL_NAMES = ("prep", "scan", "sequential", "backward")


class GdnConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("max_tokens", ctypes.c_int64), ("subchunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("l2_eps", ctypes.c_float),
                ("scale", ctypes.c_float)]


_Strides = ctypes.c_int64 * 3


class GdnIo(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("a", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("q_strides", _Strides), ("k_strides", _Strides), ("v_strides", _Strides),
                ("o_strides", _Strides), ("g_strides", _Strides)]


class GdnGrad(ctypes.Structure):
    _fields_ = [("d_o", ctypes.c_void_p), ("d_state", ctypes.c_void_p), ("state0", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("da", ctypes.c_void_p), ("dbeta", ctypes.c_void_p), ("d_state0", ctypes.c_void_p)]


class GdnAttnConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("window_tokens", ctypes.c_int32), ("max_tokens", ctypes.c_int64),
                ("scale", ctypes.c_float)]


class GdnAttnIo(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("o", ctypes.c_void_p),
                ("q_strides", _Strides), ("k_strides", _Strides), ("v_strides", _Strides), ("o_strides", _Strides)]


class GdnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"gdn error {code}: {msg}")
        self.code = code


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m gated_deltanet_streaming_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, u32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int
    sigs = {
        "gdn_stream_init": ([ctypes.POINTER(GdnConfig), i32, ctypes.POINTER(vp)], i32),
        "gdn_stream_destroy": ([vp], i32),
        "gdn_chunk_forward": ([vp, ctypes.POINTER(GdnIo), i64, u32, vp, vp], i32),
        "gdn_chunk_forward_split": ([vp, ctypes.POINTER(GdnIo), i64, i32, u32, vp, vp], i32),
        "gdn_chunk_reverse": ([vp, ctypes.POINTER(GdnIo), i64, u32, vp, vp], i32),
        "gdn_chunk_bidir": ([vp, ctypes.POINTER(GdnIo), vp, i64, u32, vp, vp], i32),
        "gdn_chunk_bidir_noalloc": ([ctypes.POINTER(GdnConfig), ctypes.POINTER(GdnIo), vp, i64, vp, vp, vp, vp], i32),
        "gdn_chunk_backward": ([vp, ctypes.POINTER(GdnIo), ctypes.POINTER(GdnGrad), i64, i32, vp], i32),
        "gdn_chunk_backward_bidir": ([vp, ctypes.POINTER(GdnIo), ctypes.POINTER(GdnGrad), ctypes.POINTER(GdnGrad), i64, vp],
                                     i32),
        "gdn_state_get": ([vp, vp, vp], i32),
        "gdn_state_set": ([vp, vp, vp], i32),
        "gdn_profile": ([vp, i32], i32),
        "gdn_profile_read": ([vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32], i32),
        "gdn_last_error": ([], ctypes.c_char_p),
        "gdn_attn_init": ([ctypes.POINTER(GdnAttnConfig), i32, ctypes.POINTER(vp)], i32),
        "gdn_attn_destroy": ([vp], i32),
        "gdn_attn_chunk": ([vp, ctypes.POINTER(GdnAttnIo), i64, u32, vp], i32),
        "gdn_attn_reset": ([vp], i32),
        "gdn_attn_cache_len": ([vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)], i32),
        "gdn_attn_cache_bytes": ([vp, ctypes.POINTER(ctypes.c_int64)], i32),
        "gdn_attn_cache_get": ([vp, vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), vp], i32),
        "gdn_attn_cache_set": ([vp, vp, i64, i64, vp], i32),
        "gdn_attn_profile": ([vp, i32], i32),
        "gdn_attn_profile_read": ([vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32], i32),
        "gdn_quantize_rows_e4m3": ([vp, i32, i64, i64, i64, vp, i64, vp, vp], i32),
        "gdn_gemm_e4m3": ([vp, i64, vp, vp, i64, vp, i64, i64, i64, vp, i64, vp], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def gdn_last_error() -> str:
    return load_library().gdn_last_error().decode()


def _check(rc):
    if rc != GDN_OK:
        raise GdnError(rc, gdn_last_error())


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides3(t):
    st = t.stride()
    return _Strides(st[0], st[1], st[2])


def _make_io(q, k, v, o, a, beta):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be [B, T, H, D] with a contiguous last dimension")
    for name, t in (("a", a), ("beta", beta)):
        if t.dim() != 3:
            raise ValueError(f"{name} must be [B, T, H]")
    if a.stride() != beta.stride():
        raise ValueError("a and beta must share strides")
    io = GdnIo()
    io.q, io.k, io.v, io.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    io.a, io.beta = a.data_ptr(), beta.data_ptr()
    io.q_strides, io.k_strides, io.v_strides = _strides3(q), _strides3(k), _strides3(v)
    io.o_strides, io.g_strides = _strides3(o), _strides3(a)
    return io


def gdn_stream_init(batch, heads, d_k, d_v, max_tokens, *, subchunk=0, io_dtype=GDN_BF16,
                    l2norm=True, l2_eps=1e-6, scale=1.0, gate_is_log=False, poison_ws=False, device=0):
    """Create a handle; returns the opaque pointer (int)."""
    lib = load_library()
    flags = ((GDN_L2NORM_QK if l2norm else 0) | (GDN_GATE_IS_LOG if gate_is_log else 0)
             | (GDN_POISON_WS if poison_ws else 0))
    cfg = GdnConfig(batch, heads, d_k, d_v, max_tokens, subchunk, io_dtype, flags, l2_eps, scale)
    h = ctypes.c_void_p()
    _check(lib.gdn_stream_init(ctypes.byref(cfg), int(device), ctypes.byref(h)))
    return h.value


def gdn_stream_destroy(handle):
    _check(load_library().gdn_stream_destroy(ctypes.c_void_p(handle)))


def gdn_chunk_forward(handle, q, k, v, a, beta, o, *, flags=0, state_out=None, stream=None):
    io = _make_io(q, k, v, o, a, beta)
    _check(load_library().gdn_chunk_forward(ctypes.c_void_p(handle), ctypes.byref(io), q.shape[1], flags,
                                            _ptr(state_out), _stream_ptr(stream, q.device)))


def gdn_chunk_forward_split(handle, q, k, v, a, beta, o, segments, *, flags=0, state_out=None, stream=None):
    io = _make_io(q, k, v, o, a, beta)
    _check(load_library().gdn_chunk_forward_split(ctypes.c_void_p(handle), ctypes.byref(io), q.shape[1], int(segments),
                                                  flags, _ptr(state_out), _stream_ptr(stream, q.device)))


def gdn_chunk_reverse(handle, q, k, v, a, beta, o, *, flags=0, state_out=None, stream=None):
    io = _make_io(q, k, v, o, a, beta)
    _check(load_library().gdn_chunk_reverse(ctypes.c_void_p(handle), ctypes.byref(io), q.shape[1], flags,
                                            _ptr(state_out), _stream_ptr(stream, q.device)))


def gdn_chunk_bidir(handle, q, k, v, a, beta, o, o_rev, *, flags=0, state_out=None, stream=None):
    if o_rev.stride() != o.stride():
        raise ValueError("o_rev must have o's strides")
    io = _make_io(q, k, v, o, a, beta)
    _check(load_library().gdn_chunk_bidir(ctypes.c_void_p(handle), ctypes.byref(io), _ptr(o_rev), q.shape[1],
                                          flags, _ptr(state_out), _stream_ptr(stream, q.device)))


def gdn_chunk_bidir_noalloc(q, k, v, a, beta, o, o_rev, status, *, state_in=None, state_out=None, subchunk=0,
                            l2norm=True, l2_eps=1e-6, scale=1.0, gate_is_log=False, stream=None):
    """Both scans of one chunk without a handle and without any device allocation: the
    workspace is the library's static scratch.  ``status`` is an int32 device tensor of one
    element that the kernels set to 1 if a wait gives up."""
    if o_rev.stride() != o.stride():
        raise ValueError("o_rev must have o's strides")
    if status.dtype.itemsize != 4 or status.numel() < 1:
        raise ValueError("status must be an int32 tensor")
    B, T, H, Dk = q.shape
    flags = (GDN_L2NORM_QK if l2norm else 0) | (GDN_GATE_IS_LOG if gate_is_log else 0)
    cfg = GdnConfig(B, H, Dk, v.shape[-1], max(T, 1), subchunk, GDN_BF16, flags, l2_eps, scale)
    io = _make_io(q, k, v, o, a, beta)
    _check(load_library().gdn_chunk_bidir_noalloc(ctypes.byref(cfg), ctypes.byref(io), _ptr(o_rev), T,
                                                  _ptr(state_in), _ptr(state_out), _ptr(status),
                                                  _stream_ptr(stream, q.device)))


def gdn_state_get(handle, dst, *, stream=None):
    _check(load_library().gdn_state_get(ctypes.c_void_p(handle), _ptr(dst), _stream_ptr(stream, dst.device)))


def gdn_state_set(handle, src, *, stream=None, device=None):
    dev = src.device if src is not None else device
    _check(load_library().gdn_state_set(ctypes.c_void_p(handle), _ptr(src), _stream_ptr(stream, dev)))


def gdn_profile(handle, enable=True):
    _check(load_library().gdn_profile(ctypes.c_void_p(handle), int(bool(enable))))


def gdn_profile_read(handle, reset=True):
    """{kernel name: (total ms, launches)} for the timed launches since the last reset."""
    ms = (ctypes.c_double * GDN_KERNEL_COUNT)()
    n = (ctypes.c_int64 * GDN_KERNEL_COUNT)()
    _check(load_library().gdn_profile_read(ctypes.c_void_p(handle), ms, n, int(bool(reset))))
    return {KERNEL_NAMES[i]: (ms[i], n[i]) for i in range(GDN_KERNEL_COUNT)}


def _make_grad(d_o, grads, d_state, state0):
    for name in ("dq", "dk", "dv", "da", "dbeta"):
        t = grads[name]
        if not t.is_contiguous() or t.dtype.itemsize != 4:
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    g = GdnGrad()
    g.d_o = d_o.data_ptr()
    g.d_state = None if d_state is None else d_state.data_ptr()
    g.state0 = None if state0 is None else state0.data_ptr()
    g.dq, g.dk, g.dv = grads["dq"].data_ptr(), grads["dk"].data_ptr(), grads["dv"].data_ptr()
    g.da, g.dbeta = grads["da"].data_ptr(), grads["dbeta"].data_ptr()
    g.d_state0 = None if grads.get("d_state0") is None else grads["d_state0"].data_ptr()
    return g


def gdn_chunk_backward(handle, q, k, v, a, beta, d_o, grads, *, reverse=False, d_state=None, state0=None,
                       stream=None):
    """Gradients of one scan.  ``grads`` maps dq, dk, dv (fp32 [B, T, H, D], contiguous), da,
    dbeta (fp32 [B, T, H], contiguous) and optionally d_state0 (fp32 [B, H, d_v, d_k]) to
    the tensors to write."""
    io = _make_io(q, k, v, d_o, a, beta)
    g = _make_grad(d_o, grads, d_state, state0)
    _check(load_library().gdn_chunk_backward(ctypes.c_void_p(handle), ctypes.byref(io), ctypes.byref(g), q.shape[1],
                                             int(bool(reverse)), _stream_ptr(stream, q.device)))


def gdn_chunk_backward_bidir(handle, q, k, v, a, beta, d_o_fwd, d_o_rev, grads_fwd, grads_rev, *, d_state=None,
                             state0=None, d_state_rev=None, stream=None):
    """Gradients of both scans of a bidirectional call in one launch pair: the forward scan's
    (d_o_fwd, d_state, state0) into ``grads_fwd`` and the reverse scan's (d_o_rev, d_state_rev)
    into ``grads_rev`` (dicts as for gdn_chunk_backward; d_o_rev must have d_o_fwd's strides)."""
    if tuple(d_o_rev.stride()) != tuple(d_o_fwd.stride()):
        raise ValueError("d_o_fwd and d_o_rev must have the same strides")
    io = _make_io(q, k, v, d_o_fwd, a, beta)
    gf = _make_grad(d_o_fwd, grads_fwd, d_state, state0)
    gr = _make_grad(d_o_rev, grads_rev, d_state_rev, None)
    _check(load_library().gdn_chunk_backward_bidir(ctypes.c_void_p(handle), ctypes.byref(io), ctypes.byref(gf),
                                                   ctypes.byref(gr), q.shape[1], _stream_ptr(stream, q.device)))


class Stream:
    """One handle: B streams x H heads of carried state on one device."""

    def __init__(self, batch, heads, d_k, d_v, max_tokens, *, subchunk=0, io_dtype="bf16", l2norm=True,
                 l2_eps=1e-6, scale=1.0, gate_is_log=False, poison_ws=False, device=0):
        self.shape = (batch, heads, d_v, d_k)
        self.device = device
        self.handle = gdn_stream_init(batch, heads, d_k, d_v, max_tokens, subchunk=subchunk,
                                      io_dtype=GDN_F32 if io_dtype == "f32" else GDN_BF16, l2norm=l2norm,
                                      l2_eps=l2_eps, scale=scale, gate_is_log=gate_is_log, poison_ws=poison_ws,
                                      device=device)

    def forward(self, q, k, v, a, beta, o, **kw):
        gdn_chunk_forward(self.handle, q, k, v, a, beta, o, **kw)

    def forward_split(self, q, k, v, a, beta, o, segments, **kw):
        gdn_chunk_forward_split(self.handle, q, k, v, a, beta, o, segments, **kw)

    def reverse(self, q, k, v, a, beta, o, **kw):
        gdn_chunk_reverse(self.handle, q, k, v, a, beta, o, **kw)

    def bidir(self, q, k, v, a, beta, o, o_rev, **kw):
        gdn_chunk_bidir(self.handle, q, k, v, a, beta, o, o_rev, **kw)

    def _grad_buffers(self, q, v):
        import torch
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        dev = q.device
        return {"dq": torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev),
                "dk": torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev),
                "dv": torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev),
                "da": torch.empty((B, T, H), dtype=torch.float32, device=dev),
                "dbeta": torch.empty((B, T, H), dtype=torch.float32, device=dev),
                "d_state0": torch.empty(self.shape, dtype=torch.float32, device=dev)}

    def backward(self, q, k, v, a, beta, d_o, *, reverse=False, d_state=None, state0=None, **kw):
        """Gradients of one scan; returns a dict of fp32 tensors dq, dk, dv, da, dbeta, d_state0."""
        g = self._grad_buffers(q, v)
        gdn_chunk_backward(self.handle, q, k, v, a, beta, d_o, g, reverse=reverse, d_state=d_state, state0=state0, **kw)
        return g

    def backward_bidir(self, q, k, v, a, beta, d_o_fwd, d_o_rev, *, d_state=None, state0=None, d_state_rev=None, **kw):
        """Gradients of both scans of a bidirectional call; returns (forward scan's dict, reverse scan's dict)."""
        gf, gr = self._grad_buffers(q, v), self._grad_buffers(q, v)
        gdn_chunk_backward_bidir(self.handle, q, k, v, a, beta, d_o_fwd, d_o_rev, gf, gr, d_state=d_state,
                                 state0=state0, d_state_rev=d_state_rev, **kw)
        return gf, gr

    def state_get(self, dst=None, **kw):
        import torch
        if dst is None:
            dst = torch.empty(self.shape, dtype=torch.float32, device=f"cuda:{self.device}")
        gdn_state_get(self.handle, dst, **kw)
        return dst

    def state_set(self, src, **kw):
        gdn_state_set(self.handle, src, device=f"cuda:{self.device}", **kw)

    def close(self):
        if self.handle:
            gdn_stream_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- softmax-block attention over the sink + window cache ----------------------------------

def gdn_attn_init(batch, heads, head_dim, sink_tokens, window_tokens, max_tokens, *, scale=0.0, device=0):
    """Create an attention handle (scale 0 selects 1/sqrt(head_dim)); returns the opaque pointer."""
    cfg = GdnAttnConfig(batch, heads, head_dim, sink_tokens, window_tokens, max_tokens, scale)
    h = ctypes.c_void_p()
    _check(load_library().gdn_attn_init(ctypes.byref(cfg), int(device), ctypes.byref(h)))
    return h.value


def gdn_attn_destroy(handle):
    _check(load_library().gdn_attn_destroy(ctypes.c_void_p(handle)))


def gdn_attn_chunk(handle, q, k, v, o, *, flags=0, stream=None):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be [B, T, H, D] with a contiguous last dimension")
    io = GdnAttnIo()
    io.q, io.k, io.v, io.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    io.q_strides, io.k_strides, io.v_strides, io.o_strides = _strides3(q), _strides3(k), _strides3(v), _strides3(o)
    _check(load_library().gdn_attn_chunk(ctypes.c_void_p(handle), ctypes.byref(io), q.shape[1], flags,
                                         _stream_ptr(stream, q.device)))


def gdn_attn_reset(handle):
    _check(load_library().gdn_attn_reset(ctypes.c_void_p(handle)))


def gdn_attn_cache_len(handle):
    s, w = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().gdn_attn_cache_len(ctypes.c_void_p(handle), ctypes.byref(s), ctypes.byref(w)))
    return s.value, w.value


def gdn_attn_cache_bytes(handle):
    n = ctypes.c_int64()
    _check(load_library().gdn_attn_cache_bytes(ctypes.c_void_p(handle), ctypes.byref(n)))
    return n.value


def gdn_attn_cache_get(handle, dst, *, stream=None):
    """Copy the cache into the uint8 device tensor ``dst``; returns (sink_len, window_total)."""
    s, w = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().gdn_attn_cache_get(ctypes.c_void_p(handle), _ptr(dst), ctypes.byref(s), ctypes.byref(w),
                                             _stream_ptr(stream, dst.device)))
    return s.value, w.value


def gdn_attn_cache_set(handle, src, sink_len, window_total, *, stream=None):
    _check(load_library().gdn_attn_cache_set(ctypes.c_void_p(handle), _ptr(src), int(sink_len), int(window_total),
                                             _stream_ptr(stream, src.device)))


def gdn_attn_profile(handle, enable=True):
    _check(load_library().gdn_attn_profile(ctypes.c_void_p(handle), int(bool(enable))))


def gdn_attn_profile_read(handle, reset=True):
    """(total ms, launches) of the attention kernel since the last reset."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().gdn_attn_profile_read(ctypes.c_void_p(handle), ctypes.byref(ms), ctypes.byref(n),
                                                int(bool(reset))))
    return ms.value, n.value


class WindowAttention:
    """One softmax block: B streams x H heads of sink + window cache on one device."""

    def __init__(self, batch, heads, head_dim, sink_tokens, window_tokens, max_tokens, *, scale=0.0, device=0):
        self.handle = gdn_attn_init(batch, heads, head_dim, sink_tokens, window_tokens, max_tokens, scale=scale,
                                    device=device)

    def chunk(self, q, k, v, o=None, *, commit=True, stream=None):
        import torch
        if o is None:
            o = torch.empty_like(v)
        gdn_attn_chunk(self.handle, q, k, v, o, flags=0 if commit else GDN_NO_COMMIT, stream=stream)
        return o

    def reset(self):
        gdn_attn_reset(self.handle)

    def cache_len(self):
        return gdn_attn_cache_len(self.handle)

    def checkpoint(self, device="cuda"):
        """(snapshot tensor, sink_len, window_total) of the cache."""
        import torch
        snap = torch.empty(gdn_attn_cache_bytes(self.handle), dtype=torch.uint8, device=device)
        s, w = gdn_attn_cache_get(self.handle, snap)
        return snap, s, w

    def restore(self, snap, sink_len, window_total):
        gdn_attn_cache_set(self.handle, snap, sink_len, window_total)

    def close(self):
        if self.handle:
            gdn_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- FP8 (E4M3) projection GEMMs ---------------------------------------------------------------------

def e4m3_codes_empty(rows, cols, device):
    """An uninitialised uint8 [rows, cols] code matrix whose row stride is cols rounded up to a multiple of 128
    bytes: the GEMM reads each row in 128-byte k steps, and rows that start on a 128-byte boundary take one
    cache line per step instead of two."""
    import torch
    return torch.empty((rows, (cols + 127) // 128 * 128), dtype=torch.uint8, device=device)[:, :cols]


def quantize_rows_e4m3(x, codes=None, scales=None, *, stream=None):
    """Per-row E4M3 quantisation of a 2-D bf16 or fp32 tensor with a contiguous last dimension; returns
    (codes uint8 [rows, cols], scales fp32 [rows]).  New code matrices come from e4m3_codes_empty."""
    import torch
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with a contiguous last dimension")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bf16 or fp32")
    rows, cols = x.shape
    if codes is None:
        codes = e4m3_codes_empty(rows, cols, x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(load_library().gdn_quantize_rows_e4m3(_ptr(x), GDN_F32 if x.dtype == torch.float32 else GDN_BF16, rows, cols,
                                                 x.stride(0), _ptr(codes), codes.stride(0), _ptr(scales),
                                                 _stream_ptr(stream, x.device)))
    return codes, scales


def gemm_e4m3(x_codes, x_scales, w_codes, w_scales, y=None, *, stream=None):
    """y [M, N] bf16 = diag(x_scales) dec(x_codes) dec(w_codes)^T diag(w_scales) for E4M3 codes x [M, K] and
    w [N, K] (uint8, contiguous last dimension)."""
    import torch
    M, K = x_codes.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != K:
        raise ValueError("x and w must share K")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x_codes.device)
    _check(load_library().gdn_gemm_e4m3(_ptr(x_codes), x_codes.stride(0), _ptr(x_scales), _ptr(w_codes),
                                        w_codes.stride(0), _ptr(w_scales), M, N, K, _ptr(y), y.stride(0),
                                        _stream_ptr(stream, x_codes.device)))
    return y
