"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from gated_deltanet_streaming_amd import binding

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, "gdn_stream.h"), os.path.join(INCLUDE, "gdn_attn.h"), os.path.join(INCLUDE, "gdn_lowp.h")]


def declared_symbols():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_boundary():
    names = declared_symbols()
    for required in ("gdn_stream_init", "gdn_stream_destroy", "gdn_chunk_forward", "gdn_chunk_reverse",
                     "gdn_state_get", "gdn_state_set", "gdn_last_error", "gdn_attn_init", "gdn_attn_chunk",
                     "gdn_attn_destroy"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_symbols() if not hasattr(lib, n)]
    assert not missing, missing


def test_only_declared_symbols_are_exported():
    out = os.popen(f"nm -D --defined-only {binding.library_path()}").read()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    gdn = {n for n in exported if n.startswith("gdn_")}
    assert gdn == set(declared_symbols())


def _cfg(**kw):
    base = dict(batch=1, heads=2, d_k=112, d_v=112, max_tokens=2640, subchunk=0, io_dtype=binding.GDN_BF16,
                flags=binding.GDN_L2NORM_QK, l2_eps=1e-6, scale=1.0)
    base.update(kw)
    return binding.GdnConfig(**base)


@pytest.mark.parametrize("bad, code", [
    (dict(batch=0), binding.GDN_E_SHAPE),
    (dict(heads=-1), binding.GDN_E_SHAPE),
    (dict(d_k=100), binding.GDN_E_SHAPE),
    (dict(d_v=144), binding.GDN_E_SHAPE),
    (dict(max_tokens=0), binding.GDN_E_SHAPE),
    (dict(subchunk=48), binding.GDN_E_SHAPE),
    (dict(io_dtype=7), binding.GDN_E_DTYPE),
    (dict(flags=0x80), binding.GDN_E_INVAL),
    (dict(l2_eps=-1.0), binding.GDN_E_INVAL),
    (dict(scale=float("nan")), binding.GDN_E_INVAL),
])
def test_init_rejects_bad_config(lib, bad, code):
    h = ctypes.c_void_p(123)
    rc = lib.gdn_stream_init(ctypes.byref(_cfg(**bad)), 0, ctypes.byref(h))
    assert rc == code
    assert h.value is None
    assert binding.gdn_last_error()


def test_null_arguments_are_rejected(lib):
    h = ctypes.c_void_p()
    assert lib.gdn_stream_init(None, 0, ctypes.byref(h)) == binding.GDN_E_INVAL
    io = binding.GdnIo()
    for fn in (lib.gdn_chunk_forward, lib.gdn_chunk_reverse):
        assert fn(None, ctypes.byref(io), 1, 0, None, None) == binding.GDN_E_INVAL
        assert "handle" in binding.gdn_last_error()
    assert lib.gdn_chunk_bidir(None, ctypes.byref(io), None, 1, 0, None, None) == binding.GDN_E_INVAL
    assert lib.gdn_chunk_forward_split(None, ctypes.byref(io), 1, 2, 0, None, None) == binding.GDN_E_INVAL
    assert lib.gdn_state_get(None, None, None) == binding.GDN_E_INVAL
    assert lib.gdn_state_set(None, None, None) == binding.GDN_E_INVAL
    assert lib.gdn_stream_destroy(None) == binding.GDN_OK


@pytest.mark.parametrize("bad, code, word", [
    (dict(io_dtype=binding.GDN_F32), binding.GDN_E_DTYPE, "bf16"),
    (dict(flags=binding.GDN_POISON_WS), binding.GDN_E_INVAL, "flag"),
    (dict(d_k=48, d_v=48), binding.GDN_E_SHAPE, "chunked"),
    (dict(subchunk=8), binding.GDN_E_SHAPE, "subchunk"),
    (dict(heads=20, max_tokens=8200), binding.GDN_E_SHAPE, "scratch"),
])
def test_noalloc_rejects_bad_calls_before_any_device_work(lib, bad, code, word):
    """Argument checks of the allocation-free call come before any HIP call, so they hold here.
    The scratch bound: B=1 H=20 d=112 T=8200 needs 2*20*129*13312 bytes > 64 MiB."""
    io = binding.GdnIo()
    status = ctypes.c_int(0)
    cfg = _cfg(**bad)
    rc = lib.gdn_chunk_bidir_noalloc(ctypes.byref(cfg), ctypes.byref(io), None, cfg.max_tokens, None, None,
                                     ctypes.byref(status), None)
    assert rc == code
    assert word in binding.gdn_last_error()


def test_noalloc_null_arguments_are_rejected(lib):
    io = binding.GdnIo()
    cfg = _cfg()
    status = ctypes.c_int(0)
    assert lib.gdn_chunk_bidir_noalloc(None, ctypes.byref(io), None, 1, None, None, ctypes.byref(status),
                                       None) == binding.GDN_E_INVAL
    assert lib.gdn_chunk_bidir_noalloc(ctypes.byref(cfg), ctypes.byref(io), None, 1, None, None, None,
                                       None) == binding.GDN_E_INVAL
    assert "status" in binding.gdn_last_error()
    # T > 0 with NULL tensors is refused before the device is touched
    assert lib.gdn_chunk_bidir_noalloc(ctypes.byref(cfg), ctypes.byref(io), None, 64, None, None,
                                       ctypes.byref(status), None) == binding.GDN_E_INVAL
    assert "q is NULL" in binding.gdn_last_error()
    assert lib.gdn_chunk_bidir_noalloc(ctypes.byref(cfg), ctypes.byref(io), None, -1, None, None,
                                       ctypes.byref(status), None) == binding.GDN_E_SHAPE


def test_peaks_library_exports_its_probes():
    """The measurement-support library (copy and MFMA probes behind the roofline peaks) is
    built beside the GDN library and exports exactly its two entry points."""
    path = os.path.join(os.path.dirname(binding.library_path()), "libgdn_peaks.so")
    if not os.path.exists(path):
        pytest.skip("libgdn_peaks.so not built (run __graft_entry__.build())")
    out = os.popen(f"nm -D --defined-only {path}").read()
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == {"gdn_peak_copy", "gdn_peak_mfma_bf16", "gdn_peak_mfma_fp8", "gdn_peak_lds_read"}
    lib = ctypes.CDLL(path)
    lib.gdn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    ms = ctypes.c_float()
    # argument checks only (no device work): null buffers and a size that is not a multiple of 16
    assert lib.gdn_peak_copy(None, None, 1024, 1, 0, None, ctypes.byref(ms)) == -1
    assert lib.gdn_peak_copy(1, 1, 1000, 1, 0, None, ctypes.byref(ms)) == -1


def _attn_cfg(**kw):
    base = dict(batch=1, heads=20, head_dim=112, sink_tokens=880, window_tokens=2640, max_tokens=2640, scale=0.0)
    base.update(kw)
    return binding.GdnAttnConfig(**base)


@pytest.mark.parametrize("bad, code", [
    (dict(batch=0), binding.GDN_E_SHAPE),
    (dict(heads=0), binding.GDN_E_SHAPE),
    (dict(head_dim=96), binding.GDN_E_SHAPE),
    (dict(head_dim=32), binding.GDN_E_SHAPE),
    (dict(sink_tokens=-1), binding.GDN_E_SHAPE),
    (dict(window_tokens=-5), binding.GDN_E_SHAPE),
    (dict(max_tokens=0), binding.GDN_E_SHAPE),
    (dict(sink_tokens=1 << 24), binding.GDN_E_SHAPE),       # 2^24 x 112 x 2 bytes > 2 GiB
    (dict(window_tokens=(1 << 30) - 1), binding.GDN_E_SHAPE),
    (dict(max_tokens=1 << 24), binding.GDN_E_SHAPE),
    (dict(scale=-1.0), binding.GDN_E_INVAL),
    (dict(scale=float("inf")), binding.GDN_E_INVAL),
])
def test_attn_init_rejects_bad_config(lib, bad, code):
    h = ctypes.c_void_p(123)
    rc = lib.gdn_attn_init(ctypes.byref(_attn_cfg(**bad)), 0, ctypes.byref(h))
    assert rc == code
    assert h.value is None
    assert binding.gdn_last_error()


def test_attn_null_arguments_are_rejected(lib):
    h = ctypes.c_void_p()
    assert lib.gdn_attn_init(None, 0, ctypes.byref(h)) == binding.GDN_E_INVAL
    io = binding.GdnAttnIo()
    assert lib.gdn_attn_chunk(None, ctypes.byref(io), 1, 0, None) == binding.GDN_E_INVAL
    assert "handle" in binding.gdn_last_error()
    assert lib.gdn_attn_reset(None) == binding.GDN_E_INVAL
    assert lib.gdn_attn_cache_len(None, None, None) == binding.GDN_E_INVAL
    assert lib.gdn_attn_profile(None, 1) == binding.GDN_E_INVAL
    assert lib.gdn_attn_cache_bytes(None, None) == binding.GDN_E_INVAL
    assert lib.gdn_attn_cache_get(None, None, None, None, None) == binding.GDN_E_INVAL
    assert lib.gdn_attn_cache_set(None, None, 0, 0, None) == binding.GDN_E_INVAL
    assert lib.gdn_attn_profile_read(None, None, None, 0) == binding.GDN_E_INVAL
    assert lib.gdn_attn_destroy(None) == binding.GDN_OK
