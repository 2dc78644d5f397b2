"""The C-ABI library loads, exports every function include/sdv.h declares, and
rejects bad arguments on the host before touching the GPU (no compute here)."""

import ctypes
import os
import re

import pytest

import draft_verification_amd as sdv
from draft_verification_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sdv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"sd_schedule", "sd_verify", "sd_markov_draft"} <= set(names)
    L = ctypes.CDLL(_lib._LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sdv.EXPORTS)


def test_version_and_status_strings():
    assert sdv.sd_abi_version() == 4
    assert sdv.sd_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, 1, 2, 4, 8, 16):
        assert sdv.sd_status_string(code) != "unknown status"
    assert sdv.sd_status_string(12345) == "unknown status"


def test_workspace_sizes():
    ws = sdv.sd_verify_workspace_size(256, 11, 151936)
    assert 0 < ws < 64 << 20
    assert sdv.sd_verify_workspace_size(-1, 1, 8) == 0
    assert sdv.sd_markov_draft_workspace_size(128, 16, 129280, 256) > 0


N = None


def _sched(R, g, mode, sps_len, conf=1, sps=1, ell=1, cap=None, ws=1 << 20, threshold=0.5):
    L = sdv.lib()
    p = lambda x: ctypes.c_void_p(16) if x else None
    return L.sd_schedule(None, R, g, None, p(conf), None, p(sps), sps_len, mode, p(cap), threshold,
                         p(ell), N, N, N, N, ctypes.c_void_p(256), ws)


def test_schedule_host_validation():
    assert _sched(-1, 4, 0, 100) == _lib.SD_EINVAL
    assert _sched(4, 256, 0, 10000) == _lib.SD_EUNSUPPORTED
    assert _sched(2048, 16, 0, 40000) == _lib.SD_EUNSUPPORTED      # 32768 slots
    assert _sched(4, 4, 4, 100) == _lib.SD_EINVAL                  # bad mode
    assert _sched(4, 4, 3, 100, threshold=float("nan")) == _lib.SD_EINVAL   # NaN threshold
    assert _sched(4, 4, 2, 100) == _lib.SD_EINVAL                  # capped without cap_k
    assert _sched(4, 4, 0, 19) == _lib.SD_ERANGE                   # table < R(1+g)
    assert _sched(4, 4, 0, 20, ell=0) == _lib.SD_EINVAL
    assert _sched(4, 4, 0, 20, ws=64) == _lib.SD_ERANGE          # workspace < 16 keys


def _ver(R=2, g=2, V=64, ld=64, dt=1, T=1.0, ws=1 << 20, ws_ptr=256, nulls=(), dstats=None, rstats=None,
         alpha=None, options=0):
    L = sdv.lib()
    P = lambda name: None if name in nulls else ctypes.c_void_p(256)
    opt = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.sd_verify(None, R, g, V, ld, dt, T, 1, None, P("tgt"), P("t0"), P("drf"), P("d0"),
                       opt(dstats), P("toks"), P("ell"), P("nacc"), P("out"), P("st"), None,
                       opt(rstats), opt(alpha), options, ctypes.c_void_p(ws_ptr), ws, None, None)


def test_verify_host_validation():
    assert _ver(V=60, ld=64) == _lib.SD_EINVAL
    assert _ver(ld=32) == _lib.SD_EINVAL
    assert _ver(ld=68) == _lib.SD_EINVAL
    assert _ver(dt=5) == _lib.SD_EINVAL
    assert _ver(T=0.0) == _lib.SD_EINVAL
    assert _ver(T=float("nan")) == _lib.SD_EINVAL
    assert _ver(g=300) == _lib.SD_EUNSUPPORTED
    assert _ver(ws=16) == _lib.SD_ERANGE
    assert _ver(ws_ptr=8) == _lib.SD_EINVAL                          # misaligned workspace
    assert _ver(nulls=("tgt",)) == _lib.SD_EINVAL
    assert _ver(nulls=("ell",)) == _lib.SD_EINVAL
    assert _ver(R=0) == _lib.SD_OK                                  # nothing to do
    assert _ver(options=2) == _lib.SD_EINVAL                        # unknown option
    assert _ver(options=sdv.SD_VERIFY_STOP_AT_REJECTION, alpha=256) == _lib.SD_EINVAL  # alpha needs every row
    assert _ver(dstats=260) == _lib.SD_EINVAL                       # (m, Z) pairs need 8 bytes
    assert _ver(rstats=260) == _lib.SD_EINVAL
    # 1024 requests x 511 rows x 64 chunks: more work-items than one launch holds
    assert _ver(R=1024, g=255, V=1 << 20, ld=1 << 20, ws=1 << 40) == _lib.SD_EUNSUPPORTED


def _mk(R=2, g=2, V=64, rank=32, H=8, re_=8, T=1.0, ws=1 << 20, nulls=(), qstats=None):
    L = sdv.lib()
    P = lambda name: None if name in nulls else ctypes.c_void_p(256)
    qs = None if qstats is None else ctypes.c_void_p(qstats)
    return L.sd_markov_draft(None, R, g, V, rank, T, 1, None, P("U"), P("A"), P("C"), P("x0"),
                             P("h"), H, P("E"), re_, P("w"), P("tok"), P("ql"), qs, P("conf"),
                             P("st"), ctypes.c_void_p(256), ws)


def test_markov_host_validation():
    assert _mk(rank=48) == _lib.SD_EINVAL
    assert _mk(rank=512) == _lib.SD_EUNSUPPORTED
    assert _mk(V=100) == _lib.SD_EINVAL
    assert _mk(H=12) == _lib.SD_EINVAL
    assert _mk(T=-1.0) == _lib.SD_EINVAL
    assert _mk(ws=8) == _lib.SD_ERANGE
    assert _mk(nulls=("C",)) == _lib.SD_EINVAL
    assert _mk(R=0) == _lib.SD_OK
    assert _mk(qstats=260) == _lib.SD_EINVAL                        # (m, Z) pairs need 8 bytes


def test_verify_noalloc_host_validation():
    """The allocation-free verify refuses, before any GPU call, sizes whose
    workspace exceeds the one the library holds (16 MiB per GPU)."""
    L = sdv.lib()
    p = ctypes.c_void_p(256)
    limit = 16 << 20
    assert sdv.sd_verify_workspace_size(256, 11, 151936) <= limit        # the headline block fits
    assert sdv.sd_verify_workspace_size(512, 16, 151936) <= limit        # the ragged step fits
    assert sdv.sd_verify_workspace_size(1024, 64, 151936) > limit

    def call(R, g, V):
        return L.sd_verify_noalloc(None, R, g, V, V, 1, 1.0, 1, None, p, p, p, p, None, p, p, p, p, p,
                                   None, None, None, 0)
    assert call(1024, 64, 151936) == _lib.SD_ERANGE
    assert call(-1, 4, 1024) == _lib.SD_EINVAL
    assert call(4, 256, 1024) == _lib.SD_EUNSUPPORTED
    assert call(0, 4, 1024) == _lib.SD_OK


def test_uniforms_host_validation():
    L = sdv.lib()
    p = ctypes.c_void_p(256)
    assert L.sd_uniforms(None, 1, -1, p, p, 0, p) == _lib.SD_EINVAL          # negative size
    assert L.sd_uniforms(None, 1, 4, p, p, -1, p) == _lib.SD_EINVAL          # negative draw
    assert L.sd_uniforms(None, 1, 4, None, p, 0, p) == _lib.SD_EINVAL        # no request ids
    assert L.sd_uniforms(None, 1, 4, p, p, 0, None) == _lib.SD_EINVAL        # no output
    assert L.sd_uniforms(None, 1, 0, None, None, 2, None) == _lib.SD_OK      # nothing to draw


def test_read_probe_is_outside_the_library():
    """The benchmark's streaming read lives in libsdv_probe.so, not in the
    library's interface; its host checks."""
    assert not hasattr(ctypes.CDLL(_lib._LIB_PATH), "probe_stream_read")
    P = ctypes.CDLL(os.path.join(os.path.dirname(_lib._LIB_PATH), "libsdv_probe.so"))
    P.probe_stream_read_sink_words.restype = ctypes.c_longlong
    P.probe_stream_read_sink_words.argtypes = [ctypes.c_longlong]
    P.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    assert P.probe_stream_read_sink_words(0) == 0              # one word per 128 KB workgroup
    assert P.probe_stream_read_sink_words(16) == 1
    assert P.probe_stream_read_sink_words(131072) == 1
    assert P.probe_stream_read_sink_words(131088) == 2
    assert P.probe_stream_read_sink_words(-16) == -1
    p = ctypes.c_void_p(256)
    assert P.probe_stream_read(None, p, 24, p) == _lib.SD_EINVAL        # not a multiple of 16
    assert P.probe_stream_read(None, None, 32, p) == _lib.SD_EINVAL     # no source
    assert P.probe_stream_read(None, ctypes.c_void_p(8), 32, p) == _lib.SD_EINVAL   # misaligned
    assert P.probe_stream_read(None, p, 0, None) == _lib.SD_OK          # nothing to read


def test_lightspec_host_validation():
    L = sdv.lib()
    p = ctypes.c_void_p(256)
    for lam in (float("nan"), -0.1, 1.5):
        assert L.sd_lightspec_update(None, 4, 4, p, p, p, lam, p, p) == _lib.SD_EINVAL
    assert L.sd_lightspec_update(None, 4, 256, p, p, p, 0.1, p, p) == _lib.SD_EUNSUPPORTED
    assert L.sd_lightspec_update(None, 4, 4, None, p, p, 0.1, p, p) == _lib.SD_EINVAL
    assert L.sd_lightspec_update(None, 0, 4, None, None, None, 0.1, None, None) == _lib.SD_OK
    ws = L.sd_lightspec_plan_workspace_size(4, 4)
    assert ws >= L.sd_schedule_workspace_size(4, 4)

    def plan(R=4, g=4, sps_len=20, wsb=ws, nulls=()):
        P = lambda name: None if name in nulls else p
        return L.sd_lightspec_plan(None, R, g, P("ema"), P("cnt"), None, P("sps"), sps_len, P("cost"),
                                   None, P("ell"), None, None, None, P("dn"), P("bn"), None, p, wsb)

    assert plan(sps_len=19) == _lib.SD_ERANGE
    assert plan(wsb=ws - 1) == _lib.SD_ERANGE
    assert plan(R=2048, g=16, sps_len=40000) == _lib.SD_EUNSUPPORTED
    assert plan(nulls=("cost",)) == _lib.SD_EINVAL
    assert plan(nulls=("dn",)) == _lib.SD_EINVAL
