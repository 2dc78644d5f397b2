"""ctypes binding of libsdv (include/sdv.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
The functions carry the C names.  A missing library is an error, never a
fallback.
"""

import ctypes
import functools
import inspect
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdv.so")
_lib = None

SD_OK = 0
SD_EINVAL = -1
SD_ERANGE = -2
SD_EUNSUPPORTED = -3
SD_ELAUNCH = -4

SD_DTYPE_F32 = 0
SD_DTYPE_BF16 = 1

SD_VERIFY_STOP_AT_REJECTION = 1

SD_SCHED_EARLY_STOP = 0
SD_SCHED_GLOBAL_ARGMAX = 1
SD_SCHED_CAPPED_TOPK = 2
SD_SCHED_THRESHOLD = 3

SD_ST_BAD_TOKEN = 1
SD_ST_NONFINITE = 2
SD_ST_ZERO_Z = 4
SD_ST_ZERO_RESIDUAL = 8
SD_ST_ZERO_Q = 16

EXPORTS = (
    "sd_abi_version", "sd_status_string", "sd_schedule_workspace_size", "sd_schedule",
    "sd_verify_workspace_size",
    "sd_verify", "sd_markov_draft_workspace_size", "sd_markov_draft",
    "sd_rnn_draft_workspace_size", "sd_rnn_draft",
    "sd_lightspec_update", "sd_lightspec_plan_workspace_size", "sd_lightspec_plan",
    "sd_uniforms", "sd_verify_noalloc",
)


class SdvError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {code} ({status_string(code)})")
        self.code = code


_P = ctypes.c_void_p
_I = ctypes.c_int
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t


def lib():
    """Load libsdv.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(_LIB_PATH)
    L.sd_abi_version.restype = _I
    L.sd_abi_version.argtypes = []
    L.sd_status_string.restype = ctypes.c_char_p
    L.sd_status_string.argtypes = [_I]
    L.sd_schedule.restype = _I
    L.sd_schedule_workspace_size.restype = _SZ
    L.sd_schedule_workspace_size.argtypes = [_I, _I]
    L.sd_schedule.argtypes = [_P, _I, _I, _P, _P, _P, _P, _I, _I, _P, ctypes.c_float, _P, _P, _P,
                              _P, _P, _P, _SZ]
    L.sd_verify_workspace_size.restype = _SZ
    L.sd_verify_workspace_size.argtypes = [_I, _I, _I]
    L.sd_verify.restype = _I
    L.sd_verify.argtypes = [_P, _I, _I, _I, _I, _I, ctypes.c_float, _U64, _P, _P, _P, _P, _P, _P,
                            _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P, _P]
    L.sd_markov_draft_workspace_size.restype = _SZ
    L.sd_markov_draft_workspace_size.argtypes = [_I, _I, _I, _I]
    L.sd_markov_draft.restype = _I
    L.sd_markov_draft.argtypes = [_P, _I, _I, _I, _I, ctypes.c_float, _U64, _P, _P, _P, _P, _P,
                                  _P, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _SZ]
    L.sd_rnn_draft_workspace_size.restype = _SZ
    L.sd_rnn_draft_workspace_size.argtypes = [_I, _I, _I, _I]
    L.sd_rnn_draft.restype = _I
    L.sd_rnn_draft.argtypes = [_P, _I, _I, _I, _I, ctypes.c_float, _U64, _P, _P, _P, _P, _P, _P, _P,
                               _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _SZ]
    L.sd_lightspec_update.restype = _I
    L.sd_lightspec_update.argtypes = [_P, _I, _I, _P, _P, _P, ctypes.c_double, _P, _P]
    L.sd_lightspec_plan_workspace_size.restype = _SZ
    L.sd_lightspec_plan_workspace_size.argtypes = [_I, _I]
    L.sd_lightspec_plan.restype = _I
    L.sd_lightspec_plan.argtypes = [_P, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P, _SZ]
    L.sd_verify_noalloc.restype = _I
    L.sd_verify_noalloc.argtypes = [_P, _I, _I, _I, _I, _I, ctypes.c_float, _U64, _P, _P, _P, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P, _I]
    L.sd_uniforms.restype = _I
    L.sd_uniforms.argtypes = [_P, _U64, ctypes.c_longlong, _P, _P, _I, _P]
    _lib = L
    return L


def sd_abi_version():
    return lib().sd_abi_version()


def status_string(code):
    return lib().sd_status_string(int(code)).decode()


sd_status_string = status_string


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on_stream(fn):
    """Run fn with its `stream` argument as torch's current stream, so the
    outputs and the temporary workspace it allocates belong to the stream the
    kernels are enqueued on: when the workspace is freed on return, the
    caching allocator hands that block only to later work of the same stream,
    never to another stream while these kernels may still use it.  Outputs
    and workspaces the caller passes in are the caller's to keep alive on
    that stream."""
    at = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        stream = kw.get("stream") if "stream" in kw else (args[at] if len(args) > at else None)
        if stream is None:  # torch's current stream already
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return wrapper


def _out(o, key, make):
    """The caller's output `key` from `o` when present, else a new tensor
    from make() (made only then)."""
    return o[key] if key in o else make()


def _check(fn, code):
    if code != SD_OK:
        raise SdvError(fn, code)


def _workspace(nbytes, device):
    # 256-byte aligned by torch's caching allocator
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def sd_schedule_workspace_size(R, gmax):
    return lib().sd_schedule_workspace_size(R, gmax)


@_on_stream
def sd_schedule(conf, sps, mode, gamma_r=None, cap_k=None, out=None, surv=True, workspace=None,
                stream=None, sts_temp=None, threshold=0.0):
    """Run the scheduler.  conf [R][gmax] fp32, sps fp32, gamma_r [R] int32 or
    None, cap_k a 1-element int32 device tensor (CAPPED_TOPK), sts_temp
    [gmax] fp32 per-position temperatures or None, threshold the survival
    threshold (THRESHOLD mode).  Returns a dict of device tensors: ell, batch,
    n_sel, theta, surv."""
    R, gmax = conf.shape
    dev = conf.device
    o = out or {}
    ell = _out(o, "ell", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    batch = _out(o, "batch", lambda: torch.empty(1, dtype=torch.int32, device=dev))
    n_sel = _out(o, "n_sel", lambda: torch.empty(1, dtype=torch.int32, device=dev))
    theta = _out(o, "theta", lambda: torch.empty(1, dtype=torch.float64, device=dev))
    sv = _out(o, "surv", lambda: torch.empty((R, gmax), dtype=torch.float32, device=dev)) if surv else None
    ws = workspace if workspace is not None else _workspace(sd_schedule_workspace_size(R, gmax), dev)
    code = lib().sd_schedule(
        _stream(stream), R, gmax, _ptr(gamma_r, torch.int32, "gamma_r"),
        _ptr(conf, torch.float32, "conf"), _ptr(sts_temp, torch.float32, "sts_temp"),
        _ptr(sps, torch.float32, "sps"), sps.numel(), int(mode), _ptr(cap_k, torch.int32, "cap_k"),
        float(threshold), _ptr(ell, torch.int32), _ptr(batch, torch.int32),
        _ptr(n_sel, torch.int32), _ptr(theta, torch.float64), _ptr(sv, torch.float32),
        ws.data_ptr(), ws.numel())
    _check("sd_schedule", code)
    return dict(ell=ell, batch=batch, n_sel=n_sel, theta=theta, surv=sv)


def sd_verify_workspace_size(R, gmax, V):
    return lib().sd_verify_workspace_size(R, gmax, V)


@_on_stream
def sd_verify(tgt, tgt_row0, drf, drf_row0, draft_tokens, ell, V, temperature=1.0, seed=0,
              pos0=None, probe=False, stats=False, alpha=False, workspace=None, out=None,
              stream=None, prof_events=None, drf_stats=None, stop_at_rejection=False):
    """Run verification.  tgt / drf: 2-D logit tensors (bf16 or fp32, ld =
    shape[1]); the rest int32 device tensors.  Returns a dict of device
    tensors: n_acc, tokens, status (and probe, row_stats, alpha if asked).
    prof_events: optional pair of raw hipEvent_t handles (ints) recorded
    around the row-statistics pass.  drf_stats: optional [R][gamma_max][2]
    fp32 (m, Z) of the draft rows (a drafting head's q_stats); the draft rows
    are then read only where needed.  stop_at_rejection: read each request's
    rows in rounds of positions and stop at its first rejection
    (SD_VERIFY_STOP_AT_REJECTION; alpha must be off)."""
    R, gmax = draft_tokens.shape
    if drf_stats is not None and drf_stats.numel() != R * gmax * 2:
        raise ValueError("drf_stats must hold R * gamma_max (m, Z) pairs")
    dev = tgt.device
    if tgt.dtype == torch.bfloat16:
        dt = SD_DTYPE_BF16
    elif tgt.dtype == torch.float32:
        dt = SD_DTYPE_F32
    else:
        raise TypeError("logits must be bf16 or fp32")
    if drf.dtype != tgt.dtype or drf.shape[1] != tgt.shape[1]:
        raise ValueError("target and draft rows must share dtype and leading dimension")
    ld = tgt.shape[1]
    o = out or {}
    n_acc = _out(o, "n_acc", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    toks = _out(o, "tokens", lambda: torch.empty((R, gmax + 1), dtype=torch.int32, device=dev))
    status = _out(o, "status", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    pp = _out(o, "probe", lambda: torch.zeros((R, gmax, 2), dtype=torch.float32, device=dev)) if probe else None
    rs = _out(o, "row_stats", lambda: torch.zeros((R, 2 * gmax + 1, 2), dtype=torch.float32, device=dev)) if stats else None
    al = _out(o, "alpha", lambda: torch.zeros((R, gmax), dtype=torch.float32, device=dev)) if alpha else None
    ws = workspace if workspace is not None else _workspace(sd_verify_workspace_size(R, gmax, V), dev)
    code = lib().sd_verify(
        _stream(stream), R, gmax, int(V), ld, dt, float(temperature), int(seed) & (2**64 - 1),
        _ptr(pos0, torch.int64, "pos0"), _ptr(tgt, None, "tgt"), _ptr(tgt_row0, torch.int32, "tgt_row0"),
        _ptr(drf, None, "drf"), _ptr(drf_row0, torch.int32, "drf_row0"),
        _ptr(drf_stats, torch.float32, "drf_stats"),
        _ptr(draft_tokens, torch.int32, "draft_tokens"), _ptr(ell, torch.int32, "ell"),
        _ptr(n_acc, torch.int32), _ptr(toks, torch.int32), _ptr(status, torch.int32),
        _ptr(pp, torch.float32), _ptr(rs, torch.float32), _ptr(al, torch.float32),
        SD_VERIFY_STOP_AT_REJECTION if stop_at_rejection else 0, ws.data_ptr(), ws.numel(),
        *(prof_events if prof_events else (None, None)))
    _check("sd_verify", code)
    return dict(n_acc=n_acc, tokens=toks, status=status, probe=pp, row_stats=rs, alpha=al)


@_on_stream
def sd_verify_noalloc(tgt, tgt_row0, drf, drf_row0, draft_tokens, ell, V, temperature=1.0, seed=0,
                      pos0=None, drf_stats=None, stop_at_rejection=False, out=None, stream=None):
    """sd_verify through the entry point that allocates nothing: the library
    holds the workspace.  The caller passes every output in `out` (n_acc,
    tokens, status, and optionally probe, row_stats, alpha), as a caller
    that cannot allocate would; returns `out`."""
    R, gmax = draft_tokens.shape
    if tgt.dtype == torch.bfloat16:
        dt = SD_DTYPE_BF16
    elif tgt.dtype == torch.float32:
        dt = SD_DTYPE_F32
    else:
        raise TypeError("logits must be bf16 or fp32")
    if drf.dtype != tgt.dtype or drf.shape[1] != tgt.shape[1]:
        raise ValueError("target and draft rows must share dtype and leading dimension")
    o = out
    code = lib().sd_verify_noalloc(
        _stream(stream), R, gmax, int(V), tgt.shape[1], dt, float(temperature), int(seed) & (2**64 - 1),
        _ptr(pos0, torch.int64, "pos0"), _ptr(tgt, None, "tgt"), _ptr(tgt_row0, torch.int32, "tgt_row0"),
        _ptr(drf, None, "drf"), _ptr(drf_row0, torch.int32, "drf_row0"),
        _ptr(drf_stats, torch.float32, "drf_stats"),
        _ptr(draft_tokens, torch.int32, "draft_tokens"), _ptr(ell, torch.int32, "ell"),
        _ptr(o["n_acc"], torch.int32, "n_acc"), _ptr(o["tokens"], torch.int32, "tokens"),
        _ptr(o["status"], torch.int32, "status"), _ptr(o.get("probe"), torch.float32, "probe"),
        _ptr(o.get("row_stats"), torch.float32, "row_stats"), _ptr(o.get("alpha"), torch.float32, "alpha"),
        SD_VERIFY_STOP_AT_REJECTION if stop_at_rejection else 0)
    _check("sd_verify_noalloc", code)
    return o


def sd_markov_draft_workspace_size(R, gamma, V, rank):
    return lib().sd_markov_draft_workspace_size(R, gamma, V, rank)


@_on_stream
def sd_markov_draft(U, A, Ct, x0, h, E, w, temperature=1.0, seed=0, pos0=None, workspace=None,
                    out=None, stream=None, stats=False):
    """Run the Markov drafting head.  Returns a dict of device tensors:
    tokens [R][gamma], q_logits [R][gamma][V] bf16, conf [R][gamma], status [R],
    and q_stats [R][gamma][2] ((m, Z) of each drafted row) if stats."""
    R, gamma, V = U.shape
    rank = A.shape[2]
    H = h.shape[2]
    rank_e = E.shape[1]
    dev = U.device
    bf = torch.bfloat16
    o = out or {}
    tokens = _out(o, "tokens", lambda: torch.empty((R, gamma), dtype=torch.int32, device=dev))
    ql = _out(o, "q_logits", lambda: torch.empty((R, gamma, V), dtype=bf, device=dev))
    conf = _out(o, "conf", lambda: torch.empty((R, gamma), dtype=torch.float32, device=dev))
    status = _out(o, "status", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    qs = _out(o, "q_stats", lambda: torch.empty((R, gamma, 2), dtype=torch.float32, device=dev)) if stats else None
    ws = workspace if workspace is not None else _workspace(sd_markov_draft_workspace_size(R, gamma, V, rank), dev)
    code = lib().sd_markov_draft(
        _stream(stream), R, gamma, V, rank, float(temperature), int(seed) & (2**64 - 1),
        _ptr(pos0, torch.int64, "pos0"), _ptr(U, bf, "U"), _ptr(A, bf, "A"), _ptr(Ct, bf, "Ct"),
        _ptr(x0, torch.int32, "x0"), _ptr(h, bf, "h"), H, _ptr(E, bf, "E"), rank_e,
        _ptr(w, torch.float32, "w"), _ptr(tokens, torch.int32), _ptr(ql, bf),
        _ptr(qs, torch.float32, "q_stats"), _ptr(conf, torch.float32), _ptr(status, torch.int32),
        ws.data_ptr(), ws.numel())
    _check("sd_markov_draft", code)
    return dict(tokens=tokens, q_logits=ql, conf=conf, status=status, q_stats=qs)


def sd_rnn_draft_workspace_size(R, gamma, V, d):
    return lib().sd_rnn_draft_workspace_size(R, gamma, V, d)


@_on_stream
def sd_rnn_draft(U, W, Es, Ct, x0, h, E, w, temperature=1.0, seed=0, pos0=None, workspace=None,
                 out=None, stream=None, stats=False):
    """Run the RNN drafting head.  Returns a dict of device tensors:
    tokens [R][gamma], q_logits [R][gamma][V] bf16, conf [R][gamma], status [R],
    and q_stats [R][gamma][2] ((m, Z) of each drafted row) if stats."""
    R, gamma, V = U.shape
    d = W.shape[0]
    H = h.shape[2]
    rank_e = E.shape[1]
    dev = U.device
    bf = torch.bfloat16
    o = out or {}
    tokens = _out(o, "tokens", lambda: torch.empty((R, gamma), dtype=torch.int32, device=dev))
    ql = _out(o, "q_logits", lambda: torch.empty((R, gamma, V), dtype=bf, device=dev))
    conf = _out(o, "conf", lambda: torch.empty((R, gamma), dtype=torch.float32, device=dev))
    status = _out(o, "status", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    qs = _out(o, "q_stats", lambda: torch.empty((R, gamma, 2), dtype=torch.float32, device=dev)) if stats else None
    ws = workspace if workspace is not None else _workspace(sd_rnn_draft_workspace_size(R, gamma, V, d),
                                                            dev)
    code = lib().sd_rnn_draft(
        _stream(stream), R, gamma, V, d, float(temperature), int(seed) & (2**64 - 1),
        _ptr(pos0, torch.int64, "pos0"), _ptr(U, bf, "U"), _ptr(W, bf, "W"), _ptr(Es, bf, "Es"),
        _ptr(Ct, bf, "Ct"), _ptr(x0, torch.int32, "x0"), _ptr(h, bf, "h"), H, _ptr(E, bf, "E"), rank_e,
        _ptr(w, torch.float32, "w"), _ptr(tokens, torch.int32), _ptr(ql, bf),
        _ptr(qs, torch.float32, "q_stats"), _ptr(conf, torch.float32), _ptr(status, torch.int32),
        ws.data_ptr(), ws.numel())
    _check("sd_rnn_draft", code)
    return dict(tokens=tokens, q_logits=ql, conf=conf, status=status, q_stats=qs)


@_on_stream
def sd_uniforms(seed, req, pos, draw, out=None, stream=None):
    """The uniforms u(seed, req[i], pos[i], draw) the library's decisions
    draw (req, pos int64 device tensors of one length).  Returns fp32."""
    n = req.numel()
    if pos.numel() != n:
        raise ValueError("req and pos must have the same length")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=req.device)
    _check("sd_uniforms", lib().sd_uniforms(_stream(stream), int(seed) & (2**64 - 1), n,
                                            _ptr(req, torch.int64, "req"), _ptr(pos, torch.int64, "pos"),
                                            int(draw), _ptr(out, torch.float32, "out")))
    return out


@_on_stream
def sd_lightspec_update(alpha, ell, status, lam, ema, count, stream=None):
    """Fold one verify step's acceptance probabilities alpha [R][gmax] fp32
    into the per-position EMA state ema [gmax] fp64 / count [gmax] int64
    (updated in place on the device)."""
    R, gmax = alpha.shape
    _check("sd_lightspec_update", lib().sd_lightspec_update(
        _stream(stream), R, gmax, _ptr(alpha, torch.float32, "alpha"), _ptr(ell, torch.int32, "ell"),
        _ptr(status, torch.int32, "status"), float(lam), _ptr(ema, torch.float64, "ema"),
        _ptr(count, torch.int64, "count")))


@_on_stream
def sd_lightspec_plan(ema, count, d_prev, sps, draft_cost, out=None, workspace=None, stream=None):
    """Both planning stages.  d_prev [R] int32 (the previous round's draft
    lengths).  Returns a dict of device tensors: conf (planning confidences),
    ell, batch, n_sel, theta (stage 1), d_next, b_next, phi (stage 2)."""
    gmax = ema.shape[0]
    R = d_prev.shape[0]
    dev = ema.device
    o = out or {}
    conf = _out(o, "conf", lambda: torch.empty(gmax, dtype=torch.float32, device=dev))
    ell = _out(o, "ell", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    batch = _out(o, "batch", lambda: torch.empty(1, dtype=torch.int32, device=dev))
    n_sel = _out(o, "n_sel", lambda: torch.empty(1, dtype=torch.int32, device=dev))
    theta = _out(o, "theta", lambda: torch.empty(1, dtype=torch.float64, device=dev))
    d_next = _out(o, "d_next", lambda: torch.empty(1, dtype=torch.int32, device=dev))
    b_next = _out(o, "b_next", lambda: torch.empty(1, dtype=torch.int32, device=dev))
    phi = _out(o, "phi", lambda: torch.empty(gmax, dtype=torch.float64, device=dev))
    ws = workspace if workspace is not None else _workspace(lib().sd_lightspec_plan_workspace_size(R, gmax), dev)
    _check("sd_lightspec_plan", lib().sd_lightspec_plan(
        _stream(stream), R, gmax, _ptr(ema, torch.float64, "ema"), _ptr(count, torch.int64, "count"),
        _ptr(d_prev, torch.int32, "d_prev"), _ptr(sps, torch.float32, "sps"), sps.numel(),
        _ptr(draft_cost, torch.float32, "draft_cost"), _ptr(conf, torch.float32),
        _ptr(ell, torch.int32), _ptr(batch, torch.int32), _ptr(n_sel, torch.int32),
        _ptr(theta, torch.float64), _ptr(d_next, torch.int32), _ptr(b_next, torch.int32),
        _ptr(phi, torch.float64), ws.data_ptr(), ws.numel()))
    return dict(conf=conf, ell=ell, batch=batch, n_sel=n_sel, theta=theta, d_next=d_next,
                b_next=b_next, phi=phi)
