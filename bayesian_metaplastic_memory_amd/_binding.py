"""ctypes binding over libpalimpsa.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/palimpsa.h``).  torch supplies device
memory and the current HIP stream.  There is no fallback: if the library is
missing or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpalimpsa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_HIP = range(5)
F32, BF16 = 0, 1
_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}

_lock = threading.Lock()
_lib = None


class PalimpsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, status_string(status), status))


def load_library() -> ctypes.CDLL:
    """Load libpalimpsa.so from the package directory (raises if it is missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    "libpalimpsa.so is not built; run `python -m bayesian_metaplastic_memory_amd.build` "
                    "(or __graft_entry__.build())")
            lib = ctypes.CDLL(LIB_PATH)
            vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
            sz = ctypes.c_size_t
            lib.palimpsa_fwd_chunked.argtypes = ([vp] * 5 + [fp] * 4 + [vp, fp, fp] + [i] * 10 +
                                                 [vp, sz, vp])
            lib.palimpsa_fwd_chunked.restype = i
            lib.palimpsa_fwd_chunked_noalloc.argtypes = ([vp] * 5 + [fp] * 4 + [vp, fp, fp] + [i] * 10 + [vp])
            lib.palimpsa_fwd_chunked_noalloc.restype = i
            lib.palimpsa_noalloc_scratch_bytes.argtypes = []
            lib.palimpsa_noalloc_scratch_bytes.restype = sz
            lib.palimpsa_fwd_workspace_size.argtypes = [i] * 6
            lib.palimpsa_fwd_workspace_size.restype = sz
            lib.palimpsa_fwd_frozen.argtypes = [vp] * 5 + [fp] * 3 + [vp, fp] + [i] * 7 + [vp]
            lib.palimpsa_fwd_frozen.restype = i
            lib.palimpsa_step.argtypes = [vp] * 5 + [fp] * 4 + [vp] + [i] * 7 + [vp]
            lib.palimpsa_step.restype = i
            lib.palimpsa_bwd.argtypes = [vp] * 5 + [fp] * 4 + [vp, fp, fp] + [fp] * 9 + [i] * 8 + [vp, sz, vp]
            lib.palimpsa_bwd.restype = i
            lib.palimpsa_bwd_workspace_size.argtypes = [i] * 6
            lib.palimpsa_bwd_frozen.argtypes = [vp] * 5 + [fp] * 3 + [vp, fp] + [fp] * 8 + [i] * 7 + [vp, sz, vp]
            lib.palimpsa_bwd_frozen.restype = i
            lib.palimpsa_bwd_workspace_size.restype = sz
            lib.palimpsa_fwd_blockdiag.argtypes = [vp] * 5 + [fp] * 4 + [vp, fp, fp] + [i] * 9 + [vp, sz, vp]
            lib.palimpsa_fwd_blockdiag.restype = i
            lib.palimpsa_step_blockdiag.argtypes = [vp] * 5 + [fp] * 4 + [vp] + [i] * 7 + [vp]
            lib.palimpsa_step_blockdiag.restype = i
            lib.palimpsa_bwd_blockdiag_workspace_size.argtypes = [i] * 6
            lib.palimpsa_bwd_blockdiag_workspace_size.restype = sz
            lib.palimpsa_bwd_blockdiag.argtypes = ([vp] * 5 + [fp] * 4 + [vp, fp, fp] + [fp] * 9 + [i] * 6 +
                                                   [i, i, i, vp, sz, vp])
            lib.palimpsa_bwd_blockdiag.restype = i
            lib.palimpsa_status_string.argtypes = [i]
            lib.palimpsa_status_string.restype = ctypes.c_char_p
            lib.palimpsa_version.argtypes = []
            lib.palimpsa_version.restype = i
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().palimpsa_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().palimpsa_version())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def check_params(A, I_prior, dt=None, beta=None, I0=None):
    """Check the data preconditions the library does not check itself (they
    live in device memory): A >= 0 and finite, I_prior > 0 and finite, and if
    given dt >= 0, beta >= 0, I0 > 0, all finite.  Raises ValueError naming
    the first violation.  Opt-in, since it reads the values back to the host
    (one synchronisation per tensor); call it once per set of parameters, not
    per step."""
    def bad(t, positive):
        x = t.detach().float()
        lo = (x <= 0) if positive else (x < 0)
        return bool((~torch.isfinite(x)).any().item()) or bool(lo.any().item())
    for t, name, positive in ((A, "A", False), (I_prior, "I_prior", True), (dt, "dt", False),
                              (beta, "beta", False), (I0, "I0", True)):
        if t is not None and bad(t, positive):
            raise ValueError("%s must be finite and %s" % (name, "> 0" if positive else ">= 0"))


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


VSTAR, PRIOR_PER_ENTRY, SAVE_CHECKPOINTS, CHECKPOINTS_SAVED = 1, 2, 4, 8


def _prior_flags(I_prior, H, dv, dk, dev, vstar):
    """Option bits from the prior's shape ([H] or [H, dv, dk]) and ``vstar``."""
    if tuple(I_prior.shape) == (H,):
        f = 0
    elif tuple(I_prior.shape) == (H, dv, dk):
        f = PRIOR_PER_ENTRY
    else:
        raise ValueError("I_prior must be [H] or [H, dv, dk]")
    _check(I_prior, "I_prior", tuple(I_prior.shape), torch.float32, dev)
    return f | (VSTAR if vstar else 0)


def workspace_size(B, T, H, dk, dv, segments: int = 0) -> int:
    """Bytes of workspace the chunked forward uses for these sizes (0: none)."""
    return int(load_library().palimpsa_fwd_workspace_size(B, T, H, dk, dv, int(segments)))


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed per-GPU scratch array of ``fwd_chunked_noalloc``."""
    return int(load_library().palimpsa_noalloc_scratch_bytes())


def fwd_chunked_noalloc(q, k, v, beta, dt, A, I_prior, mu0=None, I0=None, chunk: int = 0,
                        out_dtype=None, y=None, muT=None, IT=None, write_state: bool = True,
                        segments: int = 0, vstar: bool = False):
    """``fwd_chunked`` through ``palimpsa_fwd_chunked_noalloc``: no workspace;
    a time split uses the library's fixed scratch array on the device.  The C
    call allocates nothing (outputs not passed in are allocated here, by
    torch, before it)."""
    return fwd_chunked(q, k, v, beta, dt, A, I_prior, mu0=mu0, I0=I0, chunk=chunk, out_dtype=out_dtype,
                       y=y, muT=muT, IT=IT, write_state=write_state, segments=segments, vstar=vstar,
                       _noalloc=True)


def fwd_chunked(q, k, v, beta, dt, A, I_prior, mu0=None, I0=None, chunk: int = 0,
                out_dtype=None, y=None, muT=None, IT=None, write_state: bool = True,
                segments: int = 0, workspace=None, vstar: bool = False,
                save_checkpoints: bool = False, _noalloc: bool = False):
    """Chunked forward.  Returns ``(y, muT, IT)``; ``muT``/``IT`` are None when
    ``write_state`` is False.  Outputs are allocated unless passed in (they may
    alias ``mu0``/``I0`` for an in-place resume).  ``segments`` (0 = library's
    choice) selects the time split; its workspace is allocated here unless a
    uint8 device tensor is passed as ``workspace``.  ``I_prior`` is ``[H]`` or
    ``[H, dv, dk]`` (a prior per state entry); ``vstar`` means ``v`` holds
    ``beta * v``.

    ``save_checkpoints`` (the training forward): ``workspace`` must then be a
    backward workspace (``bwd_workspace_size`` bytes), into which the forward
    also stores the states the backward needs; pass it to ``bwd`` with
    ``checkpoints_saved=True`` to skip their recomputation."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % in_dtype)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    _check(k, "k", (B, T, H, dk), in_dtype, dev)
    _check(v, "v", (B, T, H, dv), in_dtype, dev)
    _check(beta, "beta", (B, T, H, dv), in_dtype, dev)
    _check(dt, "dt", (B, T, H), in_dtype, dev)
    _check(q, "q", (B, T, H, dk), in_dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    flags = _prior_flags(I_prior, H, dv, dk, dev, vstar)
    if save_checkpoints:
        if workspace is None:
            raise ValueError("save_checkpoints needs a backward workspace (bwd_workspace_size bytes)")
        flags |= SAVE_CHECKPOINTS
    if (mu0 is None) != (I0 is None):
        raise ValueError("give both mu0 and I0, or neither")
    if mu0 is not None:
        _check(mu0, "mu0", (B, H, dv, dk), torch.float32, dev)
        _check(I0, "I0", (B, H, dv, dk), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _check(y, "y", (B, T, H, dv), out_dtype, dev)
    if write_state:
        if muT is None:
            muT = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        if IT is None:
            IT = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        _check(muT, "muT", (B, H, dv, dk), torch.float32, dev)
        _check(IT, "IT", (B, H, dv, dk), torch.float32, dev)
    else:
        muT = IT = None
    lib = load_library()
    if _noalloc:
        with torch.cuda.device(dev):
            st = lib.palimpsa_fwd_chunked_noalloc(
                _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt), _ptr(A), _ptr(I_prior),
                _ptr(mu0), _ptr(I0), _ptr(y) if y.numel() else None,
                _ptr(muT), _ptr(IT), B, T, H, dk, dv, int(chunk), int(segments),
                _DTYPES[in_dtype], _DTYPES[out_dtype], flags, _stream_handle(dev))
        if st != OK:
            raise PalimpsaError(st, "palimpsa_fwd_chunked_noalloc")
        return y, muT, IT
    if workspace is None:
        nbytes = workspace_size(B, T, H, dk, dv, segments)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    with torch.cuda.device(dev):
        st = lib.palimpsa_fwd_chunked(
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt), _ptr(A), _ptr(I_prior),
            _ptr(mu0), _ptr(I0), _ptr(y) if y.numel() else None,
            _ptr(muT), _ptr(IT), B, T, H, dk, dv, int(chunk), int(segments),
            _DTYPES[in_dtype], _DTYPES[out_dtype], flags,
            _ptr(workspace) if workspace is not None and workspace.numel() else None,
            workspace.numel() if workspace is not None else 0, _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_fwd_chunked")
    return y, muT, IT


def step(q, k, v, beta, dt, A, I_prior, mu, I, out_dtype=None, y=None, vstar: bool = False):
    """One decode token; updates ``mu`` and ``I`` in place and returns ``y``.
    ``I_prior`` is ``[H]`` or ``[H, dv, dk]``; ``vstar`` as in ``fwd_chunked``."""
    if q.dim() != 3:
        raise ValueError("q must be [B, H, dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % in_dtype)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    _check(k, "k", (B, H, dk), in_dtype, dev)
    _check(v, "v", (B, H, dv), in_dtype, dev)
    _check(beta, "beta", (B, H, dv), in_dtype, dev)
    _check(dt, "dt", (B, H), in_dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    flags = _prior_flags(I_prior, H, dv, dk, dev, vstar)
    _check(mu, "mu", (B, H, dv, dk), torch.float32, dev)
    _check(I, "I", (B, H, dv, dk), torch.float32, dev)
    if y is None:
        y = torch.empty((B, H, dv), dtype=out_dtype, device=dev)
    else:
        _check(y, "y", (B, H, dv), out_dtype, dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.palimpsa_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt), _ptr(A),
                               _ptr(I_prior), _ptr(mu), _ptr(I), _ptr(y), B, H, dk, dv,
                               _DTYPES[in_dtype], _DTYPES[out_dtype], flags, _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_step")
    return y


def fwd_frozen(q, k, v, beta, dt, A, I_prior, mu0=None, out_dtype=None, y=None, muT=None,
               write_state: bool = True):
    """Frozen-importance (Mamba2-limit) forward on the matrix cores.  ``beta``
    may be None when ``v`` already holds beta * v.  Returns ``(y, muT)``."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % in_dtype)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    _check(k, "k", (B, T, H, dk), in_dtype, dev)
    _check(v, "v", (B, T, H, dv), in_dtype, dev)
    if beta is not None:
        _check(beta, "beta", (B, T, H, dv), in_dtype, dev)
    _check(dt, "dt", (B, T, H), in_dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(I_prior, "I_prior", (H,), torch.float32, dev)
    if mu0 is not None:
        _check(mu0, "mu0", (B, H, dv, dk), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _check(y, "y", (B, T, H, dv), out_dtype, dev)
    if write_state:
        if muT is None:
            muT = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        _check(muT, "muT", (B, H, dv, dk), torch.float32, dev)
    else:
        muT = None
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.palimpsa_fwd_frozen(
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt), _ptr(A), _ptr(I_prior), _ptr(mu0),
            _ptr(y) if y.numel() else None, _ptr(muT), B, T, H, dk, dv,
            _DTYPES[in_dtype], _DTYPES[out_dtype], _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_fwd_frozen")
    return y, muT


def bwd_workspace_size(B, T, H, dk, dv, flags: int = 0) -> int:
    """Bytes of workspace ``palimpsa_bwd`` needs (checkpoints and partials)."""
    return int(load_library().palimpsa_bwd_workspace_size(B, T, H, dk, dv, int(flags)))


def bwd(q, k, v, beta, dt, A, I_prior, gy, mu0=None, I0=None, gmuT=None, gIT=None,
        want_state_grads: bool = True, workspace=None, out=None, vstar: bool = False,
        checkpoints_saved: bool = False):
    """Backward of ``fwd_chunked`` for ``L = <gy, y> + <gmuT, muT> + <gIT, IT>``.

    Takes the forward's inputs (the library recomputes the states) and returns
    a dict of float32 gradients ``gq, gk, gv, gbeta, gdt, gA, gIp`` and, if
    ``want_state_grads``, ``gmu0, gI0``.  ``gmuT``/``gIT`` may be None (zero).
    ``out`` may supply preallocated output tensors by the same names;
    ``workspace`` a contiguous uint8 device tensor of at least
    ``bwd_workspace_size`` bytes (allocated here otherwise).  With a prior per
    state entry (``I_prior`` ``[H, dv, dk]``) ``gIp`` has that shape; with
    ``vstar`` (``v`` holds ``beta * v``) ``gv`` is the gradient w.r.t. it.
    ``checkpoints_saved``: ``workspace`` holds the checkpoints a
    ``fwd_chunked(..., save_checkpoints=True)`` call on the same inputs stored,
    and the backward skips recomputing them."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES or gy.dtype not in _DTYPES:
        raise ValueError("unsupported dtype")
    for t, name, shape in ((k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (beta, "beta", (B, T, H, dv)),
                           (dt, "dt", (B, T, H))):
        _check(t, name, shape, in_dtype, dev)
    _check(gy, "gy", (B, T, H, dv), gy.dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    flags = _prior_flags(I_prior, H, dv, dk, dev, vstar)
    if checkpoints_saved:
        if workspace is None:
            raise ValueError("checkpoints_saved needs the workspace the training forward filled")
        flags |= CHECKPOINTS_SAVED
    if (mu0 is None) != (I0 is None):
        raise ValueError("give both mu0 and I0, or neither")
    for t, name in ((mu0, "mu0"), (I0, "I0"), (gmuT, "gmuT"), (gIT, "gIT")):
        if t is not None:
            _check(t, name, (B, H, dv, dk), torch.float32, dev)
    shapes = {"gq": (B, T, H, dk), "gk": (B, T, H, dk), "gv": (B, T, H, dv), "gbeta": (B, T, H, dv),
              "gdt": (B, T, H), "gA": (H,), "gIp": tuple(I_prior.shape)}
    if want_state_grads:
        shapes.update(gmu0=(B, H, dv, dk), gI0=(B, H, dv, dk))
    res = {}
    for name, shape in shapes.items():
        t = (out or {}).get(name)
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=dev)
        _check(t, name, shape, torch.float32, dev)
        res[name] = t
    lib = load_library()
    nbytes = bwd_workspace_size(B, T, H, dk, dv, flags)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    nz = lambda t: _ptr(t) if t is not None and t.numel() else None
    with torch.cuda.device(dev):
        st = lib.palimpsa_bwd(
            nz(q), nz(k), nz(v), nz(beta), nz(dt), _ptr(A), _ptr(I_prior), _ptr(mu0), _ptr(I0),
            nz(gy), _ptr(gmuT), _ptr(gIT),
            nz(res["gq"]), nz(res["gk"]), nz(res["gv"]), nz(res["gbeta"]), nz(res["gdt"]),
            _ptr(res["gA"]), _ptr(res["gIp"]), _ptr(res.get("gmu0")), _ptr(res.get("gI0")),
            B, T, H, dk, dv, _DTYPES[in_dtype], _DTYPES[gy.dtype], flags,
            _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_bwd")
    return res


def bwd_frozen(q, k, v, beta, dt, A, I_prior, gy, mu0=None, gmuT=None, want_state_grads: bool = True,
               workspace=None, out=None):
    """Backward of ``fwd_frozen`` (frozen importance) for ``L = <gy, y> + <gmuT, muT>``.

    Takes the forward's inputs and returns a dict of float32 gradients ``gq,
    gk, gv, gbeta, gdt, gA, gIp`` and, if ``want_state_grads``, ``gmu0``.
    ``beta`` None means ``v`` holds the write ``beta * v``; ``gv`` is then the
    gradient w.r.t. it and ``gbeta`` is None.  ``out`` and ``workspace`` as in
    ``bwd`` (workspace: ``bwd_workspace_size(B, T, H, dk, dv)`` bytes)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES or gy.dtype not in _DTYPES:
        raise ValueError("unsupported dtype")
    for t, name, shape in ((k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (dt, "dt", (B, T, H))):
        _check(t, name, shape, in_dtype, dev)
    if beta is not None:
        _check(beta, "beta", (B, T, H, dv), in_dtype, dev)
    _check(gy, "gy", (B, T, H, dv), gy.dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(I_prior, "I_prior", (H,), torch.float32, dev)
    for t, name in ((mu0, "mu0"), (gmuT, "gmuT")):
        if t is not None:
            _check(t, name, (B, H, dv, dk), torch.float32, dev)
    shapes = {"gq": (B, T, H, dk), "gk": (B, T, H, dk), "gv": (B, T, H, dv), "gdt": (B, T, H), "gA": (H,),
              "gIp": (H,)}
    if beta is not None:
        shapes["gbeta"] = (B, T, H, dv)
    if want_state_grads:
        shapes["gmu0"] = (B, H, dv, dk)
    res = {}
    for name, shape in shapes.items():
        t = (out or {}).get(name)
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=dev)
        _check(t, name, shape, torch.float32, dev)
        res[name] = t
    lib = load_library()
    nbytes = bwd_workspace_size(B, T, H, dk, dv, 0)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    nz = lambda t: _ptr(t) if t is not None and t.numel() else None
    with torch.cuda.device(dev):
        st = lib.palimpsa_bwd_frozen(
            nz(q), nz(k), nz(v), nz(beta), nz(dt), _ptr(A), _ptr(I_prior), _ptr(mu0), nz(gy), _ptr(gmuT),
            nz(res["gq"]), nz(res["gk"]), nz(res["gv"]), nz(res.get("gbeta")), nz(res["gdt"]),
            _ptr(res["gA"]), _ptr(res["gIp"]), _ptr(res.get("gmu0")),
            B, T, H, dk, dv, _DTYPES[in_dtype], _DTYPES[gy.dtype],
            _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_bwd_frozen")
    res.setdefault("gbeta", None)
    return res


def fwd_blockdiag(q, k, v, beta, dt, A, I_prior, block: int = 2, mu0=None, P0=None, out_dtype=None,
                  y=None, muT=None, PT=None, write_state: bool = True, save_checkpoints: bool = False,
                  workspace=None):
    """Forward with the precision kept block-diagonal along the key axis
    (``block`` = 2, or 4 with d_k of 64 or 128).  Returns ``(y, muT, PT)`` with
    ``PT`` ``[B, H, dv, dk/block, block, block]``; ``mu0``/``P0`` likewise
    (both or neither).  ``save_checkpoints`` (the training forward) also stores
    the backward's checkpoints in ``workspace``, a contiguous uint8 device
    tensor of ``bwd_blockdiag_workspace_size`` bytes, for a following
    ``bwd_blockdiag(..., workspace=workspace, checkpoints_saved=True)``."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % in_dtype)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    for t, name, shape in ((k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (beta, "beta", (B, T, H, dv)),
                           (dt, "dt", (B, T, H))):
        _check(t, name, shape, in_dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(I_prior, "I_prior", (H,), torch.float32, dev)
    nb = dk // block if block > 0 else 0
    if (mu0 is None) != (P0 is None):
        raise ValueError("give both mu0 and P0, or neither")
    if mu0 is not None:
        _check(mu0, "mu0", (B, H, dv, dk), torch.float32, dev)
        _check(P0, "P0", (B, H, dv, nb, block, block), torch.float32, dev)
    if y is None:
        y = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    _check(y, "y", (B, T, H, dv), out_dtype, dev)
    if write_state:
        muT = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if muT is None else muT
        PT = torch.empty((B, H, dv, nb, block, block), dtype=torch.float32, device=dev) if PT is None else PT
        _check(muT, "muT", (B, H, dv, dk), torch.float32, dev)
        _check(PT, "PT", (B, H, dv, nb, block, block), torch.float32, dev)
    else:
        muT = PT = None
    if save_checkpoints:
        if workspace is None:
            raise ValueError("save_checkpoints needs a backward workspace (bwd_blockdiag_workspace_size bytes)")
        if workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    else:
        workspace = None
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.palimpsa_fwd_blockdiag(
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt), _ptr(A), _ptr(I_prior), _ptr(mu0), _ptr(P0),
            _ptr(y) if y.numel() else None, _ptr(muT), _ptr(PT), B, T, H, dk, dv, int(block),
            _DTYPES[in_dtype], _DTYPES[out_dtype], SAVE_CHECKPOINTS if save_checkpoints else 0,
            _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_fwd_blockdiag")
    return y, muT, PT


def step_blockdiag(q, k, v, beta, dt, A, I_prior, mu, P, block: int = 2, out_dtype=None, y=None):
    """One decode token of the block-diagonal-precision path; updates ``mu``
    ``[B, H, dv, dk]`` and ``P`` ``[B, H, dv, dk/block, block, block]`` in place
    and returns ``y`` ``[B, H, dv]``."""
    if q.dim() != 3:
        raise ValueError("q must be [B, H, dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES:
        raise ValueError("unsupported input dtype %s" % in_dtype)
    out_dtype = in_dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPES:
        raise ValueError("unsupported output dtype %s" % out_dtype)
    for t, name, shape in ((k, "k", (B, H, dk)), (v, "v", (B, H, dv)), (beta, "beta", (B, H, dv)), (dt, "dt", (B, H))):
        _check(t, name, shape, in_dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(I_prior, "I_prior", (H,), torch.float32, dev)
    nb = dk // block if block > 0 else 0
    _check(mu, "mu", (B, H, dv, dk), torch.float32, dev)
    _check(P, "P", (B, H, dv, nb, block, block), torch.float32, dev)
    if y is None:
        y = torch.empty((B, H, dv), dtype=out_dtype, device=dev)
    else:
        _check(y, "y", (B, H, dv), out_dtype, dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.palimpsa_step_blockdiag(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(dt), _ptr(A), _ptr(I_prior),
                                         _ptr(mu), _ptr(P), _ptr(y), B, H, dk, dv, int(block),
                                         _DTYPES[in_dtype], _DTYPES[out_dtype], _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_step_blockdiag")
    return y


def bwd_blockdiag_workspace_size(B, T, H, dk, dv, block: int = 2) -> int:
    """Bytes of workspace ``palimpsa_bwd_blockdiag`` needs (0 if unsupported)."""
    return int(load_library().palimpsa_bwd_blockdiag_workspace_size(B, T, H, dk, dv, int(block)))


def bwd_blockdiag(q, k, v, beta, dt, A, I_prior, gy, block: int = 2, mu0=None, P0=None, gmuT=None, gPT=None,
                  want_state_grads: bool = True, workspace=None, out=None, checkpoints_saved: bool = False):
    """Backward of ``fwd_blockdiag`` (``block`` 2, or 4 with d_k of 64 or 128) for
    ``L = <gy, y> + <gmuT, muT> + <gPT, PT>``.

    Returns a dict of float32 gradients ``gq, gk, gv, gbeta, gdt, gA, gIp`` and,
    if ``want_state_grads``, ``gmu0`` and ``gP0`` (the gradient for a
    symmetric P0).  ``gmuT``/``gPT`` may be None (zero); ``out`` and
    ``workspace`` as in ``bwd``.  ``checkpoints_saved``: ``workspace`` holds the
    checkpoints a ``fwd_blockdiag(..., save_checkpoints=True)`` call on the
    same inputs stored, and the checkpoint pass is skipped."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    in_dtype = q.dtype
    if in_dtype not in _DTYPES or gy.dtype not in _DTYPES:
        raise ValueError("unsupported dtype")
    for t, name, shape in ((k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (beta, "beta", (B, T, H, dv)),
                           (dt, "dt", (B, T, H))):
        _check(t, name, shape, in_dtype, dev)
    _check(gy, "gy", (B, T, H, dv), gy.dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(I_prior, "I_prior", (H,), torch.float32, dev)
    nb = dk // block if block > 0 else 0
    pshape = (B, H, dv, nb, block, block)
    for t, name, shape in ((mu0, "mu0", (B, H, dv, dk)), (P0, "P0", pshape), (gmuT, "gmuT", (B, H, dv, dk)),
                           (gPT, "gPT", pshape)):
        if t is not None:
            _check(t, name, shape, torch.float32, dev)
    shapes = {"gq": (B, T, H, dk), "gk": (B, T, H, dk), "gv": (B, T, H, dv), "gbeta": (B, T, H, dv),
              "gdt": (B, T, H), "gA": (H,), "gIp": (H,)}
    if want_state_grads:
        shapes["gmu0"] = (B, H, dv, dk)
        shapes["gP0"] = pshape
    res = {}
    for name, shape in shapes.items():
        t = (out or {}).get(name)
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=dev)
        _check(t, name, shape, torch.float32, dev)
        res[name] = t
    lib = load_library()
    nbytes = bwd_blockdiag_workspace_size(B, T, H, dk, dv, block)
    if checkpoints_saved and workspace is None:
        raise ValueError("checkpoints_saved needs the workspace the training forward wrote")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    nz = lambda t: _ptr(t) if t is not None and t.numel() else None
    with torch.cuda.device(dev):
        st = lib.palimpsa_bwd_blockdiag(
            nz(q), nz(k), nz(v), nz(beta), nz(dt), _ptr(A), _ptr(I_prior), _ptr(mu0), _ptr(P0), nz(gy),
            _ptr(gmuT), _ptr(gPT),
            nz(res["gq"]), nz(res["gk"]), nz(res["gv"]), nz(res["gbeta"]), nz(res["gdt"]),
            _ptr(res["gA"]), _ptr(res["gIp"]), _ptr(res.get("gmu0")), _ptr(res.get("gP0")),
            B, T, H, dk, dv, int(block), _DTYPES[in_dtype], _DTYPES[gy.dtype],
            CHECKPOINTS_SAVED if checkpoints_saved else 0, _ptr(workspace), workspace.numel(), _stream_handle(dev))
    if st != OK:
        raise PalimpsaError(st, "palimpsa_bwd_blockdiag")
    return res
