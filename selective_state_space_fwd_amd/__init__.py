"""MI355X (gfx950) selective state-space scan: Python binding of libssm.

The library (``libssm.so``, built from ``csrc/`` by ``build.py``) exports the
C ABI declared in ``include/ssm.h``.  This module only marshals arguments:
it checks tensor shapes and dtypes, allocates the outputs and the workspace
with PyTorch (device memory and streams are the only things torch provides),
and passes raw pointers plus the current HIP stream to the library.  Every
step of the computation runs in the HIP kernels; there is no fallback.

    y, last_state = ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias,
                                 softplus=True, return_last_state=True,
                                 initial_state=None, cu_seqlens=None)
    y = ssm_state_update(state, u, delta, A, B, C, D, z)   # state updated in place
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

__all__ = ["ssm_scan_fwd", "ssm_scan_fwd_conv", "ssm_scan_bwd", "ssm_state_update",
           "ckpt_shape", "PreparedCall", "ssm_scan_workspace_bytes", "ssm_scan_chunk_size", "scan_plan",
           "ssm_status_string", "SsmError", "load_library", "LIB_PATH"]

LIB_PATH = Path(__file__).resolve().parent / "libssm.so"

SSM_F32, SSM_BF16 = 0, 1


class SsmError(RuntimeError):
    """A libssm call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class SsmDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("d_inner", ctypes.c_int64),
        ("d_state", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("profile_begin", ctypes.c_void_p),
        ("profile_end", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


_lib = None


def load_library(path: str | os.PathLike | None = None) -> ctypes.CDLL:
    """Load libssm.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(
            f"{p} is missing: build the HIP library first "
            "(python -m selective_state_space_fwd_amd.build)")
    lib = ctypes.CDLL(str(p))
    vp, dp = ctypes.c_void_p, ctypes.POINTER(SsmDesc)
    lib.ssm_scan_workspace_bytes.argtypes = [dp]
    lib.ssm_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_chunk_size.argtypes = [dp]
    lib.ssm_scan_chunk_size.restype = ctypes.c_int64
    lib.ssm_scan_plan.argtypes = [dp]
    lib.ssm_scan_plan.restype = ctypes.c_char_p
    lib.ssm_scan_bwd_plan.argtypes = [dp, ctypes.c_int]
    lib.ssm_scan_bwd_plan.restype = ctypes.c_char_p
    lib.ssm_scan_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp,
                                         vp, vp]
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_scan_fwd_ex.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                    ctypes.c_int64, vp, vp, vp]
    lib.ssm_scan_fwd_ex.restype = ctypes.c_int
    lib.ssm_scan_fwd_conv.argtypes = [dp, vp, vp, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                      vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int64, vp,
                                      vp, vp, vp]
    lib.ssm_scan_fwd_conv.restype = ctypes.c_int
    lib.ssm_state_update.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssm_state_update.restype = ctypes.c_int
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [dp]
    lib.ssm_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_bwd.argtypes = [dp] + [vp] * 8 + [ctypes.c_int] + [vp] * 12 + [vp]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_bwd_ex.argtypes = ([dp] + [vp] * 8 + [ctypes.c_int] + [vp, vp, ctypes.c_int64] +
                                    [vp] * 12 + [vp])
    lib.ssm_scan_fwd_ckpt.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                      ctypes.c_int64, vp, vp, vp, vp]
    lib.ssm_scan_fwd_ckpt.restype = ctypes.c_int
    lib.ssm_scan_ckpt_bytes.argtypes = [dp]
    lib.ssm_scan_ckpt_bytes.restype = ctypes.c_size_t
    lib.ssm_scan_bwd_ex.restype = ctypes.c_int
    lib.ssm_status_string.argtypes = [ctypes.c_int]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_version.argtypes = []
    lib.ssm_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def ssm_status_string(status: int) -> str:
    return load_library().ssm_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise SsmError(status, ssm_status_string(status))


# ---------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _io_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return SSM_F32
    if dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"io dtype must be float32 or bfloat16, got {dtype}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _expect(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


class PreparedCall:
    """One entry point's call with its arguments checked and marshalled once:
    the descriptor, the device pointers and the stream.  Calling it enqueues
    the same work again on the same buffers, and returns what the plain call
    returns (the same output tensors).  For loops in which the binding's own
    checks would cost as much host time as the kernels take on the GPU.

    It holds a reference to every tensor it points at, so none is freed while
    it lives; new inputs are written into those tensors in place.  The stream
    is the one current when it was prepared, unless a call names another.
    """

    __slots__ = ("_fn", "desc", "_dref", "_args", "_keep", "result")

    def __init__(self, fn, desc, args, keep, result):
        self._fn, self.desc, self._args, self._keep, self.result = fn, desc, args, keep, result
        self._dref = ctypes.byref(desc)

    def __call__(self, profile_events=None, stream=None):
        """Enqueue the call; profile_events: optional pair of raw hipEvent_t
        handles for entry points that record them; stream: a raw hipStream_t
        to enqueue on instead of the prepared one (for instance the stream
        that a graph capture makes current)."""
        if profile_events is not None:
            self.desc.profile_begin, self.desc.profile_end = profile_events
        args = self._args if stream is None else self._args[:-1] + (stream,)
        st = self._fn(self._dref, *args)
        if st != 0:
            _check(st)
        return self.result


def _issue(prepare, fn, desc, args, keep, result):
    if prepare:
        return PreparedCall(fn, desc, args, keep, result)
    _check(fn(ctypes.byref(desc), *args))
    return result


SSM_FLAG_ZOH = 1
SSM_FLAG_INDEPENDENT_CHUNKS = 2


def _flags(zoh, independent_chunks):
    return (SSM_FLAG_ZOH if zoh else 0) | (SSM_FLAG_INDEPENDENT_CHUNKS if independent_chunks else 0)


def make_desc(batch, d_inner, d_state, seqlen, io_dtype, chunk_size=0, flags=0) -> SsmDesc:
    return SsmDesc(batch, d_inner, d_state, seqlen, io_dtype, chunk_size, None, 0, None, None,
                   flags, 0)


def ssm_scan_workspace_bytes(batch, d_inner, d_state, seqlen, io_dtype, chunk_size=0) -> int:
    d = make_desc(batch, d_inner, d_state, seqlen, io_dtype, chunk_size)
    return int(load_library().ssm_scan_workspace_bytes(ctypes.byref(d)))


def ssm_scan_chunk_size(batch, d_inner, d_state, seqlen, io_dtype, chunk_size=0) -> int:
    d = make_desc(batch, d_inner, d_state, seqlen, io_dtype, chunk_size)
    return int(load_library().ssm_scan_chunk_size(ctypes.byref(d)))


def scan_plan(batch, d_inner, d_state, seqlen, io_dtype, chunk_size=0) -> str:
    """The schedule ssm_scan_fwd runs for these shapes (ssm_scan_plan)."""
    d = make_desc(batch, d_inner, d_state, seqlen, io_dtype, chunk_size)
    return load_library().ssm_scan_plan(ctypes.byref(d)).decode()


def scan_bwd_plan(batch, d_inner, d_state, seqlen, io_dtype, chunk_size=0, zoh=False,
                  with_ckpt=False) -> str:
    """The schedule ssm_scan_bwd runs for these shapes, with or without the
    forward's checkpoints (ssm_scan_bwd_plan)."""
    d = make_desc(batch, d_inner, d_state, seqlen, io_dtype, chunk_size,
                  SSM_FLAG_ZOH if zoh else 0)
    return load_library().ssm_scan_bwd_plan(ctypes.byref(d), 1 if with_ckpt else 0).decode()


# ---------------------------------------------------------------- entry points

def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
                 return_last_state=True, chunk_size=0, y=None, last_state=None,
                 workspace=None, profile_events=None, initial_state=None, cu_seqlens=None,
                 zoh=False, independent_chunks=False, ckpt=None, prepare=False):
    """Fused selective-scan forward pass on the GPU.

    u, delta, z: (batch, d_inner, L); B, C: (batch, N, L), all float32 or all
    bfloat16.  A: (d_inner, N), D and delta_bias: (d_inner,), float32.
    initial_state: float32 start states, or None for zeros.
    cu_seqlens: optional int32 device tensor of n_seqs + 1 token offsets; the
    sequences are packed along L of a single batch row (batch must be 1) and
    the state starts over at each of them.  States (initial_state,
    last_state) have one row per batch row, or per sequence when packed:
    (rows, d_inner, N).
    zoh: zero-order-hold input term (exp(dt A) - 1) / A * B u instead of dt B u.
    independent_chunks: no chunk waits for the operators of the chunks before
    it; each computes them itself (same result bits, more work).
    ckpt: optional float32 tensor of shape ckpt_shape(batch, d_inner, L)
    (d_state <= 16): also filled with the state entering every 8-token tile,
    for ssm_scan_bwd(ckpt=...).
    prepare: check and marshal everything but launch nothing; return a
    PreparedCall that launches this call each time it is called.
    Returns (y, last_state); last_state is None unless requested.
    profile_events: optional pair of raw hipEvent_t handles, recorded at the
    start of the scan's first kernel and the end of its last.
    """
    torch = _torch()
    lib = load_library()
    batch, d_inner, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev, io = u.device, u.dtype
    code = _io_code(io)
    _expect(u, "u", (batch, d_inner, L), io, dev)
    _expect(delta, "delta", (batch, d_inner, L), io, dev)
    _expect(A, "A", (d_inner, N), torch.float32, dev)
    _expect(B, "B", (batch, N, L), io, dev)
    _expect(C, "C", (batch, N, L), io, dev)
    _expect(D, "D", (d_inner,), torch.float32, dev)
    _expect(z, "z", (batch, d_inner, L), io, dev)
    _expect(delta_bias, "delta_bias", (d_inner,), torch.float32, dev)
    n_seqs = 0
    rows = batch
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must hold n_seqs + 1 >= 2 offsets")
        n_seqs = cu_seqlens.numel() - 1
        _expect(cu_seqlens, "cu_seqlens", (n_seqs + 1,), torch.int32, dev)
        rows = n_seqs
    _expect(initial_state, "initial_state", (rows, d_inner, N), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, d_inner, L), dtype=io, device=dev)
    _expect(y, "y", (batch, d_inner, L), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((rows, d_inner, N), dtype=torch.float32, device=dev)
    _expect(last_state, "last_state", (rows, d_inner, N), torch.float32, dev)
    desc = make_desc(batch, d_inner, N, L, code, chunk_size, _flags(zoh, independent_chunks))
    need = int(lib.ssm_scan_workspace_bytes(ctypes.byref(desc)))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    if profile_events is not None:
        desc.profile_begin, desc.profile_end = profile_events
    head = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(softplus)))
    if ckpt is not None:
        _expect(ckpt, "ckpt", ckpt_shape(batch, d_inner, L), torch.float32, dev)
        fn, args = lib.ssm_scan_fwd_ckpt, head + (_ptr(initial_state), _ptr(cu_seqlens), n_seqs,
                                                  _ptr(y), _ptr(last_state), _ptr(ckpt))
    elif initial_state is None and cu_seqlens is None:
        fn, args = lib.ssm_scan_fwd, head + (_ptr(y), _ptr(last_state))
    else:
        fn, args = lib.ssm_scan_fwd_ex, head + (_ptr(initial_state), _ptr(cu_seqlens), n_seqs,
                                                _ptr(y), _ptr(last_state))
    keep = (u, delta, A, B, C, D, z, delta_bias, initial_state, cu_seqlens, y, last_state, ckpt,
            workspace)
    return _issue(prepare, fn, desc, args + (_stream(dev),), keep, (y, last_state))


def ssm_scan_fwd_conv(x, conv_weight, conv_bias, delta, A, B, C, D=None, z=None,
                      delta_bias=None, softplus=True, conv_silu=True, conv_state=None,
                      initial_state=None, cu_seqlens=None, return_last_state=True,
                      return_u=False, chunk_size=0, y=None, last_state=None, u_out=None,
                      workspace=None, profile_events=None, zoh=False,
                      independent_chunks=False, prepare=False):
    """The scan with the causal depthwise convolution fused in front: the scan
    input is u = silu(conv(x) + conv_bias) (identity instead of silu when
    conv_silu is False), computed on the fly.

    x: (batch, d_inner, L) like u of ssm_scan_fwd; conv_weight: (d_inner, W)
    float32, W <= 4, column W-1 on the current token; conv_bias: (d_inner,) or
    None; conv_state: (rows, d_inner, W-1) float32 inputs before each
    sequence, or None for zeros.  Returns (y, last_state, u) with u only when
    return_u (else None).  prepare: as in ssm_scan_fwd.
    """
    torch = _torch()
    lib = load_library()
    batch, d_inner, L = x.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev, io = x.device, x.dtype
    code = _io_code(io)
    if conv_weight.dim() != 2 or conv_weight.shape[0] != d_inner:
        raise ValueError(f"conv_weight must be (d_inner, W), got {tuple(conv_weight.shape)}")
    W = conv_weight.shape[1]
    for t, name, shape in ((x, "x", (batch, d_inner, L)), (delta, "delta", (batch, d_inner, L)),
                           (B, "B", (batch, N, L)), (C, "C", (batch, N, L)),
                           (z, "z", (batch, d_inner, L))):
        _expect(t, name, shape, io, dev)
    for t, name, shape in ((A, "A", (d_inner, N)), (D, "D", (d_inner,)),
                           (delta_bias, "delta_bias", (d_inner,)),
                           (conv_weight, "conv_weight", (d_inner, W)),
                           (conv_bias, "conv_bias", (d_inner,))):
        _expect(t, name, shape, torch.float32, dev)
    n_seqs, rows = 0, batch
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must hold n_seqs + 1 >= 2 offsets")
        n_seqs = rows = cu_seqlens.numel() - 1
        _expect(cu_seqlens, "cu_seqlens", (n_seqs + 1,), torch.int32, dev)
    _expect(initial_state, "initial_state", (rows, d_inner, N), torch.float32, dev)
    _expect(conv_state, "conv_state", (rows, d_inner, W - 1), torch.float32, dev)
    if y is None:
        y = torch.empty((batch, d_inner, L), dtype=io, device=dev)
    _expect(y, "y", (batch, d_inner, L), io, dev)
    if last_state is None and return_last_state:
        last_state = torch.empty((rows, d_inner, N), dtype=torch.float32, device=dev)
    _expect(last_state, "last_state", (rows, d_inner, N), torch.float32, dev)
    if u_out is None and return_u:
        u_out = torch.empty((batch, d_inner, L), dtype=io, device=dev)
    _expect(u_out, "u_out", (batch, d_inner, L), io, dev)
    desc = make_desc(batch, d_inner, N, L, code, chunk_size, _flags(zoh, independent_chunks))
    need = int(lib.ssm_scan_workspace_bytes(ctypes.byref(desc)))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    if profile_events is not None:
        desc.profile_begin, desc.profile_end = profile_events
    args = (_ptr(x), _ptr(conv_weight), _ptr(conv_bias), int(W), int(bool(conv_silu)),
            _ptr(conv_state), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), int(bool(softplus)), _ptr(initial_state), _ptr(cu_seqlens), n_seqs,
            _ptr(y), _ptr(last_state), _ptr(u_out), _stream(dev))
    keep = (x, conv_weight, conv_bias, conv_state, delta, A, B, C, D, z, delta_bias,
            initial_state, cu_seqlens, y, last_state, u_out, workspace)
    return _issue(prepare, lib.ssm_scan_fwd_conv, desc, args, keep, (y, last_state, u_out))


def ckpt_shape(batch, d_inner, seqlen):
    """Shape of the checkpoint tensor of ssm_scan_fwd(ckpt=...): the 16-float
    state entering every 8-token tile of every (batch, channel) row."""
    return (batch, d_inner, (seqlen + 7) // 8, 16)


def ssm_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True,
                 initial_state=None, dlast=None, chunk_size=0, workspace=None, cu_seqlens=None,
                 zoh=False, ckpt=None, prepare=False):
    """Gradients of sum(dy * y) + sum(dlast * last_state) of ssm_scan_fwd with
    respect to all its inputs (d_state up to 256; above 16 without
    cu_seqlens or ckpt; zoh: the zero-order-hold input term, as in
    ssm_scan_fwd).  Returns a dict of
    float32 tensors: du, ddelta (of the raw delta), dA, dB, dC, dD (None
    without D), dz (None without z), ddelta_bias, dh0 (None without
    initial_state).  cu_seqlens: packed sequences as in ssm_scan_fwd; the
    states (initial_state, dlast, dh0) then have one row per sequence.
    ckpt: the checkpoints of the matching ssm_scan_fwd(ckpt=...) call, which
    spare the backward its forward recompute.  prepare: as in ssm_scan_fwd."""
    torch = _torch()
    lib = load_library()
    batch, d_inner, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    dev, io = u.device, u.dtype
    code = _io_code(io)
    for t, name, shape in ((u, "u", (batch, d_inner, L)), (delta, "delta", (batch, d_inner, L)),
                           (B, "B", (batch, N, L)), (C, "C", (batch, N, L)),
                           (z, "z", (batch, d_inner, L)), (dy, "dy", (batch, d_inner, L))):
        _expect(t, name, shape, io, dev)
    n_seqs, rows = 0, batch
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must hold n_seqs + 1 >= 2 offsets")
        n_seqs = rows = cu_seqlens.numel() - 1
        _expect(cu_seqlens, "cu_seqlens", (n_seqs + 1,), torch.int32, dev)
    for t, name, shape in ((A, "A", (d_inner, N)), (D, "D", (d_inner,)),
                           (delta_bias, "delta_bias", (d_inner,)),
                           (initial_state, "initial_state", (rows, d_inner, N)),
                           (dlast, "dlast", (rows, d_inner, N)),
                           (ckpt, "ckpt", ckpt_shape(batch, d_inner, L))):
        _expect(t, name, shape, torch.float32, dev)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    out = {"du": f32(batch, d_inner, L), "ddelta": f32(batch, d_inner, L), "dA": f32(d_inner, N),
           "dB": f32(batch, N, L), "dC": f32(batch, N, L),
           "dD": f32(d_inner) if D is not None else None,
           "dz": f32(batch, d_inner, L) if z is not None else None,
           "ddelta_bias": f32(d_inner),
           "dh0": f32(rows, d_inner, N) if initial_state is not None else None}
    desc = make_desc(batch, d_inner, N, L, code, chunk_size, _flags(zoh, False))
    need = int(lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc)))
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        desc.workspace = workspace.data_ptr()
        desc.workspace_bytes = workspace.numel() * workspace.element_size()
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            int(bool(softplus)), _ptr(initial_state), _ptr(cu_seqlens), n_seqs, _ptr(ckpt),
            _ptr(dy), _ptr(dlast), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
            _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
            _ptr(out["ddelta_bias"]), _ptr(out["dh0"]), _stream(dev))
    keep = (u, delta, A, B, C, D, z, delta_bias, initial_state, cu_seqlens, ckpt, dy, dlast,
            workspace)
    return _issue(prepare, lib.ssm_scan_bwd_ex, desc, args, keep, out)


def ssm_state_update(state, u, delta, A, B, C, D=None, z=None, y=None, zoh=False,
                     prepare=False):
    """One single-token update of ``state`` (batch, d_inner, N) float32, in place.

    u, delta, z: (batch, d_inner); B, C: (batch, N); float32 or bfloat16.
    delta is the final step size; zoh selects the zero-order-hold input term.
    prepare: as in ssm_scan_fwd.  Returns y (batch, d_inner).
    """
    torch = _torch()
    lib = load_library()
    batch, d_inner, N = state.shape
    dev, io = u.device, u.dtype
    code = _io_code(io)
    _expect(state, "state", (batch, d_inner, N), torch.float32, dev)
    _expect(u, "u", (batch, d_inner), io, dev)
    _expect(delta, "delta", (batch, d_inner), io, dev)
    _expect(A, "A", (d_inner, N), torch.float32, dev)
    _expect(B, "B", (batch, N), io, dev)
    _expect(C, "C", (batch, N), io, dev)
    _expect(D, "D", (d_inner,), torch.float32, dev)
    _expect(z, "z", (batch, d_inner), io, dev)
    if y is None:
        y = torch.empty((batch, d_inner), dtype=io, device=dev)
    _expect(y, "y", (batch, d_inner), io, dev)
    desc = make_desc(batch, d_inner, N, 0, code, 0, SSM_FLAG_ZOH if zoh else 0)
    args = (_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(y), _stream(dev))
    return _issue(prepare, lib.ssm_state_update, desc, args, (state, u, delta, A, B, C, D, z, y),
                  y)
