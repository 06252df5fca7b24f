"""fp64 CPU oracle of the selective scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it, and it never calls the product path.

The arithmetic lives in ``ssm_oracle.c`` (plain C, double precision, libm,
no fast-math), described there with its sources.  This module only builds
that file with gcc, loads it with ctypes and marshals numpy arrays.

Pins (each checked by a ``-m "not gpu"`` test in tests/test_oracle_pins.py):
  * brute-force unrolled sum  y_t = sum_k C_t (prod_{s=k+1..t} dA_s) dt_k B_k u_k + D u_t
    on tiny inputs (page "From FlashAttention to Mamba", §三.2 closed form of
    the scan; the decay-product form of the Mamba-2/SSD article, §2.2);
  * geometric closed form for constant delta, B, u (recurrence of the ufo.work
    article, §1.1);
  * time-invariant special case == numpy.convolve with kernel
    K_j = sum_n C_n a_n^j dt B_n (convolution/recurrence duality, SSM
    engineering essay §1.1);
  * chunked route (transfer operators, fold and tree combine) == sequential
    loop (ufo.work article, §3.1);
  * single-token update applied L times == the scan (ufo.work article, §4.1);
  * delta = 0 gives y = D u; a decay so strong that exp underflows gives the
    closed form y_t = dt u_t (C_t . B_t) + D u_t; z = 0 zeroes y; softplus of
    the inverse-softplus bias returns the drawn step size;
  * a hand-worked example with exact rational values;
  * packed variable-length sequences (``scan_varlen``): the brute-force sum
    with an initial-state term y_t += sum_n C_t[n] (prod_{s<=t} dA_s[n]) h0[n]
    per sequence, and a packing of sequences that all start from zero equals
    scanning each as its own batch row;
  * the backward pass (``scan_bwd``): every gradient against central finite
    differences of the forward oracle's loss on tiny inputs;
  * the causal convolution (``causal_conv1d``): impulse response = the
    reversed kernel, a constant input through the exponentially decaying
    kernel of "From FlashAttention to Mamba" §三.3 = its geometric partial
    sums, and a direct double loop on random data.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SRC = _HERE / "ssm_oracle.c"
LIB = _HERE / "libssm_oracle.so"

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (no fast-math)."""
    if not force and LIB.exists() and LIB.stat().st_mtime >= SRC.stat().st_mtime:
        return LIB
    tmp = LIB.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           str(SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(str(LIB))
    i64, dp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.oracle_scan_fwd.argtypes = [i64, i64, i64, i64] + [dp] * 8 + [c_int, dp, dp, dp, c_int,
                                                                        c_int]
    lib.oracle_scan_fwd.restype = c_int
    lib.oracle_scan_chunked.argtypes = ([i64, i64, i64, i64] + [dp] * 8 +
                                        [c_int, dp, dp, dp, c_int, i64, c_int, c_int])
    lib.oracle_scan_chunked.restype = c_int
    lib.oracle_state_update.argtypes = [i64, i64, i64] + [dp] * 9 + [c_int]
    lib.oracle_scan_bwd.argtypes = ([i64, i64, i64, i64] + [dp] * 8 + [c_int] + [dp] * 3 +
                                    [dp] * 9 + [c_int, c_int])
    lib.oracle_scan_bwd.restype = c_int
    lib.oracle_state_update.restype = c_int
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x, shape=None):
    if x is None:
        return None
    a = np.ascontiguousarray(x, dtype=np.float64)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _scan_args(u, delta, A, B, C, D, z, delta_bias, initial_state):
    u = _f64(u)
    if u.ndim != 3:
        raise ValueError("u must be (batch, d_inner, L)")
    batch, d_inner, L = u.shape
    A = _f64(A)
    N = A.shape[1]
    return (batch, d_inner, N, L, u, _f64(delta, u.shape), _f64(A, (d_inner, N)),
            _f64(B, (batch, N, L)), _f64(C, (batch, N, L)), _f64(D, (d_inner,)),
            _f64(z, u.shape), _f64(delta_bias, (d_inner,)),
            _f64(initial_state, (batch, d_inner, N)))


def scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
             initial_state=None, threads: int | None = None, zoh: bool = False):
    """Sequential fp64 scan.  Returns (y, last_state), both float64.
    zoh: zero-order-hold input term (exp(dt A) - 1) / A * B u instead of dt B u."""
    lib = _load()
    (batch, d_inner, N, L, u, delta, A, B, C, D, z, bias, h0) = _scan_args(
        u, delta, A, B, C, D, z, delta_bias, initial_state)
    y = np.zeros((batch, d_inner, L))
    last = np.zeros((batch, d_inner, N))
    rc = lib.oracle_scan_fwd(batch, d_inner, N, L, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                             _ptr(C), _ptr(D), _ptr(z), _ptr(bias), int(bool(softplus)),
                             _ptr(h0), _ptr(y), _ptr(last), int(bool(zoh)),
                             threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_scan_fwd failed ({rc})")
    return y, last


def scan_chunked(u, delta, A, B, C, D=None, z=None, delta_bias=None, softplus=True,
                 initial_state=None, chunk: int = 256, tree: bool = True,
                 threads: int | None = None, zoh: bool = False):
    """Chunked fp64 route (transfer operators + combine).  Returns (y, last_state)."""
    lib = _load()
    (batch, d_inner, N, L, u, delta, A, B, C, D, z, bias, h0) = _scan_args(
        u, delta, A, B, C, D, z, delta_bias, initial_state)
    y = np.zeros((batch, d_inner, L))
    last = np.zeros((batch, d_inner, N))
    rc = lib.oracle_scan_chunked(batch, d_inner, N, L, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(z), _ptr(bias), int(bool(softplus)),
                                 _ptr(h0), _ptr(y), _ptr(last), int(bool(zoh)), int(chunk),
                                 int(bool(tree)), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_scan_chunked failed ({rc})")
    return y, last


def scan_varlen(u, delta, A, B, C, cu_seqlens, D=None, z=None, delta_bias=None, softplus=True,
                initial_state=None, threads: int | None = None, zoh: bool = False):
    """Packed variable-length sequences, fp64.  Returns (y, last_state).

    u, delta, z: (1, d_inner, total); B, C: (1, N, total); cu_seqlens:
    n_seqs + 1 nondecreasing offsets with cu_seqlens[0] = 0 and
    cu_seqlens[-1] = total.  Sequence s is the token range
    [cu_seqlens[s], cu_seqlens[s+1]); the state is reset at its first token
    to initial_state[s] (zeros when None), so each sequence is scanned on its
    own, exactly as ``scan_fwd`` scans one batch row -- the packed-sequence
    batching of the ufo.work article, §4.2 (cu_seqlens marks the boundaries,
    the state is reset there), with the start state of §4.1.  last_state is
    (n_seqs, d_inner, N); an empty sequence keeps its initial state.
    """
    u = _f64(u)
    if u.ndim != 3 or u.shape[0] != 1:
        raise ValueError("packed sequences need u of shape (1, d_inner, total)")
    _, d_inner, total = u.shape
    N = np.asarray(A).shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = cu.size - 1
    if n < 1 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to the total length")
    h0 = None if initial_state is None else _f64(initial_state, (n, d_inner, N))
    y = np.zeros((1, d_inner, total))
    last = np.zeros((n, d_inner, N))
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        hs = None if h0 is None else h0[s:s + 1]
        if a == b:
            last[s] = 0.0 if hs is None else hs[0]
            continue
        part = lambda x: None if x is None else np.asarray(x)[:, :, a:b]
        ys, ls = scan_fwd(part(u), part(delta), A, part(B), part(C), D, part(z), delta_bias,
                          softplus=softplus, initial_state=hs, threads=threads, zoh=zoh)
        y[:, :, a:b] = ys
        last[s] = ls[0]
    return y, last


def causal_conv1d(x, weight, bias=None, silu=True, cu_seqlens=None, conv_state=None):
    """Depthwise causal 1-D convolution along the token axis, fp64.

    x: (batch, d_inner, L); weight: (d_inner, W); bias: (d_inner,) or None.
    out[b, d, t] = bias[d] + sum_k weight[d, k] x[b, d, t - (W - 1) + k], then
    silu(out) = out / (1 + exp(-out)) when ``silu`` -- the short convolution
    that precedes the scan in the Mamba layer ("From FlashAttention to Mamba",
    §三.3), fused with it per §四.3.  Tokens before a sequence's first token
    are conv_state[s, d, W - 1 - j] for x_{start - 1 - j} (zeros when
    conv_state is None).  Sequences are the batch rows, or, with cu_seqlens
    (batch 1), the packed ranges [cu[s], cu[s+1]).  Each channel of each
    sequence is one numpy.convolve call.
    """
    x = _f64(x)
    batch, d_inner, L = x.shape
    w = _f64(weight)
    W = w.shape[1]
    bvec = np.zeros(d_inner) if bias is None else _f64(bias, (d_inner,))
    if cu_seqlens is None:
        bounds = [(b, 0, L) for b in range(batch)]
    else:
        if batch != 1:
            raise ValueError("packed sequences need batch == 1")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        bounds = [(0, int(cu[s]), int(cu[s + 1])) for s in range(cu.size - 1)]
    rows = len(bounds)
    cs = None if conv_state is None else _f64(conv_state, (rows, d_inner, W - 1))
    out = np.zeros_like(x)
    for s, (b, a, e) in enumerate(bounds):
        if a == e:
            continue
        for d in range(d_inner):
            head = np.zeros(W - 1) if cs is None else cs[s, d]
            seq = np.concatenate([head, x[b, d, a:e]])
            out[b, d, a:e] = np.convolve(seq, w[d][::-1], mode="valid") + bvec[d]
    if silu:
        out = out / (1.0 + np.exp(-out))
    return out


def scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, softplus=True,
             initial_state=None, dlast=None, threads: int | None = None, zoh: bool = False):
    """Gradients of sum(dy * y) + sum(dlast * last_state) for the scan, fp64
    (the reverse walk is written out in ssm_oracle.c; zoh: the zero-order-hold
    input term).  Returns a dict with du, ddelta (w.r.t. the raw step before
    bias and softplus), dz (None without a gate), dA, dB, dC, dD, ddelta_bias,
    dh0 (w.r.t. initial_state)."""
    lib = _load()
    (batch, d_inner, N, L, u, delta, A, B, C, D, z, bias, h0) = _scan_args(
        u, delta, A, B, C, D, z, delta_bias, initial_state)
    dy = _f64(dy, (batch, d_inner, L))
    dlast = _f64(dlast, (batch, d_inner, N))
    out = {k: np.zeros((batch, d_inner, L)) for k in ("du", "ddelta")}
    out["dz"] = np.zeros((batch, d_inner, L)) if z is not None else None
    out["dA"] = np.zeros((d_inner, N))
    out["dB"] = np.zeros((batch, N, L))
    out["dC"] = np.zeros((batch, N, L))
    out["dD"] = np.zeros(d_inner)
    out["ddelta_bias"] = np.zeros(d_inner)
    out["dh0"] = np.zeros((batch, d_inner, N))
    rc = lib.oracle_scan_bwd(batch, d_inner, N, L, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                             _ptr(C), _ptr(D), _ptr(z), _ptr(bias), int(bool(softplus)),
                             _ptr(h0), _ptr(dy), _ptr(dlast), _ptr(out["du"]),
                             _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]),
                             _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                             _ptr(out["ddelta_bias"]), _ptr(out["dh0"]),
                             threads or default_threads(), int(bool(zoh)))
    if rc != 0:
        raise RuntimeError(f"oracle_scan_bwd failed ({rc})")
    return out


def scan_bwd_varlen(u, delta, A, B, C, cu_seqlens, dy, D=None, z=None, delta_bias=None,
                    softplus=True, initial_state=None, dlast=None, threads: int | None = None,
                    zoh: bool = False):
    """Backward pass of ``scan_varlen`` (packed sequences), fp64: the gradients
    of sum(dy * y) + sum(dlast * last_state).  Each sequence is its own scan
    (``scan_varlen``), so its gradients are those of ``scan_bwd`` on its token
    range with its own initial state and last-state gradient; the token
    gradients (du, ddelta, dz, dB, dC) of the ranges are placed side by side
    and the parameter gradients (dA, dD, ddelta_bias) summed over the
    sequences in order.  An empty sequence passes its initial state straight
    to its last state, so its dh0 is its dlast.  States are (n_seqs, d_inner,
    N)."""
    u = _f64(u)
    if u.ndim != 3 or u.shape[0] != 1:
        raise ValueError("packed sequences need u of shape (1, d_inner, total)")
    _, d_inner, total = u.shape
    N = np.asarray(A).shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = cu.size - 1
    if n < 1 or cu[0] != 0 or cu[-1] != total or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to the total length")
    h0 = None if initial_state is None else _f64(initial_state, (n, d_inner, N))
    dl = None if dlast is None else _f64(dlast, (n, d_inner, N))
    out = {k: np.zeros((1, d_inner, total)) for k in ("du", "ddelta")}
    out["dz"] = np.zeros((1, d_inner, total)) if z is not None else None
    out["dA"] = np.zeros((d_inner, N))
    out["dB"] = np.zeros((1, N, total))
    out["dC"] = np.zeros((1, N, total))
    out["dD"] = np.zeros(d_inner)
    out["ddelta_bias"] = np.zeros(d_inner)
    out["dh0"] = np.zeros((n, d_inner, N))
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            if dl is not None:
                out["dh0"][s] = dl[s]
            continue
        part = lambda x: None if x is None else np.asarray(x)[:, :, a:b]
        g = scan_bwd(part(u), part(delta), A, part(B), part(C), part(dy), D, part(z), delta_bias,
                     softplus=softplus, initial_state=None if h0 is None else h0[s:s + 1],
                     dlast=None if dl is None else dl[s:s + 1], threads=threads, zoh=zoh)
        for k in ("du", "ddelta", "dB", "dC"):
            out[k][:, :, a:b] = g[k]
        if z is not None:
            out["dz"][:, :, a:b] = g["dz"]
        for k in ("dA", "dD", "ddelta_bias"):
            out[k] += g[k]
        out["dh0"][s] = g["dh0"][0]
    return out


def state_update(state, u, delta, A, B, C, D=None, z=None, zoh: bool = False):
    """One fp64 single-token update.  Returns (new_state, y); inputs untouched."""
    lib = _load()
    s = np.array(state, dtype=np.float64, copy=True, order="C")
    batch, d_inner, N = s.shape
    u = _f64(u, (batch, d_inner))
    delta = _f64(delta, (batch, d_inner))
    A = _f64(A, (d_inner, N))
    B = _f64(B, (batch, N))
    C = _f64(C, (batch, N))
    D = _f64(D, (d_inner,))
    z = _f64(z, (batch, d_inner))
    y = np.zeros((batch, d_inner))
    rc = lib.oracle_state_update(batch, d_inner, N, _ptr(s), _ptr(u), _ptr(delta), _ptr(A),
                                 _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), int(bool(zoh)))
    if rc != 0:
        raise RuntimeError(f"oracle_state_update failed ({rc})")
    return s, y


def scan_rows(inputs_f64: dict, rows, threads: int | None = None):
    """Oracle on a subset of (b, d) rows of one workload.

    ``inputs_f64`` holds decoded float64 arrays (keys u, delta, A, B, C, D, z,
    delta_bias, softplus, optional initial_state).  Returns (y_rows, state_rows) with
    shapes (len(rows), L) and (len(rows), N), in the order of ``rows``.
    """
    u = inputs_f64["u"]
    L = u.shape[2]
    N = inputs_f64["A"].shape[1]
    ys = np.zeros((len(rows), L))
    hs = np.zeros((len(rows), N))
    by_batch: dict[int, list[int]] = {}
    for i, (b, d) in enumerate(rows):
        by_batch.setdefault(int(b), []).append(i)
    for b, idx in by_batch.items():
        ds = np.array([rows[i][1] for i in idx])
        sel = lambda key: None if inputs_f64.get(key) is None else inputs_f64[key][b:b + 1, ds]
        vec = lambda key: None if inputs_f64.get(key) is None else inputs_f64[key][ds]
        h0 = inputs_f64.get("initial_state")
        y, h = scan_fwd(sel("u"), sel("delta"), inputs_f64["A"][ds], inputs_f64["B"][b:b + 1],
                        inputs_f64["C"][b:b + 1], vec("D"), sel("z"), vec("delta_bias"),
                        softplus=bool(inputs_f64.get("softplus", 1)),
                        initial_state=None if h0 is None else h0[b:b + 1, ds],
                        threads=threads)
        ys[idx] = y[0]
        hs[idx] = h[0]
    return ys, hs
