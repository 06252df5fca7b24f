"""Seeded synthetic inputs for the selective scan and its single-token update.

This module only draws and encodes inputs. It performs none of the scan's own
arithmetic (no discretisation, no recurrence, no softplus, no gate), so the
fp64 oracle and the HIP path can both take their inputs from it without
sharing any step of the method.

Recipe (one generator per call, numpy PCG64, fixed draw order):
  u      ~ N(0, 1)                       shape (batch, d_inner, L)
  delta  = 0.5 * N(0, 1)  (raw, pre-bias) shape (batch, d_inner, L)
  dt0    = exp(U(ln 1e-3, ln 1e-1))      shape (d_inner,)
  B, C   ~ N(0, 1)                       shape (batch, N, L)
  D      ~ N(0, 1)                       shape (d_inner,)
  z      ~ N(0, 1)                       shape (batch, d_inner, L)   (gated configs)
  A[d,n] = -exp(log(n + 1)) evaluated in float64 and stored as float32, which
           is exactly -(n + 1)
  delta_bias = inverse softplus of dt0, y + log(-expm1(-y)), in float64,
           stored as float32.  (The inverse of the step-size activation: it
           places the initial step sizes in [1e-3, 1e-1], the range the SSM
           engineering essay (discosf.com) recommends in its §1.2.)

Normals are drawn as float32 (numpy's float32 ziggurat), which keeps the
largest configurations (1.3e8 elements per tensor) cheap to generate.

bf16 inputs are produced from those float32 values by round-to-nearest-even
on the bit pattern and are carried as uint16 arrays; ``to_f64`` decodes any
stored input exactly.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"
IO_DTYPES = (F32, BF16)


# ---------------------------------------------------------------- encodings

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits.

    NaN inputs map to a quiet NaN.  Input encoding only.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def encode(x: np.ndarray, io_dtype: str) -> np.ndarray:
    """Store float values in the I/O dtype (float32 array or bf16 bits)."""
    if io_dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if io_dtype == BF16:
        return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(f"unknown io dtype {io_dtype!r}")


def to_f64(x: np.ndarray | None, io_dtype: str = F32) -> np.ndarray | None:
    """Decode a stored input (float32, or bf16 bits when io_dtype is bf16)."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- recipes

def a_matrix(d_inner: int, d_state: int) -> np.ndarray:
    """A = -exp(A_log) with A_log[d, n] = log(n + 1); float32, == -(n + 1)."""
    a_log = np.log(np.arange(1, d_state + 1, dtype=np.float64))
    a = -np.exp(a_log)
    return np.ascontiguousarray(np.broadcast_to(a, (d_inner, d_state)), dtype=np.float32)


def random_a_matrix(rng: np.random.Generator, d_inner: int, d_state: int) -> np.ndarray:
    """Unstructured negative A = -exp(N(0, 1)) (no pattern across n or d)."""
    return (-np.exp(rng.standard_normal((d_inner, d_state)))).astype(np.float32)


def inverse_softplus_bias(dt0: np.ndarray) -> np.ndarray:
    """delta_bias such that the step-size activation maps it back to dt0."""
    y = np.asarray(dt0, dtype=np.float64)
    return (y + np.log(-np.expm1(-y))).astype(np.float32)


def make_scan_inputs(batch: int, d_inner: int, d_state: int, seqlen: int,
                     io_dtype: str = F32, gate: bool = True, seed: int = 0,
                     random_a: bool = False) -> dict:
    """Inputs of one prefill scan, drawn with the recipe in the module doc.

    Returns a dict with keys u, delta, A, B, C, D, z (or None), delta_bias and
    softplus (=1).  u, delta, z, B, C are stored in ``io_dtype`` (float32, or
    uint16 bf16 bits); A, D, delta_bias are float32.
    """
    if io_dtype not in IO_DTYPES:
        raise ValueError(io_dtype)
    rng = np.random.default_rng(seed)
    f = np.float32
    u = rng.standard_normal((batch, d_inner, seqlen), dtype=f)
    delta = rng.standard_normal((batch, d_inner, seqlen), dtype=f)
    delta *= f(0.5)
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=d_inner))
    B = rng.standard_normal((batch, d_state, seqlen), dtype=f)
    C = rng.standard_normal((batch, d_state, seqlen), dtype=f)
    D = rng.standard_normal(d_inner, dtype=f)
    z = rng.standard_normal((batch, d_inner, seqlen), dtype=f) if gate else None
    A = random_a_matrix(rng, d_inner, d_state) if random_a else a_matrix(d_inner, d_state)
    return {
        "u": encode(u, io_dtype),
        "delta": encode(delta, io_dtype),
        "A": A,
        "B": encode(B, io_dtype),
        "C": encode(C, io_dtype),
        "D": D.astype(np.float32),
        "z": None if z is None else encode(z, io_dtype),
        "delta_bias": inverse_softplus_bias(dt0),
        "softplus": 1,
        "io_dtype": io_dtype,
        "shape": (batch, d_inner, d_state, seqlen),
    }


def make_update_inputs(batch: int, d_inner: int, d_state: int, io_dtype: str = F32,
                       gate: bool = True, seed: int = 0) -> dict:
    """Inputs of one single-token state update.

    The update takes the final step size, so delta is drawn directly as
    dt0 * exp(0.5 * N(0, 1)) with dt0 = exp(U(ln 1e-3, ln 1e-1)) per channel:
    a log-normal around dt0 with the same spread that the raw-plus-bias recipe
    produces for step sizes in [1e-3, 1e-1].  state ~ N(0, 1) float32.
    """
    rng = np.random.default_rng(seed)
    f = np.float32
    u = rng.standard_normal((batch, d_inner), dtype=f)
    g = rng.standard_normal((batch, d_inner), dtype=f)
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=d_inner))
    delta = (dt0[None, :] * np.exp(0.5 * g.astype(np.float64))).astype(f)
    B = rng.standard_normal((batch, d_state), dtype=f)
    C = rng.standard_normal((batch, d_state), dtype=f)
    D = rng.standard_normal(d_inner, dtype=f)
    z = rng.standard_normal((batch, d_inner), dtype=f) if gate else None
    state = rng.standard_normal((batch, d_inner, d_state), dtype=f)
    return {
        "state": state,
        "u": encode(u, io_dtype),
        "delta": encode(delta, io_dtype),
        "A": a_matrix(d_inner, d_state),
        "B": encode(B, io_dtype),
        "C": encode(C, io_dtype),
        "D": D.astype(np.float32),
        "z": None if z is None else encode(z, io_dtype),
        "io_dtype": io_dtype,
        "shape": (batch, d_inner, d_state),
    }


# Named workloads: the shapes of the pages' workloads (d_inner 1.5k-5k,
# N 16-256, L up to 64k).
def make_conv_params(d_inner: int, width: int = 4, seed: int = 0, decay_kernel: bool = True):
    """Weights (d_inner, width) and bias (d_inner) of the short causal
    convolution ahead of the scan, float32.

    decay_kernel: the initialisation the pages describe for it, taps that decay
    exponentially away from the current token, e^{-l}, e^{-2l}, ... (weight
    column width-1 multiplies the current token), with l ~ U(0.1, 1) per
    channel; otherwise N(0, 1/width) weights.  Bias ~ 0.1 N(0, 1).
    """
    rng = np.random.default_rng(seed)
    if decay_kernel:
        lam = rng.uniform(0.1, 1.0, size=(d_inner, 1))
        w = np.exp(-lam * np.arange(width, 0, -1)[None, :])
    else:
        w = rng.standard_normal((d_inner, width)) / np.sqrt(width)
    bias = 0.1 * rng.standard_normal(d_inner)
    return w.astype(np.float32), bias.astype(np.float32)


CONFIGS = {
    "c0_tiny_f32": dict(batch=1, d_inner=64, d_state=16, seqlen=256, io_dtype=F32, gate=False),
    "c1_mamba130m_f32": dict(batch=2, d_inner=1536, d_state=16, seqlen=2048, io_dtype=F32, gate=True),
    "c2_mamba2p8b_bf16": dict(batch=8, d_inner=5120, d_state=16, seqlen=2048, io_dtype=BF16, gate=True),
    "c3_long_bf16": dict(batch=1, d_inner=2048, d_state=16, seqlen=65536, io_dtype=BF16, gate=True),
    "c4_bigstate_f32": dict(batch=4, d_inner=2048, d_state=256, seqlen=4096, io_dtype=F32, gate=False),
}
DECODE_CONFIG = dict(batch=256, d_inner=5120, d_state=16, io_dtype=F32)
