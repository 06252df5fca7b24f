"""Helpers for the parity tests: device upload, decoding and the error measure."""
import numpy as np

import ssm_inputs


def to_device(arr, device):
    """numpy float32 array or bf16 bit array (uint16) -> torch tensor on device."""
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
        return t.to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_f64(t):
    """torch tensor (float32 or bfloat16, any device) -> float64 numpy array."""
    import torch
    if t is None:
        return None
    return t.detach().to(torch.float64).cpu().numpy()


def to_f32(t):
    """torch tensor (float32 or bfloat16, any device) -> float32 numpy array
    (exact for both)."""
    import torch
    if t is None:
        return None
    return t.detach().to(torch.float32).cpu().numpy()


def decoded(inp):
    """Float64 view of a generated input dict, for the oracle."""
    out = {k: ssm_inputs.to_f64(inp.get(k)) for k in ("u", "delta", "B", "C", "z")}
    out.update(A=inp["A"], D=inp["D"], delta_bias=inp["delta_bias"], softplus=inp["softplus"])
    return out


def floored_err(got, ref, block=1 << 24):
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): relative error with a floor at
    the tensor's RMS, so outputs that cross zero do not divide by ~0.  Large
    tensors are taken in blocks of `block` elements (same result)."""
    got = np.asarray(got).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    ss = 0.0
    for i in range(0, ref.size, block):
        r = ref[i:i + block].astype(np.float64)
        ss += float(np.dot(r, r))
    rms = float(np.sqrt(ss / ref.size))
    floor = rms if rms > 0 else 1e-300
    worst = 0.0
    for i in range(0, ref.size, block):
        r = ref[i:i + block].astype(np.float64)
        g = got[i:i + block].astype(np.float64)
        worst = max(worst, float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor))))
    return worst


# Bar for floating-point parity: float32 I/O 1e-4, bfloat16 I/O (float32 state
# and accumulation, bf16-rounded output) 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}
