"""GPU parity of start states and packed variable-length sequences
(ssm_scan_fwd_ex) against the fp64 oracle, through the C ABI.

Sequences are packed along the token axis of one batch row with a cu_seqlens
offset table; the state starts over at each sequence, from its initial state
or zero.  Cases: empty sequences, sequences shorter than a tile, boundaries
inside tiles and on chunk edges, many chunks (carry kernel) and few (fold),
d_state on both kernels (<= 16 and > 16), fp32 and bf16.
"""
import sys

import numpy as np
import pytest

import oracle
import selective_state_space_fwd_amd as ssm
import ssm_inputs
from ssm_testutil import TOL, decoded, floored_err, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ssm.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_packed(lens, d_inner, N, io, gate, seed, with_h0):
    total = int(sum(lens))
    inp = ssm_inputs.make_scan_inputs(1, d_inner, N, total, io_dtype=io, gate=gate, seed=seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rng = np.random.default_rng(seed + 7)
    h0 = rng.standard_normal((len(lens), d_inner, N)).astype(np.float32) if with_h0 else None
    return inp, cu, h0


def run_packed(inp, cu, h0, dev, chunk_size):
    import torch
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    cu_t = torch.from_numpy(cu).to(dev)
    h0_t = None if h0 is None else torch.from_numpy(h0).to(dev)
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], softplus=inp["softplus"], chunk_size=chunk_size,
                            initial_state=h0_t, cu_seqlens=cu_t)
    torch.cuda.synchronize()
    return y, h


def oracle_packed(inp, cu, h0):
    f = decoded(inp)
    return oracle.scan_varlen(f["u"], f["delta"], f["A"], f["B"], f["C"], cu, f["D"], f["z"],
                              f["delta_bias"], softplus=bool(f["softplus"]),
                              initial_state=None if h0 is None else h0.astype(np.float64))


LENS = {
    "mixed": [37, 0, 1, 200, 16, 0, 64, 5, 129, 0],
    "short": [3, 1, 4, 1, 5, 9, 2, 6],
    "one": [300],
    "trailing_empty": [100, 60, 0, 0],
    "leading_empty": [0, 0, 77, 50],
}


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 5, 64])
@pytest.mark.parametrize("lens", sorted(LENS))
@pytest.mark.parametrize("K,with_h0", [(0, True), (16, True), (64, False), (32, True)])
def test_packed_sequences(dev, io, N, lens, K, with_h0):
    inp, cu, h0 = make_packed(LENS[lens], 40, N, io, gate=True, seed=len(LENS[lens]) + N,
                              with_h0=with_h0)
    say(f"packed {lens} io={io} N={N} K={K} h0={with_h0}")
    y, h = run_packed(inp, cu, h0, dev, K)
    yr, hr = oracle_packed(inp, cu, h0)
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"  err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 40])
@pytest.mark.parametrize("K", [0, 64, 16])
def test_initial_state_batch_rows(dev, io, N, K):
    """No packing: every batch row starts from its own initial state."""
    import torch
    inp = ssm_inputs.make_scan_inputs(3, 50, N, 700, io_dtype=io, gate=True, seed=3)
    h0 = np.random.default_rng(5).standard_normal((3, 50, N)).astype(np.float32)
    t = {k: to_device(inp.get(k), dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                  "delta_bias")}
    y, h = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                            t["delta_bias"], chunk_size=K,
                            initial_state=torch.from_numpy(h0).to(dev))
    torch.cuda.synchronize()
    f = decoded(inp)
    yr, hr = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                             f["delta_bias"], softplus=True, initial_state=h0.astype(np.float64))
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"initial state io={io} N={N} K={K}: err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL[io] and eh <= TOL[io]


def test_split_sequence_continues_bit_exact(dev):
    """Exact-integer inputs (unit decay, integer B, C, u, dt = 1): scanning the
    first m tokens and then the rest from the returned state gives the same
    bits as scanning everything; and packing the two halves as two sequences
    with the second starting from that state gives the same bits again."""
    import torch
    d_inner, N, L, m = 24, 16, 260, 97
    rng = np.random.default_rng(11)
    u = rng.integers(-3, 4, size=(1, d_inner, L)).astype(np.float32)
    B = rng.integers(-2, 3, size=(1, N, L)).astype(np.float32)
    C = rng.integers(-2, 3, size=(1, N, L)).astype(np.float32)
    dt = np.ones((1, d_inner, L), np.float32)
    A = np.zeros((d_inner, N), np.float32)            # exp(dt * 0) = 1: h is a running sum
    g = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    y, h = ssm.ssm_scan_fwd(g(u), g(dt), g(A), g(B), g(C), softplus=False, chunk_size=16)
    y1, h1 = ssm.ssm_scan_fwd(g(u[..., :m]), g(dt[..., :m]), g(A), g(B[..., :m]),
                              g(C[..., :m]), softplus=False, chunk_size=32)
    y2, h2 = ssm.ssm_scan_fwd(g(u[..., m:]), g(dt[..., m:]), g(A), g(B[..., m:]),
                              g(C[..., m:]), softplus=False, chunk_size=48, initial_state=h1)
    assert torch.equal(torch.cat([y1, y2], dim=-1), y)
    assert torch.equal(h2, h)
    cu = torch.tensor([0, m, L], dtype=torch.int32, device=dev)
    h0 = torch.stack([torch.zeros_like(h1[0]), h1[0]])
    yp, hp = ssm.ssm_scan_fwd(g(u), g(dt), g(A), g(B), g(C), softplus=False, chunk_size=64,
                              initial_state=h0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(yp, y)
    assert torch.equal(hp[0], h1[0]) and torch.equal(hp[1], h[0])


def test_empty_total_copies_initial_state(dev):
    import torch
    h0 = torch.randn(3, 8, 16, device=dev)
    e = torch.empty((1, 8, 0), device=dev)
    B = torch.empty((1, 16, 0), device=dev)
    A = -torch.ones(8, 16, device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    y, h = ssm.ssm_scan_fwd(e, e, A, B, B, initial_state=h0, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert y.shape == (1, 8, 0) and torch.equal(h, h0)


def test_many_sequences_long_row(dev):
    """Hundreds of sequences of mixed length in a long row with the library's
    own chunking (few wavefronts: many chunks)."""
    rng = np.random.default_rng(21)
    lens = rng.integers(0, 300, size=120)
    inp, cu, h0 = make_packed(lens, 64, 16, "bf16", gate=True, seed=21, with_h0=True)
    say(f"many sequences: total {int(cu[-1])}, chunk {ssm.ssm_scan_chunk_size(1, 64, 16, int(cu[-1]), 1)}")
    y, h = run_packed(inp, cu, h0, dev, 0)
    yr, hr = oracle_packed(inp, cu, h0)
    ey, eh = floored_err(to_f64(y), yr), floored_err(to_f64(h), hr)
    say(f"  err y={ey:.3e} last_state={eh:.3e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]
