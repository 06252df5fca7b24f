"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each check uses a route that differs from the oracle's sequential loop, so a
dropped term, a wrong sign, a shifted index or a transposed operand in the
oracle fails at least one of them:

* brute force: the unrolled sum over source tokens with the decay written as
  exp(A * sum of step sizes) -- closed form of the scan on the page "From
  FlashAttention to Mamba" (§三.2) and the decay-product form of the Mamba-2/SSD
  article (§2.2);
* a geometric series for constant step size, B and u (recurrence of the ufo.work
  article, §1.1);
* numpy.convolve for the time-invariant case (convolution / recurrence duality,
  SSM engineering essay §1.1);
* exact integer arithmetic (decay 1, unit step) against numpy.cumsum;
* the chunked route with transfer operators (ufo.work article §3.1);
* the single-token update repeated over the sequence (ufo.work article §4.1);
* special cases: zero step size, underflowing decay, zero / large gate,
  softplus against its inverse, and a hand-worked two-state example.
"""
import math

import numpy as np
import pytest

import oracle
import ssm_inputs

RNG = np.random.default_rng(1234)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def tiny_inputs(batch, d_inner, N, L, rng, random_a=True):
    u = rng.standard_normal((batch, d_inner, L))
    dt = np.exp(rng.uniform(np.log(1e-2), np.log(1.0), size=(batch, d_inner, L)))
    A = -np.exp(rng.standard_normal((d_inner, N))) if random_a else \
        -np.broadcast_to(np.arange(1, N + 1, dtype=np.float64), (d_inner, N)).copy()
    B = rng.standard_normal((batch, N, L))
    C = rng.standard_normal((batch, N, L))
    D = rng.standard_normal(d_inner)
    return u, dt, A, B, C, D


def brute_force(u, dt, A, B, C, D):
    """y_t = sum_{k<=t} sum_n C_t[n] exp(A_n sum_{s=k+1..t} dt_s) dt_k B_k[n] u_k + D u_t."""
    batch, d_inner, L = u.shape
    N = A.shape[1]
    y = np.zeros_like(u)
    last = np.zeros((batch, d_inner, N))
    for b in range(batch):
        for d in range(d_inner):
            cs = np.concatenate([[0.0], np.cumsum(dt[b, d])])  # cs[t+1] = sum_{s<=t} dt_s
            for t in range(L):
                acc = 0.0
                for k in range(t + 1):
                    decay = np.exp(A[d] * (cs[t + 1] - cs[k + 1]))      # (N,)
                    acc += np.sum(C[b, :, t] * decay * dt[b, d, k] * B[b, :, k] * u[b, d, k])
                y[b, d, t] = acc + D[d] * u[b, d, t]
            for n in range(N):
                last[b, d, n] = sum(np.exp(A[d, n] * (cs[L] - cs[k + 1])) * dt[b, d, k] *
                                    B[b, n, k] * u[b, d, k] for k in range(L))
    return y, last


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 3, 4, 17), (2, 5, 3, 40), (2, 2, 4, 64)])
def test_brute_force_unrolled_sum(shape):
    batch, d_inner, N, L = shape
    u, dt, A, B, C, D = tiny_inputs(batch, d_inner, N, L, RNG)
    y, last = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    yb, lb = brute_force(u, dt, A, B, C, D)
    assert rel(y, yb) < 1e-12
    assert rel(last, lb) < 1e-12


def test_brute_force_structured_a():
    # A[d, n] = -(n + 1), the workloads' initialisation.
    u, dt, A, B, C, D = tiny_inputs(2, 3, 4, 33, RNG, random_a=False)
    y, last = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    yb, lb = brute_force(u, dt, A, B, C, D)
    assert rel(y, yb) < 1e-12 and rel(last, lb) < 1e-12


def test_geometric_closed_form():
    L, N = 300, 4
    dt = 0.05
    A = np.array([[-0.5, -1.0, -3.0, 0.0]])
    Bn = np.array([0.7, -1.3, 2.0, 0.25])
    uval = 1.7
    Cn = np.array([1.0, 0.5, -2.0, 0.1])
    u = np.full((1, 1, L), uval)
    delta = np.full((1, 1, L), dt)
    B = np.broadcast_to(Bn[None, :, None], (1, N, L)).copy()
    C = np.broadcast_to(Cn[None, :, None], (1, N, L)).copy()
    D = np.array([0.3])
    y, last = oracle.scan_fwd(u, delta, A, B, C, D, softplus=False)
    a = np.exp(dt * A[0])
    b = dt * Bn * uval
    t = np.arange(L)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        h = np.where(a == 1.0, (t + 1) * b, b * (1 - a ** (t + 1)) / (1 - a))
    assert rel(last[0, 0], h[-1]) < 1e-12
    assert rel(y[0, 0], h @ Cn + 0.3 * uval) < 1e-12


def test_lti_equals_convolution():
    L, N = 200, 6
    rng = np.random.default_rng(7)
    dt = 0.1
    A = -np.exp(rng.standard_normal((1, N)))
    Bn, Cn = rng.standard_normal(N), rng.standard_normal(N)
    u = rng.standard_normal((1, 1, L))
    delta = np.full((1, 1, L), dt)
    B = np.broadcast_to(Bn[None, :, None], (1, N, L)).copy()
    C = np.broadcast_to(Cn[None, :, None], (1, N, L)).copy()
    D = np.array([-0.8])
    y, _ = oracle.scan_fwd(u, delta, A, B, C, D, softplus=False)
    a = np.exp(dt * A[0])
    kern = np.array([np.sum(Cn * a ** j * dt * Bn) for j in range(L)])
    ref = np.convolve(u[0, 0], kern)[:L] + D[0] * u[0, 0]
    assert rel(y[0, 0], ref) < 1e-12


def test_integer_cumsum_exact():
    # Decay 1 and unit step: h_t = sum_{k<=t} B_k u_k, every value an integer.
    rng = np.random.default_rng(3)
    batch, d_inner, N, L = 2, 3, 5, 500
    u = rng.integers(-3, 4, (batch, d_inner, L)).astype(np.float64)
    B = rng.integers(-3, 4, (batch, N, L)).astype(np.float64)
    C = rng.integers(-3, 4, (batch, N, L)).astype(np.float64)
    D = rng.integers(-3, 4, d_inner).astype(np.float64)
    A = np.zeros((d_inner, N))
    y, last = oracle.scan_fwd(u, np.ones_like(u), A, B, C, D, softplus=False)
    for b in range(batch):
        for d in range(d_inner):
            h = np.cumsum(B[b] * u[b, d][None, :], axis=1)      # (N, L)
            ref = np.sum(C[b] * h, axis=0) + D[d] * u[b, d]
            assert np.array_equal(y[b, d], ref)
            assert np.array_equal(last[b, d], h[:, -1])


@pytest.mark.parametrize("chunk", [1, 7, 64, 300, 301, 1000])
@pytest.mark.parametrize("tree", [True, False])
def test_chunked_equals_sequential(chunk, tree):
    inp = ssm_inputs.make_scan_inputs(2, 3, 16, 300, gate=True, seed=11, random_a=True)
    args = dict(u=inp["u"], delta=inp["delta"], A=inp["A"], B=inp["B"], C=inp["C"],
                D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"], softplus=True)
    y, last = oracle.scan_fwd(**args)
    yc, lc = oracle.scan_chunked(**args, chunk=chunk, tree=tree)
    assert rel(yc, y) < 1e-12
    assert rel(lc, last) < 1e-12


def test_chunked_with_initial_state():
    inp = ssm_inputs.make_scan_inputs(1, 4, 8, 129, gate=False, seed=5)
    h0 = np.random.default_rng(2).standard_normal((1, 4, 8))
    args = dict(u=inp["u"], delta=inp["delta"], A=inp["A"], B=inp["B"], C=inp["C"],
                D=inp["D"], delta_bias=inp["delta_bias"], initial_state=h0)
    y, last = oracle.scan_fwd(**args)
    yc, lc = oracle.scan_chunked(**args, chunk=16)
    assert rel(yc, y) < 1e-12 and rel(lc, last) < 1e-12


def test_initial_state_splits_sequence():
    # Running [0, L) equals running [0, m) then [m, L) from the state at m.
    inp = ssm_inputs.make_scan_inputs(2, 3, 16, 200, gate=True, seed=9)
    f = {k: ssm_inputs.to_f64(inp[k]) for k in ("u", "delta", "B", "C", "z")}
    args = dict(A=inp["A"], D=inp["D"], delta_bias=inp["delta_bias"])
    y, last = oracle.scan_fwd(f["u"], f["delta"], B=f["B"], C=f["C"], z=f["z"], **args)
    m = 77
    cut = lambda x, s: x[..., s]
    y1, h1 = oracle.scan_fwd(cut(f["u"], slice(0, m)), cut(f["delta"], slice(0, m)),
                             B=cut(f["B"], slice(0, m)), C=cut(f["C"], slice(0, m)),
                             z=cut(f["z"], slice(0, m)), **args)
    y2, h2 = oracle.scan_fwd(cut(f["u"], slice(m, None)), cut(f["delta"], slice(m, None)),
                             B=cut(f["B"], slice(m, None)), C=cut(f["C"], slice(m, None)),
                             z=cut(f["z"], slice(m, None)), initial_state=h1, **args)
    assert rel(np.concatenate([y1, y2], axis=2), y) < 1e-13
    assert rel(h2, last) < 1e-13


def test_update_repeated_equals_scan():
    inp = ssm_inputs.make_scan_inputs(2, 4, 16, 50, gate=True, seed=4)
    f = {k: ssm_inputs.to_f64(inp[k]) for k in ("u", "delta", "B", "C", "z")}
    y, last = oracle.scan_fwd(f["u"], f["delta"], inp["A"], f["B"], f["C"], inp["D"], f["z"],
                              inp["delta_bias"], softplus=True)
    # The update takes the final step size; form it here from the same raw
    # values with an independent softplus spelling, log(1 + e^x).
    dt = np.log1p(np.exp(f["delta"] + inp["delta_bias"].astype(np.float64)[None, :, None]))
    state = np.zeros((2, 4, 16))
    for t in range(50):
        state, yt = oracle.state_update(state, f["u"][..., t], dt[..., t], inp["A"],
                                        f["B"][..., t], f["C"][..., t], inp["D"], f["z"][..., t])
        assert rel(yt, y[..., t]) < 1e-12
    assert rel(state, last) < 1e-12


def test_update_against_closed_form():
    # One update: s' = exp(dt A) s + dt B u;  y = (C.s' + D u) silu(z).
    s0 = np.array([[[1.0, -2.0, 0.5]]])
    A = np.array([[-1.0, -0.5, -2.0]])
    dt, u = 0.2, 3.0
    Bv, Cv = np.array([[1.0, 2.0, -1.0]]), np.array([[0.5, -1.0, 4.0]])
    z = math.log(3.0)          # sigmoid(ln 3) = 3/4
    s, y = oracle.state_update(s0, [[u]], [[dt]], A, Bv, Cv, D=[0.25], z=[[z]])
    exp_s = np.exp(dt * A[0]) * s0[0, 0] + dt * Bv[0] * u
    assert rel(s[0, 0], exp_s) < 1e-15
    expected_y = (Cv[0] @ exp_s + 0.25 * u) * z * 0.75
    assert abs(y[0, 0] - expected_y) < 1e-14 * abs(expected_y)


def test_zero_step_gives_skip_only():
    inp = ssm_inputs.make_scan_inputs(1, 5, 16, 64, gate=False, seed=2)
    u = ssm_inputs.to_f64(inp["u"])
    y, last = oracle.scan_fwd(u, np.zeros_like(u), inp["A"], inp["B"], inp["C"], inp["D"],
                              softplus=False)
    assert np.array_equal(y, inp["D"].astype(np.float64)[None, :, None] * u)
    assert np.array_equal(last, np.zeros_like(last))


def test_underflowing_decay_closed_form():
    # dt*|A| >= 1000: exp underflows to 0, h_t = dt B_t u_t.
    rng = np.random.default_rng(5)
    batch, d_inner, N, L = 1, 3, 8, 40
    u = rng.standard_normal((batch, d_inner, L))
    dt = np.full_like(u, 50.0)
    A = -np.full((d_inner, N), 20.0)
    B = rng.standard_normal((batch, N, L))
    C = rng.standard_normal((batch, N, L))
    D = rng.standard_normal(d_inner)
    y, last = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    cb = np.sum(C[0] * B[0], axis=0)
    ref = 50.0 * u[0] * cb[None, :] + D[:, None] * u[0]
    assert rel(y[0], ref) < 1e-13
    assert rel(last[0], 50.0 * B[0][:, -1][None, :] * u[0][:, -1][:, None]) < 1e-13


def test_gate_identities():
    inp = ssm_inputs.make_scan_inputs(1, 4, 16, 80, gate=False, seed=6)
    f = {k: ssm_inputs.to_f64(inp[k]) for k in ("u", "delta", "B", "C")}
    base = dict(u=f["u"], delta=f["delta"], A=inp["A"], B=f["B"], C=f["C"], D=inp["D"],
                delta_bias=inp["delta_bias"])
    y, _ = oracle.scan_fwd(**base)
    y0, _ = oracle.scan_fwd(**base, z=np.zeros_like(f["u"]))
    assert np.array_equal(y0, np.zeros_like(y))
    ybig, _ = oracle.scan_fwd(**base, z=np.full_like(f["u"], 40.0))
    assert rel(ybig, 40.0 * y) < 1e-15       # silu(40) = 40 (1 - 4e-18)
    yln3, _ = oracle.scan_fwd(**base, z=np.full_like(f["u"], math.log(3.0)))
    assert rel(yln3, y * math.log(3.0) * 0.75) < 1e-15


def test_softplus_against_inverse():
    # softplus(inverse_softplus(dt0)) == dt0: the flag path with raw 0 and the
    # inverse bias must equal the flag-off path fed dt0 directly.
    rng = np.random.default_rng(8)
    d_inner, N, L = 6, 4, 30
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=d_inner))
    bias = ssm_inputs.inverse_softplus_bias(dt0).astype(np.float64)
    u = rng.standard_normal((1, d_inner, L))
    B = rng.standard_normal((1, N, L))
    C = rng.standard_normal((1, N, L))
    A = -np.exp(rng.standard_normal((d_inner, N)))
    y_on, _ = oracle.scan_fwd(u, np.zeros_like(u), A, B, C, delta_bias=bias, softplus=True)
    # bias was rounded to float32; map it back with an independent spelling
    # of softplus, log(1 + e^x), valid for these moderate arguments.
    dt_exact = np.log1p(np.exp(bias))
    y_off, _ = oracle.scan_fwd(u, np.broadcast_to(dt_exact[None, :, None], u.shape).copy(), A,
                               B, C, softplus=False)
    assert rel(y_on, y_off) < 1e-13
    assert np.allclose(dt_exact, dt0, rtol=1e-6)   # float32 bias keeps ~7 digits


def test_softplus_extremes():
    # Very large raw step: softplus(x) = x; very negative: softplus(x) = e^x.
    u = np.ones((1, 1, 2))
    A = np.array([[0.0]])
    B = np.ones((1, 1, 2))
    C = np.ones((1, 1, 2))
    y, _ = oracle.scan_fwd(u, np.array([[[800.0, -800.0]]]), A, B, C, softplus=True)
    assert y[0, 0, 0] == 800.0
    assert y[0, 0, 1] == 800.0 + math.exp(-800.0)


def test_hand_worked_example():
    # Two states, three tokens, unit step, decays 1/2 and 1/4 (A = -ln 2, -ln 4),
    # no softplus, D = 1/2.  By hand:
    #   state 0: B = (1, 1, 1), C = (1, 2, 1):  h = 2, 1 + 4 = 5, 2.5 - 2 = 0.5
    #   state 1: B = (2, 0, 1), C = (1, 1, 1):  h = 4, 1 + 0 = 1, 0.25 - 2 = -1.75
    #   u = (2, 4, -2)
    #   y0 = 1*2 + 1*4 + 0.5*2 = 7;  y1 = 2*5 + 1*1 + 0.5*4 = 13;
    #   y2 = 1*0.5 + 1*(-1.75) + 0.5*(-2) = -2.25
    u = np.array([[[2.0, 4.0, -2.0]]])
    A = np.array([[-math.log(2.0), -math.log(4.0)]])
    B = np.array([[[1.0, 1.0, 1.0], [2.0, 0.0, 1.0]]])
    C = np.array([[[1.0, 2.0, 1.0], [1.0, 1.0, 1.0]]])
    y, last = oracle.scan_fwd(u, np.ones_like(u), A, B, C, D=[0.5], softplus=False)
    assert np.allclose(y[0, 0], [7.0, 13.0, -2.25], rtol=0, atol=1e-14)
    assert np.allclose(last[0, 0], [0.5, -1.75], rtol=0, atol=1e-14)


def test_batch_permutation_and_layout():
    inp = ssm_inputs.make_scan_inputs(3, 4, 16, 40, gate=True, seed=12)
    f = {k: ssm_inputs.to_f64(inp[k]) for k in ("u", "delta", "B", "C", "z")}
    common = dict(A=inp["A"], D=inp["D"], delta_bias=inp["delta_bias"])
    y, last = oracle.scan_fwd(f["u"], f["delta"], B=f["B"], C=f["C"], z=f["z"], **common)
    p = [2, 0, 1]
    yp, lp = oracle.scan_fwd(f["u"][p], f["delta"][p], B=f["B"][p], C=f["C"][p], z=f["z"][p],
                             **common)
    assert np.array_equal(yp, y[p]) and np.array_equal(lp, last[p])


def test_scan_rows_matches_full():
    inp = ssm_inputs.make_scan_inputs(2, 6, 16, 64, gate=True, seed=13)
    f = {k: ssm_inputs.to_f64(inp.get(k)) for k in ("u", "delta", "B", "C", "z")}
    f.update(A=inp["A"], D=inp["D"], delta_bias=inp["delta_bias"], softplus=1)
    y, last = oracle.scan_fwd(f["u"], f["delta"], f["A"], f["B"], f["C"], f["D"], f["z"],
                              f["delta_bias"])
    rows = [(1, 5), (0, 0), (1, 2)]
    ys, hs = oracle.scan_rows(f, rows)
    for i, (b, d) in enumerate(rows):
        assert np.array_equal(ys[i], y[b, d]) and np.array_equal(hs[i], last[b, d])


def test_threads_do_not_change_result():
    inp = ssm_inputs.make_scan_inputs(2, 7, 16, 100, gate=True, seed=14)
    args = dict(u=inp["u"], delta=inp["delta"], A=inp["A"], B=inp["B"], C=inp["C"],
                D=inp["D"], z=inp["z"], delta_bias=inp["delta_bias"])
    y1, l1 = oracle.scan_fwd(**args, threads=1)
    y8, l8 = oracle.scan_fwd(**args, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(l1, l8)


def test_bad_arguments_raise():
    with pytest.raises(ValueError):
        oracle.scan_fwd(np.zeros((1, 2, 3)), np.zeros((1, 2, 4)), np.zeros((2, 1)),
                        np.zeros((1, 1, 3)), np.zeros((1, 1, 3)))
    with pytest.raises(RuntimeError):
        oracle.scan_chunked(np.zeros((1, 1, 3)), np.zeros((1, 1, 3)), np.zeros((1, 1)),
                            np.zeros((1, 1, 3)), np.zeros((1, 1, 3)), chunk=0)


def test_golden_integer_fixture():
    import importlib.util
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(here, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    u, dt, A, B, C, D = mg.inputs()
    stored = {}
    with open(os.path.join(here, "integer_scan.txt")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            key, *vals = line.split()
            stored[key] = np.array([float(v) for v in vals])
    y, last = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    for d in range(2):
        assert np.array_equal(y[0, d], stored[f"y{d}"])
        assert np.array_equal(last[0, d], stored[f"h{d}"])
        # independent route: running sums
        h = np.cumsum(B[0] * u[0, d][None, :], axis=1)
        assert np.array_equal(np.sum(C[0] * h, axis=0) + D[d] * u[0, d], stored[f"y{d}"])


def brute_force_h0(u, dt, A, B, C, D, h0):
    """brute_force plus the start-state term: each output gains
    sum_n C_t[n] exp(A_n sum_{s<=t} dt_s) h0[n]; the final state gains
    exp(A_n sum_s dt_s) h0[n]."""
    y, last = brute_force(u, dt, A, B, C, D)
    batch, d_inner, L = u.shape
    for b in range(batch):
        for d in range(d_inner):
            cs = np.cumsum(dt[b, d])                       # cs[t] = sum_{s<=t} dt_s
            for t in range(L):
                y[b, d, t] += np.sum(C[b, :, t] * np.exp(A[d] * cs[t]) * h0[b, d])
            last[b, d] += np.exp(A[d] * (cs[-1] if L else 0.0)) * h0[b, d]
    return y, last


def test_varlen_brute_force_with_initial_state():
    """Packed sequences (ufo.work article §4.2): every sequence restarts from its
    own initial state at its first token; an empty sequence keeps it."""
    d_inner, N = 3, 4
    lens = [5, 0, 1, 9, 0, 4]
    total = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    u, dt, A, B, C, D = tiny_inputs(1, d_inner, N, total, RNG)
    h0 = RNG.standard_normal((len(lens), d_inner, N))
    y, last = oracle.scan_varlen(u, dt, A, B, C, cu, D, softplus=False, initial_state=h0)
    for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        if a == b:
            assert np.array_equal(last[s], h0[s])
            continue
        yb, lb = brute_force_h0(u[:, :, a:b], dt[:, :, a:b], A, B[:, :, a:b], C[:, :, a:b], D,
                                h0[s:s + 1])
        assert rel(y[:, :, a:b], yb) < 1e-12
        assert rel(last[s], lb[0]) < 1e-12


def test_varlen_zero_start_equals_batch_rows():
    """Equal-length sequences packed along time, all from zero, equal the same
    sequences scanned as separate batch rows."""
    d_inner, N, n, Ls = 4, 3, 3, 7
    u, dt, A, B, C, D = tiny_inputs(n, d_inner, N, Ls, RNG)
    pack = lambda x: np.concatenate(list(x), axis=-1)[None]
    cu = np.arange(n + 1) * Ls
    y, last = oracle.scan_varlen(pack(u), pack(dt), A, pack(B), pack(C), cu, D, softplus=False)
    yb, lb = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    assert np.array_equal(y[0], np.concatenate(list(yb), axis=-1))
    assert np.array_equal(last, lb)


def test_varlen_rejects_bad_offsets():
    u = np.zeros((1, 2, 5))
    A = -np.ones((2, 2))
    B = np.zeros((1, 2, 5))
    for cu in ([0, 3], [1, 5], [0, 4, 3, 5], [0]):
        with pytest.raises(ValueError):
            oracle.scan_varlen(u, u, A, B, B, cu)


# ------------------------------------------------------------ causal conv1d

def conv_direct(x, w, bias, start_state=None):
    """Double loop: out_t = bias + sum_k w[k] x_{t-(W-1)+k}, x_{<0} from start_state."""
    L = x.size
    W = w.size
    head = np.zeros(W - 1) if start_state is None else start_state
    out = np.zeros(L)
    for t in range(L):
        acc = bias
        for k in range(W):
            src = t - (W - 1) + k
            acc += w[k] * (x[src] if src >= 0 else head[W - 1 + src])
        out[t] = acc
    return out


def test_conv_impulse_response():
    """A unit impulse at t0 leaves the taps, newest first: out_{t0+j} = w[W-1-j]."""
    W, L, t0 = 4, 12, 3
    w = RNG.standard_normal((2, W))
    x = np.zeros((1, 2, L))
    x[0, :, t0] = 1.0
    out = oracle.causal_conv1d(x, w, None, silu=False)
    for d in range(2):
        expect = np.zeros(L)
        expect[t0:t0 + W] = w[d][::-1]
        assert np.array_equal(out[0, d], expect)


def test_conv_exponential_kernel_geometric_sums():
    """The pages' initial kernel K = [e^-l, e^-2l, ..., e^-kl] (nearest token
    first) on a constant input of ones gives the partial geometric sums
    sum_{j=1..min(t+1,W)} e^{-j l} plus the bias, then silu."""
    W, L = 4, 9
    lam = np.array([0.3, 1.1])
    w = np.stack([np.exp(-lam[d] * np.arange(W, 0, -1)) for d in range(2)])  # w[W-1] = e^-l
    bias = np.array([0.25, -0.5])
    out = oracle.causal_conv1d(np.ones((1, 2, L)), w, bias, silu=True)
    for d in range(2):
        for t in range(L):
            m = min(t + 1, W)
            r = math.exp(-lam[d])
            pre = bias[d] + r * (1 - r ** m) / (1 - r)
            assert abs(out[0, d, t] - pre / (1 + math.exp(-pre))) < 1e-14


def test_conv_matches_double_loop_with_state_and_packing():
    W, d_inner = 3, 3
    lens = [6, 0, 1, 10]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = RNG.standard_normal((1, d_inner, cu[-1]))
    w = RNG.standard_normal((d_inner, W))
    bias = RNG.standard_normal(d_inner)
    cs = RNG.standard_normal((len(lens), d_inner, W - 1))
    out = oracle.causal_conv1d(x, w, bias, silu=False, cu_seqlens=cu, conv_state=cs)
    for s in range(len(lens)):
        for d in range(d_inner):
            ref = conv_direct(x[0, d, cu[s]:cu[s + 1]], w[d], bias[d], cs[s, d])
            assert rel(out[0, d, cu[s]:cu[s + 1]], ref) < 1e-14 if ref.size else True
    # without a start state the batch rows start from zeros
    xb = RNG.standard_normal((2, d_inner, 7))
    outb = oracle.causal_conv1d(xb, w, bias, silu=False)
    for b in range(2):
        for d in range(d_inner):
            assert rel(outb[b, d], conv_direct(xb[b, d], w[d], bias[d])) < 1e-14


# ------------------------------------------------------------ zero-order hold

def test_zoh_matches_continuous_solution():
    """Zero-order hold (SSM engineering essay, §1.2) is exact for an input held
    constant: L steps of size dt reach the continuous solution at T = L dt,
    h(T) = e^{A T} h0 + (e^{A T} - 1) / A * B u, whatever the step count."""
    N, dt, u0 = 4, 0.037, 1.3
    A = -np.array([[0.5, 1.0, 2.0, 7.0]])
    Bn = np.array([0.3, -1.1, 0.7, 2.0])
    Cn = np.array([1.0, 0.5, -0.25, 0.125])
    h0 = np.array([[[0.2, -0.4, 1.5, 0.9]]])
    for L in (1, 2, 7, 50):
        u = np.full((1, 1, L), u0)
        dts = np.full((1, 1, L), dt)
        B = np.broadcast_to(Bn[None, :, None], (1, N, L)).copy()
        C = np.broadcast_to(Cn[None, :, None], (1, N, L)).copy()
        y, last = oracle.scan_fwd(u, dts, A, B, C, softplus=False, initial_state=h0, zoh=True)
        T = L * dt
        for t in range(L):
            Tt = (t + 1) * dt
            ht = np.exp(A[0] * Tt) * h0[0, 0] + np.expm1(A[0] * Tt) / A[0] * Bn * u0
            assert abs(y[0, 0, t] - np.sum(Cn * ht)) < 1e-12
        hT = np.exp(A[0] * T) * h0[0, 0] + np.expm1(A[0] * T) / A[0] * Bn * u0
        assert rel(last[0, 0], hT) < 1e-12


def test_zoh_reduces_to_euler_at_zero_decay():
    """At A = 0 the hold rule's input factor (e^{dt A} - 1) / A has the limit
    dt, the Euler factor, so both rules give the same scan."""
    u, dt, _, B, C, D = tiny_inputs(1, 3, 4, 20, RNG)
    A = np.zeros((3, 4))
    y0, h0 = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    y1, h1 = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False, zoh=True)
    assert np.array_equal(y0, y1) and np.array_equal(h0, h1)


def test_zoh_chunked_and_decode_agree():
    u, dt, A, B, C, D = tiny_inputs(2, 3, 5, 37, RNG)
    y, h = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False, zoh=True)
    yc, hc = oracle.scan_chunked(u, dt, A, B, C, D, softplus=False, chunk=8, zoh=True)
    assert rel(yc, y) < 1e-13 and rel(hc, h) < 1e-13
    s = np.zeros((2, 3, 5))
    for t in range(37):
        s, yt = oracle.state_update(s, u[:, :, t], dt[:, :, t], A, B[:, :, t], C[:, :, t], D,
                                    zoh=True)
        assert rel(yt, y[:, :, t]) < 1e-12
    assert rel(s, h) < 1e-12


# ------------------------------------------------------------ backward

def _loss(u, dt, A, B, C, D, z, bias, h0, dy, dlast, zoh=False):
    y, last = oracle.scan_fwd(u, dt, A, B, C, D, z, bias, softplus=True, initial_state=h0,
                              zoh=zoh)
    return float(np.sum(dy * y) + np.sum(dlast * last))


@pytest.mark.parametrize("gate,zoh", [(False, False), (True, False), (True, True),
                                      (False, True)])
def test_backward_against_finite_differences(gate, zoh):
    """Every gradient of sum(dy*y) + sum(dlast*last_state) from the hand-written
    reverse walk equals the central difference of the forward oracle's loss
    (step 1e-6, fp64) on a tiny problem: a dropped term or a wrong index in
    any one gradient fails.  With the zero-order-hold input term too, where
    the steps dt*A fall on both sides of 1 in magnitude (the two branches of
    the factor's A-derivative)."""
    rng = np.random.default_rng(7 + gate + 2 * zoh)
    b, d, N, L = 2, 3, 4, 9
    u = rng.standard_normal((b, d, L))
    raw = 0.5 * rng.standard_normal((b, d, L))
    A = -np.exp(rng.standard_normal((d, N)))
    B = rng.standard_normal((b, N, L))
    C = rng.standard_normal((b, N, L))
    D = rng.standard_normal(d)
    z = rng.standard_normal((b, d, L)) if gate else None
    bias = rng.uniform(-3, -1, d)
    h0 = rng.standard_normal((b, d, N))
    dy = rng.standard_normal((b, d, L))
    dlast = rng.standard_normal((b, d, N))
    if zoh:
        A[0, 0] = -8.0          # dt*A beyond -1 for this state; the others within
        A[1, 1] = 0.0           # the A = 0 limit: the factor is dt
    g = oracle.scan_bwd(u, raw, A, B, C, dy, D, z, bias, softplus=True, initial_state=h0,
                        dlast=dlast, zoh=zoh)
    args = dict(u=u, dt=raw, A=A, B=B, C=C, D=D, z=z, bias=bias, h0=h0)
    names = {"u": "du", "dt": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "bias": "ddelta_bias", "h0": "dh0"}
    if gate:
        names["z"] = "dz"
    eps = 1e-6
    for key, gname in names.items():
        arr = args[key]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in args.items()}
            minus = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in args.items()}
            plus[key][idx] += eps
            minus[key][idx] -= eps
            num[idx] = (_loss(**plus, dy=dy, dlast=dlast, zoh=zoh) -
                        _loss(**minus, dy=dy, dlast=dlast, zoh=zoh)) / (2 * eps)
        assert rel(g[gname], num) < 1e-7, (gname, rel(g[gname], num))


def test_backward_threads_do_not_change_result():
    rng = np.random.default_rng(3)
    u, dt, A, B, C, D = tiny_inputs(2, 5, 3, 30, rng)
    dy = rng.standard_normal(u.shape)
    g1 = oracle.scan_bwd(u, dt, A, B, C, dy, D, softplus=False, threads=1)
    g4 = oracle.scan_bwd(u, dt, A, B, C, dy, D, softplus=False, threads=4)
    for k in ("du", "ddelta", "dA", "dD", "ddelta_bias", "dh0"):
        assert np.array_equal(g1[k], g4[k]), k
    for k in ("dB", "dC"):
        assert rel(g1[k], g4[k]) < 1e-14


def _loss_varlen(u, dt, A, B, C, D, z, bias, h0, cu, dy, dlast):
    y, last = oracle.scan_varlen(u, dt, A, B, C, cu, D, z, bias, softplus=True, initial_state=h0)
    return float(np.sum(dy * y) + np.sum(dlast * last))


def test_backward_packed_sequences_against_finite_differences():
    """Packed sequences (one empty, one of a single token): every gradient of
    sum(dy*y) + sum(dlast*last_state) from ``scan_bwd_varlen`` equals the
    central difference of the packed forward oracle's loss.  This pins where
    the state gradient starts (each sequence's dlast at its last token), where
    it stops (dh0 at its first token, dlast for the empty one) and that no
    gradient crosses a boundary."""
    rng = np.random.default_rng(11)
    lens = [3, 0, 1, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    d, N, L, n = 2, 3, int(cu[-1]), len(lens)
    u = rng.standard_normal((1, d, L))
    raw = 0.5 * rng.standard_normal((1, d, L))
    A = -np.exp(rng.standard_normal((d, N)))
    B = rng.standard_normal((1, N, L))
    C = rng.standard_normal((1, N, L))
    D = rng.standard_normal(d)
    z = rng.standard_normal((1, d, L))
    bias = rng.uniform(-3, -1, d)
    h0 = rng.standard_normal((n, d, N))
    dy = rng.standard_normal((1, d, L))
    dlast = rng.standard_normal((n, d, N))
    g = oracle.scan_bwd_varlen(u, raw, A, B, C, cu, dy, D, z, bias, softplus=True,
                               initial_state=h0, dlast=dlast)
    args = dict(u=u, dt=raw, A=A, B=B, C=C, D=D, z=z, bias=bias, h0=h0)
    names = {"u": "du", "dt": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "z": "dz", "bias": "ddelta_bias", "h0": "dh0"}
    eps = 1e-6
    for key, gname in names.items():
        arr = args[key]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = {k: v.copy() for k, v in args.items()}
            minus = {k: v.copy() for k, v in args.items()}
            plus[key][idx] += eps
            minus[key][idx] -= eps
            num[idx] = (_loss_varlen(**plus, cu=cu, dy=dy, dlast=dlast) -
                        _loss_varlen(**minus, cu=cu, dy=dy, dlast=dlast)) / (2 * eps)
        assert rel(g[gname], num) < 1e-7, (gname, rel(g[gname], num))
    # the empty sequence: its initial state goes straight to its last state
    assert np.array_equal(g["dh0"][1], dlast[1])
