"""Benchmark of the MI355X selective scan (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
the fused prefill scan of the workload (softplus step size, discretisation,
recurrence, chunk carry, output with skip term and gate, last_state), then
one single-token state update of every channel continuing from that
last_state.  Inputs are resident in HBM before timing starts; the step cycles
through several independent input sets whose total size exceeds the 256 MB
last-level cache, so every step reads from HBM.

Prints one JSON line.  ``value`` is channel-tokens per second over the timed
steps (batch * d_inner * (L + 1) per step).  ``roofline`` covers the dominant
kernel, the pass that writes y, timed with HIP events recorded around it on
its stream inside the timed region.  ``cpu_baseline`` is the fp64 oracle on
the host cores (rank 0, one GPU only) on a bounded sample of the workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ssm_inputs  # noqa: E402

METRIC = "selective-scan channel-tokens/sec"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
# MI355X fp32 vector peak, published: 157.3 TFLOP/s = 256 CUs x 2.4 GHz x 128
# FMA lanes per clock.  ALU work below is counted in FMA-equivalent issue
# slots (2 FLOP each).  A transcendental (exp2, log2, rcp) occupies the VALU
# about twice as long as an FMA -- measured on MI355X with independent chains
# of wave64 instructions: 9.3 SIMD-cycles per v_exp_f32 against 4.5 per
# v_fma_f32 -- and so counts as 2 slots.
VALU_PEAK_TFLOPS = 157.3
# That published figure counts packed FP32 (v_pk_fma_f32: two FMAs per lane per
# clock).  These kernels are compiled with packed FP32 disabled, so the vector
# ceiling they can reach is one FMA per lane per clock:
# 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz = 78.6 TFLOP/s.
VALU_PEAK_NONPACKED_TFLOPS = 78.6
DEFAULT_CONFIG = "c3_long_bf16"
# Chunk lengths a workload names (the long-sequence layer: K in {256, 512,
# 1024} with the state carried from chunk to chunk), and the one the headline
# line runs at; the others, and the library's own choice, are timed beside it.
CONFIG_CHUNKS = {"c3_long_bf16": (256, 512, 1024)}
HEADLINE_CHUNK = {"c3_long_bf16": 256}
CACHE_BYTES = 256 << 20        # MI355X last-level (Infinity) cache

# Minimal instruction mix of the method, in FMA-equivalent slots.
TRANS_SLOTS = 2
SLOTS_PER_UPDATE = 4 + TRANS_SLOTS      # dt*A', w*B, state FMA, output FMA; one exp2
SLOTS_PER_CHTOK = {                     # per (batch, channel, token), outside the N loop
    "softplus": 7 + 2 * TRANS_SLOTS,    # 7 VALU + exp2 + log2
    "common": 4,                        # bias add, w = dt*u, D*u, (y + Du)
    "gate": 3 + 2 * TRANS_SLOTS,        # 3 VALU + exp2 + rcp
}
# The library's plan (mirrored here only to name the timed kernel): with
# d_state <= 16 and 2..32 chunks of at least this many tokens the whole
# chunked scan is one launch.
FUSED_MIN_CHUNK = 1024


# Backward pass, minimal work of the method (states are not stored by the
# forward pass, so one recompute of the recurrence is part of it):
# per (channel-token, state): recompute dt*A', exp2, w*B, state FMA (5);
# reverse walk dh = G + dO*C, dO*h and w*dh with their channel sums (5),
# dh.B, dh*h_prev, the dA and ddelta terms (2 + 2), G = dh*a (1): 17 in all.
# Per channel-token: softplus (11), its derivative (sigmoid: 1 + exp2 + rcp),
# silu and its derivative (exp2 + rcp + 4), w, dO, the output o and the five
# token gradients and two sums (9): 35.
BWD_SLOTS_PER_UPDATE = 5 + 12
BWD_SLOTS_PER_CHTOK = 35


def algorithmic_bytes(batch, d_inner, N, L, io, gate, last_state=True):
    """Bytes the scan must move once: u, delta, (z) read and y written per
    channel-token; B and C read once per (batch, token); A, D, bias per
    channel; last_state written per channel."""
    e = 2 if io == "bf16" else 4
    per_chtok = (3 + (1 if gate else 0)) * e
    return (batch * d_inner * L * per_chtok + 2 * batch * N * L * e +
            d_inner * (N + 2) * 4 + (batch * d_inner * N * 4 if last_state else 0))


def algorithmic_slots(batch, d_inner, N, L, gate):
    """FMA-equivalent VALU issue slots the scan needs at minimum."""
    chtok = batch * d_inner * L
    per = SLOTS_PER_CHTOK["softplus"] + SLOTS_PER_CHTOK["common"]
    if gate:
        per += SLOTS_PER_CHTOK["gate"]
    return chtok * (N * SLOTS_PER_UPDATE + per)


def versions():
    import torch
    out = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            out["rocm"] = f.read().strip()
    except OSError:
        out["rocm"] = None
    return out


class HipEvents:
    """Raw hipEvent_t handles via the HIP runtime (the library records them on
    its own stream around the pass that writes y)."""

    def __init__(self):
        import torch  # noqa: F401  (loads the HIP runtime torch uses)
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def upload(arr, dev):
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def cpu_baseline(cfg, budget_s=12.0):
    """The fp64 oracle on the host cores, on a bounded sample of the workload
    (whole channels, every token), scaled to channel-tokens/s."""
    import oracle
    batch, d_inner, N, L = cfg["batch"], cfg["d_inner"], cfg["d_state"], cfg["seqlen"]
    threads = oracle.default_threads()
    # sample: the first rows of batch row 0, all L tokens; grow until the
    # budget is used
    inp = ssm_inputs.make_scan_inputs(1, min(d_inner, 4096), N, L, io_dtype=cfg["io_dtype"],
                                      gate=cfg["gate"], seed=0)
    f = {k: ssm_inputs.to_f64(inp.get(k)) for k in ("u", "delta", "B", "C", "z")}
    total_rows = f["u"].shape[1]
    rows = min(threads, total_rows)
    done_chtok, spent, passes = 0, 0.0, 0
    while spent < budget_s:
        sl = slice(0, rows)
        t0 = time.perf_counter()
        oracle.scan_fwd(f["u"][:, sl], f["delta"][:, sl], inp["A"][sl], f["B"], f["C"],
                        inp["D"][sl], None if f["z"] is None else f["z"][:, sl],
                        inp["delta_bias"][sl], softplus=True, threads=threads)
        dt = time.perf_counter() - t0
        done_chtok += rows * L
        spent += dt
        passes += 1
        if rows < total_rows and dt < budget_s / 8:
            rows = min(total_rows, rows * 2)
    # the same oracle on one core: whole channels, one after another, for about
    # a quarter of the budget
    one_done, one_spent, c = 0, 0.0, 0
    while one_spent < budget_s / 4 and c < total_rows:
        sl = slice(c, c + 1)
        t0 = time.perf_counter()
        oracle.scan_fwd(f["u"][:, sl], f["delta"][:, sl], inp["A"][sl], f["B"], f["C"],
                        inp["D"][sl], None if f["z"] is None else f["z"][:, sl],
                        inp["delta_bias"][sl], softplus=True, threads=1)
        one_spent += time.perf_counter() - t0
        one_done += L
        c += 1
    return {"value": done_chtok / spent, "unit": "channel-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} passes over up to {rows} whole channels of batch row 0 "
                      f"({done_chtok // L} channel rows x {L} tokens, N={N}, "
                      f"{cfg['io_dtype']} inputs), {spent:.1f} s of oracle time",
            "one_core": {"value": one_done / one_spent, "unit": "channel-tokens/s", "cores": 1,
                         "sample": f"{c} whole channels of batch row 0, {one_spent:.1f} s"}}


def bench_decode(args, torch, ssm, dev):
    """The decode step alone: every channel of 256 sequences advances its
    persistent state by one token.  An HBM-bound stream: the state is read and
    written once; per channel also u, dt, z, y, and B, C per sequence."""
    cfg = dict(ssm_inputs.DECODE_CONFIG)
    batch, d_inner, N = cfg["batch"], cfg["d_inner"], cfg["d_state"]
    sets = []
    per_set = batch * d_inner * N * 8
    n_sets = max(2, min(8, -(-3 * CACHE_BYTES // per_set)))
    for s in range(n_sets):
        inp = ssm_inputs.make_update_inputs(batch, d_inner, N, io_dtype="f32", gate=True,
                                            seed=2000 + s)
        t = {k: upload(inp[k], dev) for k in ("u", "delta", "B", "C", "z", "A", "D", "state")}
        t["y"] = torch.empty_like(t["u"])
        sets.append(t)
    torch.cuda.synchronize()

    # The step is ~30 us of GPU work, close to the binding's own Python cost, so
    # the arguments are marshalled once and the C ABI is called directly.
    lib = ssm.load_library()
    desc = ssm.make_desc(batch, d_inner, N, 0, 0)
    stream = torch.cuda.current_stream(dev).cuda_stream
    argv = [[t[k].data_ptr() for k in ("state", "u", "delta", "A", "B", "C", "D", "z", "y")]
            for t in sets]

    def step(i):
        st = lib.ssm_state_update(ctypes.byref(desc), *argv[i % n_sets], stream)
        if st != 0:
            raise RuntimeError(ssm.ssm_status_string(st))

    settled = settle_clocks(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    nbytes = (batch * d_inner * (N * 8 + 4 * 4) + 2 * batch * N * 4 + d_inner * (N + 1) * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9

    # The practical ceiling of such a stream on this GPU: torch's own
    # device-to-device copy of as many bytes (half read, half written), over
    # as many buffers in rotation as the step has input sets.
    half = nbytes // 2 // 4
    src = [torch.empty(half, dtype=torch.float32, device=dev).fill_(1.0) for _ in range(n_sets)]
    dst = [torch.empty_like(x) for x in src]
    for i in range(n_sets):
        dst[i].copy_(src[i])
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        dst[i % n_sets].copy_(src[i % n_sets])
    end.record()
    torch.cuda.synchronize()
    copy_ms = start.elapsed_time(end) / args.steps
    copy_gbs = 2 * half * 4 / (copy_ms * 1e-3) / 1e9
    del src, dst
    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f).get("decode")
        if tj and tj.get("bytes_per_launch") and not tj.get("stale"):
            traffic = tj["bytes_per_launch"]
    except (OSError, ValueError):
        traffic = None
    return {
        "metric": "single-token state update, channels/sec",
        "value": batch * d_inner / (ms * 1e-3), "unit": "channels/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "steps": settled}, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode: {batch} sequences x {d_inner} channels x N={N}, "
                               "fp32 state, gate", "batch": batch, "d_inner": d_inner,
                   "d_state": N, "input_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": nbytes,
                     "kernel_ms": ms, "copy_gbs": copy_gbs, "frac_of_copy": gbs / copy_gbs},
        "versions": versions(),
    }


def bench_backward(args, torch, ssm, dev):
    """The backward pass alone on the workload: every gradient of
    sum(dy * y) + sum(dlast * last_state).  Algorithmic bytes: the forward
    inputs read once, dy read, and du, ddelta, dz (fp32) and dB, dC written.
    With --ckpt the backward reads the checkpoints that the forward pass of
    the same inputs wrote (one forward with checkpoints, outside the timed
    region, as a training step's forward would have); their 16 floats per
    8 tokens per channel count as read bytes.  The algorithmic work is the
    same either way: one recompute of the recurrence (from the checkpoints,
    the tiles' recompute is that one; without them the forward sweep that
    writes them comes on top and is not counted)."""
    cfg = dict(ssm_inputs.CONFIGS[args.config])
    batch, d_inner, N, L = cfg["batch"], cfg["d_inner"], cfg["d_state"], cfg["seqlen"]
    io, gate = cfg["io_dtype"], cfg["gate"]
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=gate, seed=0)
    t = {k: upload(inp[k], dev) for k in ("u", "delta", "B", "C", "z", "A", "D", "delta_bias")}
    rng = np.random.default_rng(1)
    dy = upload(ssm_inputs.encode(rng.standard_normal((batch, d_inner, L)).astype(np.float32),
                                  io), dev)
    dlast = upload(rng.standard_normal((batch, d_inner, N)).astype(np.float32), dev)
    code = 1 if io == "bf16" else 0
    desc = ssm.make_desc(batch, d_inner, N, L, code, args.chunk)
    lib = ssm.load_library()
    ws = torch.empty(max(1, int(lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc)))),
                     dtype=torch.uint8, device=dev)
    ck = None
    if args.ckpt:
        ck = torch.empty(ssm.ckpt_shape(batch, d_inner, L), dtype=torch.float32, device=dev)
        ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                         t["delta_bias"], softplus=True, ckpt=ck)

    def step():
        ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                         t["delta_bias"], softplus=True, dlast=dlast, chunk_size=args.chunk,
                         workspace=ws, ckpt=ck)

    settled = settle_clocks(torch, lambda i: step(), args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    e = 2 if io == "bf16" else 4
    chtok = batch * d_inner * L
    nbytes = (chtok * ((4 if gate else 3) * e + (3 if gate else 2) * 4) +
              2 * batch * N * L * (e + 4) + d_inner * (N + 2) * 4)
    if ck is not None:
        nbytes += ck.numel() * 4
    slots = chtok * (N * BWD_SLOTS_PER_UPDATE + BWD_SLOTS_PER_CHTOK)
    tflops = 2.0 * slots / (ms * 1e-3) / 1e12
    return {
        "metric": "selective-scan backward channel-tokens/sec", "value": chtok / (ms * 1e-3),
        "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "steps": settled},
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.config}: backward of the scan, batch={batch} "
                               f"d_inner={d_inner} N={N} L={L} {io} I/O"
                               f"{' + gate' if gate else ''}"
                               f"{', forward checkpoints given' if ck is not None else ''}",
                   "batch": batch, "d_inner": d_inner, "d_state": N, "seqlen": L,
                   "io_dtype": io, "gate": gate, "checkpoints": ck is not None,
                   "plan": ssm.scan_bwd_plan(batch, d_inner, N, L, 1 if io == "bf16" else 0,
                                             args.chunk or 0, with_ckpt=ck is not None)},
        "roofline": {"bound": "alu", "achieved": tflops, "peak": VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / VALU_PEAK_TFLOPS, "traffic": None,
                     "peak_nonpacked": VALU_PEAK_NONPACKED_TFLOPS,
                     "frac_nonpacked": tflops / VALU_PEAK_NONPACKED_TFLOPS,
                     "kernel": "the whole backward call (forward chunk aggregates, reverse "
                               "chunk aggregates, bwd_kernel, bwd_reduce_kernel)",
                     "kernel_ms": ms, "algorithmic_slots": slots,
                     "hbm_achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
                     "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "algorithmic_bytes": nbytes},
        "hbm_achieved_gbs": nbytes / (ms * 1e-3) / 1e9, "algorithmic_bytes": nbytes,
        "versions": versions(),
    }


def bench_train(args, torch, ssm, dev):
    """One training step of the scan on the workload: the forward pass that
    keeps the state entering every 8-token tile (ssm_scan_fwd_ckpt), then the
    backward pass that reads them (every gradient).  Algorithmic work: the
    forward's slots plus the backward's (its one recompute of the recurrence
    included)."""
    cfg = dict(ssm_inputs.CONFIGS[args.config])
    batch, d_inner, N, L = cfg["batch"], cfg["d_inner"], cfg["d_state"], cfg["seqlen"]
    io, gate = cfg["io_dtype"], cfg["gate"]
    inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=gate, seed=0)
    t = {k: upload(inp[k], dev) for k in ("u", "delta", "B", "C", "z", "A", "D", "delta_bias")}
    rng = np.random.default_rng(1)
    dy = upload(ssm_inputs.encode(rng.standard_normal((batch, d_inner, L)).astype(np.float32),
                                  io), dev)
    dlast = upload(rng.standard_normal((batch, d_inner, N)).astype(np.float32), dev)
    ck = torch.empty(ssm.ckpt_shape(batch, d_inner, L), dtype=torch.float32, device=dev)
    args_f = (t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"])
    fwd = ssm.ssm_scan_fwd(*args_f, softplus=True, chunk_size=args.chunk, ckpt=ck, prepare=True)
    bwd = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["z"],
                           t["delta_bias"], softplus=True, dlast=dlast, chunk_size=args.chunk,
                           ckpt=ck, prepare=True)

    def step():
        fwd()
        bwd()

    settled = settle_clocks(torch, lambda i: step(), args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    chtok = batch * d_inner * L
    slots = (algorithmic_slots(batch, d_inner, N, L, gate) +
             chtok * (N * BWD_SLOTS_PER_UPDATE + BWD_SLOTS_PER_CHTOK))
    tflops = 2.0 * slots / (ms * 1e-3) / 1e12
    return {
        "metric": "selective-scan training step (forward keeping checkpoints + backward) "
                  "channel-tokens/sec",
        "value": chtok / (ms * 1e-3), "unit": "channel-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "steps": settled}, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: forward with checkpoints + backward, "
                               f"batch={batch} d_inner={d_inner} N={N} L={L} {io} I/O"
                               f"{' + gate' if gate else ''}",
                   "batch": batch, "d_inner": d_inner, "d_state": N, "seqlen": L,
                   "io_dtype": io, "gate": gate},
        "roofline": {"bound": "alu", "achieved": tflops, "peak": VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / VALU_PEAK_TFLOPS, "traffic": None,
                     "peak_nonpacked": VALU_PEAK_NONPACKED_TFLOPS,
                     "frac_nonpacked": tflops / VALU_PEAK_NONPACKED_TFLOPS,
                     "kernel": "the whole step (forward passes, backward passes)",
                     "kernel_ms": ms, "algorithmic_slots": slots},
        "versions": versions(),
    }


# Extra minimal work of the forward variants:
# ZOH, per (channel-token, state): x = dt A (1), e^x - 1 (1), rcp(x) (2 slots),
# the quotient (1) and its product with w B (1);
# the fused convolution, per channel-token: 4 taps (4 FMA) and silu (7).
ZOH_SLOTS_PER_UPDATE = 4 + TRANS_SLOTS
CONV_SLOTS_PER_CHTOK = 4 + SLOTS_PER_CHTOK["gate"]
# Packed sequences: the workload's batch x seqlen tokens of every channel,
# cut into sequences of this length mix (fractions of the total), each with a
# start state.
VARLEN_MIX = (0.25, 0.125, 0.375, 0.0625, 0.1875)


def bench_variant(args, torch, ssm, dev):
    """The forward scan alone with one of the method's variants on the
    workload: the zero-order-hold input term (zoh), the causal convolution
    fused in front (conv, width 4, silu), or the tokens packed as sequences of
    mixed lengths with start states (varlen).  `achieved` is the variant's
    algorithmic slots over the pass that writes y, timed by events its own
    dispatch records."""
    cfg = dict(ssm_inputs.CONFIGS[args.config])
    batch, d_inner, N, L = cfg["batch"], cfg["d_inner"], cfg["d_state"], cfg["seqlen"]
    io, gate = cfg["io_dtype"], cfg["gate"]
    v = args.variant
    cu = None
    if v == "varlen":
        total = batch * L
        lens = [int(round(f * total)) for f in VARLEN_MIX]
        lens[-1] = total - sum(lens[:-1])
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        batch, L = 1, total
    rows = len(cu) - 1 if cu is not None else batch
    n_sets = max(2, min(8, -(-3 * CACHE_BYTES // algorithmic_bytes(batch, d_inner, N, L, io,
                                                                  gate))))
    sets = []
    for s_ in range(n_sets):
        inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=gate, seed=s_)
        t = {k: upload(inp[k], dev) for k in ("u", "delta", "B", "C", "z", "A", "D",
                                                "delta_bias")}
        t["y"] = torch.empty_like(t["u"])
        t["last"] = torch.empty((rows, d_inner, N), dtype=torch.float32, device=dev)
        if v == "varlen":
            h0 = np.random.default_rng(50 + s_).standard_normal((rows, d_inner, N))
            t["h0"] = upload(h0.astype(np.float32), dev)
        sets.append(t)
        del inp
    cu_t = torch.from_numpy(cu).to(dev) if cu is not None else None
    if v == "conv":
        w, cb = ssm_inputs.make_conv_params(d_inner, 4, seed=7)
        w_t, cb_t = upload(w, dev), upload(cb, dev)
    calls = []
    for t in sets:
        common = dict(softplus=True, chunk_size=args.chunk, y=t["y"], last_state=t["last"],
                      prepare=True)
        if v == "conv":
            calls.append(ssm.ssm_scan_fwd_conv(t["u"], w_t, cb_t, t["delta"], t["A"], t["B"],
                                               t["C"], t["D"], t["z"], t["delta_bias"],
                                               **common))
        else:
            calls.append(ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"],
                                          t["z"], t["delta_bias"], zoh=(v == "zoh"),
                                          initial_state=t.get("h0"), cu_seqlens=cu_t,
                                          **common))
    torch.cuda.synchronize()
    hip = HipEvents()
    ev = hip.create(2 * (args.steps + args.warmup))
    settled = settle_clocks(torch, lambda i: calls[i % n_sets](None), args.settle_ms)
    for i in range(args.warmup):
        calls[i % n_sets]((ev[2 * i], ev[2 * i + 1]))
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    base = 2 * args.warmup
    start.record()
    for i in range(args.steps):
        calls[i % n_sets]((ev[base + 2 * i], ev[base + 2 * i + 1]))
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    kavg = float(np.mean([hip.elapsed_ms(ev[base + 2 * i], ev[base + 2 * i + 1])
                          for i in range(args.steps)]))
    hip.destroy(ev)
    chtok = batch * d_inner * L
    slots = algorithmic_slots(batch, d_inner, N, L, gate)
    if v == "zoh":
        slots += chtok * N * ZOH_SLOTS_PER_UPDATE
    if v == "conv":
        slots += chtok * CONV_SLOTS_PER_CHTOK
    tflops = 2.0 * slots / (kavg * 1e-3) / 1e12
    K = ssm.ssm_scan_chunk_size(batch, d_inner, N, L, 1 if io == "bf16" else 0, args.chunk)
    what = {"zoh": "zero-order-hold input term", "conv": "causal convolution (width 4, silu) "
            "fused in front", "varlen": f"{rows} packed sequences of lengths "
            f"{[int(x) for x in np.diff(cu)] if cu is not None else ''} with start states"}[v]
    return {
        "metric": f"selective-scan channel-tokens/sec, {v}", "value": chtok / (ms * 1e-3),
        "unit": "channel-tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "steps": settled},
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{args.config}: selective scan, {what}, batch={batch} "
                               f"d_inner={d_inner} N={N} L={L} {io} I/O"
                               f"{' + silu gate' if gate else ''}",
                   "batch": batch, "d_inner": d_inner, "d_state": N, "seqlen": L,
                   "io_dtype": io, "gate": gate, "variant": v, "chunk": K,
                   "input_sets": n_sets},
        "roofline": {"bound": "alu", "achieved": tflops, "peak": VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / VALU_PEAK_TFLOPS, "traffic": None,
                     "peak_nonpacked": VALU_PEAK_NONPACKED_TFLOPS,
                     "frac_nonpacked": tflops / VALU_PEAK_NONPACKED_TFLOPS,
                     "kernel": "the whole call: every dispatch of the scan (first to last, "
                               "mean of the timed steps)", "kernel_ms": kavg,
                     "algorithmic_slots": slots},
        "versions": versions(),
    }


def kernel_sources_sha():
    """Digest of the sources of the forward scan and decode kernels (every file
    of csrc/ but the backward's, which no forward kernel is built from):
    counter figures taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name == "ssm_bwd.hip":
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(path, key):
    """HBM bytes per scan (FETCH_SIZE + WRITE_SIZE of every pass, scaled by
    the copy calibration) recorded for this workload, or None when none was
    taken or the kernels have changed since."""
    try:
        with open(path) as f:
            tj = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not tj or not tj.get("bytes_per_scan") or tj.get("src_sha") != kernel_sources_sha():
        return None
    return tj["bytes_per_scan"]


def pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def settle_clocks(torch, step, ms):
    """Untimed calls of step(i) for `ms` of wall time, synchronising every 8,
    so that the warmup and timed steps that follow run at settled clocks.
    Returns the number of calls."""
    n = 0
    deadline = time.perf_counter() + ms * 1e-3
    while ms > 0 and time.perf_counter() < deadline:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_scan_steps(torch, ssm, sets, cfg, chunk, steps, warmup, hip, decode=True,
                    settle_ms=0.0):
    """Warm up, then time `steps` steps, each the scan of one input set (the
    sets in rotation) followed by one decode token per channel.  Returns the
    total time, the per-step durations of the scan's kernels (from the events
    that its first and last dispatch record) and the number of clock-settling
    steps: before the warmup steps, untimed steps run for `settle_ms` of wall
    time, since the GPU's clocks rise over the first few hundred
    milliseconds of work (the long sequence's scan: 0.86-0.89 ms in the first
    steps of a fresh process, 0.75-0.78 ms after about a second)."""
    batch, d_inner, N, L = cfg["batch"], cfg["d_inner"], cfg["d_state"], cfg["seqlen"]
    code = 1 if cfg["io_dtype"] == "bf16" else 0
    ws = torch.empty(max(1, ssm.ssm_scan_workspace_bytes(batch, d_inner, N, L, code, chunk)),
                     dtype=torch.uint8, device=sets[0]["u"].device)
    # Each input set's two calls are checked and marshalled once: the binding's
    # per-call checks would otherwise leave the GPU waiting between short steps.
    calls = []
    for t in sets:
        scan = ssm.ssm_scan_fwd(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                t["delta_bias"], softplus=True, chunk_size=chunk,
                                y=t["y"], last_state=t["last"], workspace=ws, prepare=True)
        dec = ssm.ssm_state_update(t["last"], t["dec_u"], t["dec_delta"], t["A"], t["dec_B"],
                                   t["dec_C"], t["D"], t["dec_z"], y=t["dec_y"],
                                   prepare=True) if decode else None
        calls.append((scan, dec))
    n_sets = len(sets)
    ev = hip.create(2 * (steps + warmup))

    def step(i, evs):
        scan, dec = calls[i % n_sets]
        scan(evs)
        if dec is not None:
            dec()

    settle_steps = 0
    if settle_ms > 0:
        deadline = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < deadline:
            for _ in range(8):
                step(settle_steps, None)
                settle_steps += 1
            torch.cuda.synchronize()
    for i in range(warmup):
        step(i, (ev[2 * i], ev[2 * i + 1]))
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    base = 2 * warmup
    start.record()
    for i in range(steps):
        step(i, (ev[base + 2 * i], ev[base + 2 * i + 1]))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    kern_ms = [hip.elapsed_ms(ev[base + 2 * i], ev[base + 2 * i + 1]) for i in range(steps)]
    hip.destroy(ev)
    del ws
    return total_ms, kern_ms, settle_steps


def bench_scan_step(args, torch, ssm, dev):
    """The default line: one step = the scan of the workload + one decode
    token per channel; the roofline covers every pass of the scan."""
    cfg = dict(ssm_inputs.CONFIGS[args.config])
    batch, d_inner, N, L = cfg["batch"], cfg["d_inner"], cfg["d_state"], cfg["seqlen"]
    io, gate = cfg["io_dtype"], cfg["gate"]
    code = 1 if io == "bf16" else 0
    set_bytes = algorithmic_bytes(batch, d_inner, N, L, io, gate)
    n_sets = max(2, min(8, -(-3 * CACHE_BYTES // set_bytes)))
    named = CONFIG_CHUNKS.get(args.config, ())
    chunk = args.chunk if args.chunk is not None else HEADLINE_CHUNK.get(args.config, 0)

    # ---- inputs, resident in HBM
    sets = []
    for s in range(n_sets):
        inp = ssm_inputs.make_scan_inputs(batch, d_inner, N, L, io_dtype=io, gate=gate, seed=s)
        dec = ssm_inputs.make_update_inputs(batch, d_inner, N, io_dtype=io, gate=gate,
                                            seed=1000 + s)
        t = {k: upload(inp[k], dev) for k in ("u", "delta", "B", "C", "z")}
        t.update({k: upload(inp[k], dev) for k in ("A", "D", "delta_bias")})
        t["y"] = torch.empty_like(t["u"])
        t["last"] = torch.empty((batch, d_inner, N), dtype=torch.float32, device=dev)
        t.update({"dec_" + k: upload(dec[k], dev) for k in ("u", "delta", "B", "C", "z")})
        t["dec_y"] = torch.empty_like(t["dec_u"])
        sets.append(t)
        del inp, dec
    torch.cuda.synchronize()
    hip = HipEvents()

    total_ms, kern_ms, settle_steps = time_scan_steps(torch, ssm, sets, cfg, chunk, args.steps,
                                                      args.warmup, hip, settle_ms=args.settle_ms)
    K = ssm.ssm_scan_chunk_size(batch, d_inner, N, L, code, chunk)
    plan = ssm.scan_plan(batch, d_inner, N, L, code, chunk)

    ms_per_step = total_ms / args.steps
    chtok = batch * d_inner * (L + 1)
    value = chtok / (ms_per_step * 1e-3)
    kmed = pct(kern_ms, 50)
    hbm_gbs = set_bytes / (kmed * 1e-3) / 1e9
    slots = algorithmic_slots(batch, d_inner, N, L, gate)
    alu_tflops = 2.0 * slots / (kmed * 1e-3) / 1e12
    traffic = load_traffic(args.traffic_json, f"{args.config}@{chunk}")

    # the other chunk lengths the workload names, and the library's own
    # choice, each timed briefly beside the headline (scan and decode steps)
    variants = {}
    if not args.no_variants:
        for k in [c for c in named if c != chunk] + ([0] if chunk != 0 else []):
            vt, vk, _ = time_scan_steps(torch, ssm, sets, cfg, k, max(3, args.steps // 2), 2, hip)
            variants[str(k) if k else "auto"] = {
                "chunk": ssm.ssm_scan_chunk_size(batch, d_inner, N, L, code, k),
                "plan": ssm.scan_plan(batch, d_inner, N, L, code, k),
                "ms_per_step": vt / max(3, args.steps // 2),
                "scan_ms_p50": pct(vk, 50),
                "hbm_frac": set_bytes / (pct(vk, 50) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            }

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "channel-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle": {"ms": args.settle_ms, "steps": settle_steps},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: selective scan batch={batch} d_inner={d_inner} "
                        f"N={N} L={L} {io} I/O (fp32 state and arithmetic)"
                        f"{' + silu gate' if gate else ''}, chunk {K} ({plan}), then one "
                        f"decode token per channel",
            "batch": batch, "d_inner": d_inner, "d_state": N, "seqlen": L, "io_dtype": io,
            "gate": gate, "chunk": K, "chunk_requested": chunk, "plan": plan,
            "input_sets": n_sets,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": hbm_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": hbm_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": f"the whole scan: every dispatch of ssm_scan_fwd ({plan})",
            "kernel_ms": kmed,
            "kernel_ms_p10": pct(kern_ms, 10),
            "kernel_ms_p90": pct(kern_ms, 90),
            "kernel_ms_mean": float(np.mean(kern_ms)),
            "algorithmic_bytes": set_bytes,
            "alu_tflops": alu_tflops,
            "alu_frac_nonpacked": alu_tflops / VALU_PEAK_NONPACKED_TFLOPS,
            "alu_peak_nonpacked": VALU_PEAK_NONPACKED_TFLOPS,
            "alu_frac_packed": alu_tflops / VALU_PEAK_TFLOPS,
            "algorithmic_slots": slots,
        },
        "chunk_variants": variants,
        "versions": versions(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed steps for this much wall time before the warmup steps, so "
                         "that the timed steps run at settled clocks (0: none)")
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(ssm_inputs.CONFIGS))
    ap.add_argument("--chunk", type=int, default=None,
                    help="chunk length (0 = the library's choice; default: the workload's "
                         "headline chunk length, else the library's choice)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the brief timings of the workload's other chunk lengths")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="HBM bytes per launch measured with rocprofv3 counters")
    ap.add_argument("--decode", action="store_true",
                    help="time only the single-token state update of 256 sequences x 5120 "
                         "channels x N=16 (fp32 state, gate) and report it against HBM")
    ap.add_argument("--backward", action="store_true",
                    help="time only the backward pass (ssm_scan_bwd) of the workload, with "
                         "upstream gradients of y and last_state")
    ap.add_argument("--train", action="store_true",
                    help="time one training step of the scan: the forward pass keeping "
                         "checkpoints, then the backward pass reading them")
    ap.add_argument("--variant", choices=("zoh", "conv", "varlen"),
                    help="time only the forward scan of the workload with the zero-order-hold "
                         "term, the fused causal convolution, or packed sequences")
    ap.add_argument("--ckpt", action="store_true",
                    help="with --backward: the backward reads the forward pass's checkpoints "
                         "(the state entering every 8-token tile) instead of recomputing them")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    args = ap.parse_args()

    if args.chunk is None and (args.decode or args.backward or args.train or args.variant):
        args.chunk = 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, "
                 f"WORLD_SIZE={world}); this build has no multi-GPU path.")

    import torch
    import selective_state_space_fwd_amd as ssm

    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": src.numel() * 4, "copies": 5}))
        return

    ssm.load_library()
    dev = torch.device("cuda:0")
    if args.decode:
        print(json.dumps(bench_decode(args, torch, ssm, dev)), flush=True)
        return
    if args.backward:
        print(json.dumps(bench_backward(args, torch, ssm, dev)), flush=True)
        return
    if args.train:
        print(json.dumps(bench_train(args, torch, ssm, dev)), flush=True)
        return
    if args.variant:
        print(json.dumps(bench_variant(args, torch, ssm, dev)), flush=True)
        return
    print(json.dumps(bench_scan_step(args, torch, ssm, dev)), flush=True)


if __name__ == "__main__":
    main()
