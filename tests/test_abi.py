"""The C ABI on the CPU: the library loads, exports every symbol that
include/ssm.h declares, and validates arguments on the host before any launch.
No kernel is launched here."""
import ctypes
import os
import re

import pytest

import selective_state_space_fwd_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return ssm.load_library()


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("ssm_scan_fwd", "ssm_scan_fwd_ex", "ssm_scan_fwd_conv", "ssm_scan_bwd", "ssm_scan_bwd_ex",
              "ssm_scan_fwd_ckpt", "ssm_scan_ckpt_bytes",
              "ssm_scan_bwd_workspace_bytes", "ssm_state_update", "ssm_scan_workspace_bytes",
              "ssm_scan_chunk_size", "ssm_scan_plan", "ssm_scan_bwd_plan", "ssm_status_string",
              "ssm_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert ssm.ssm_status_string(0) == "SSM_OK"
    for s in range(1, 7):
        assert ssm.ssm_status_string(s).startswith("SSM_ERR_")
    assert ssm.ssm_status_string(99) == "unknown status"
    assert lib.ssm_version() >= 400


def desc(**kw):
    base = dict(batch=2, d_inner=64, d_state=16, seqlen=2048, io_dtype=0, chunk_size=0)
    base.update(kw)
    return ssm.make_desc(**base)


def _al(x):
    return -(-x // 256) * 256


def test_workspace_and_chunk_plan(lib):
    # desc(): batch 2, d_inner 64, N 16, L 2048 -> the d_state <= 16 path,
    # which reads B and C in place (no packed copy) and, with at most 32
    # chunks, folds the chunk operators in the scan pass (no start states):
    # 2 x 4 channel blocks are 8 wavefronts per chunk, so the library cuts the
    # most chunks its minimum length allows (K = 64)
    d = desc()
    K = lib.ssm_scan_chunk_size(ctypes.byref(d))
    assert K == 64
    J = 2048 // K
    need = lib.ssm_scan_workspace_bytes(ctypes.byref(d))
    # chunk end states, step-size sums, and one "keeps its incoming state" flag
    # per (batch row, chunk)
    ops = _al(2 * 64 * J * 16 * 4) + _al(2 * 64 * J * 4) + _al(2 * J * 4)
    assert need == ops
    # chunks of 1024 tokens or more run in one launch, with one 8-byte
    # publication flag per (batch row, channel block, chunk) in addition
    d = desc(seqlen=8192, chunk_size=1024)
    J = 8
    ops = _al(2 * 64 * J * 16 * 4) + _al(2 * 64 * J * 4) + _al(2 * J * 4)
    need = lib.ssm_scan_workspace_bytes(ctypes.byref(d))
    assert need == ops + _al(2 * 4 * J * 8)
    # the scheduling flag changes neither the plan nor the workspace
    d = desc(seqlen=8192, chunk_size=1024, flags=ssm.SSM_FLAG_INDEPENDENT_CHUNKS)
    assert lib.ssm_scan_chunk_size(ctypes.byref(d)) == 1024
    assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == need
    for k in (16, 256, 1024):
        d = desc(chunk_size=k)
        assert lib.ssm_scan_chunk_size(ctypes.byref(d)) == k
    # more than 32 chunks: start states come from the carry kernel
    d = desc(chunk_size=16)
    J = 2048 // 16
    assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == (
        2 * _al(2 * 64 * J * 16 * 4) + _al(2 * 64 * J * 4) + _al(2 * J * 4))
    d = desc(chunk_size=4096)
    assert lib.ssm_scan_chunk_size(ctypes.byref(d)) == 2048     # one chunk
    assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == 0
    d = desc(batch=8, d_inner=5120 * 4)                         # enough channels
    assert lib.ssm_scan_chunk_size(ctypes.byref(d)) == 2048
    # one chunk needs no workspace for any d_state
    for N in (1, 16, 17, 33, 100, 256):
        d = desc(d_state=N, chunk_size=2048)
        assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == 0
    # d_state > 16: operator rows of 32 * 2^k states (wavefronts of 32 states,
    # padded to a power of two)
    for N, NS in ((17, 32), (33, 64), (100, 128), (256, 256)):
        d = desc(d_state=N, chunk_size=256)
        assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == (
            _al(2 * 64 * 8 * NS * 4) + _al(2 * 64 * 8 * 4) + _al(2 * 8 * 4))


def test_in_wave_plan_choice(lib):
    """Chunks of 128 or 256 tokens requested, or chosen by the library for
    1024 to 8192 channels (or fewer channels and at most 1024 tokens), run as
    the in-wave scan (no workspace for a plain
    call, with or without checkpoints); the workspace query still covers the
    chunked plan that calls with packed sequences or the convolution run."""
    def plan(**kw):
        d = desc(**kw)
        return (lib.ssm_scan_plan(ctypes.byref(d)).decode(),
                lib.ssm_scan_chunk_size(ctypes.byref(d)),
                lib.ssm_scan_workspace_bytes(ctypes.byref(d)))
    # the Mamba-130M-shaped layer (3072 channels): chunks of 128
    p, K, ws = plan(batch=2, d_inner=1536)
    assert p.startswith("in-wave") and K == 128 and ws > 0
    # the long sequence (2048 channels): chunks of 256
    p, K, _ = plan(batch=1, d_inner=2048, seqlen=65536, io_dtype=1)
    assert p.startswith("in-wave") and K == 256
    # enough channels for the serial mapping in one chunk
    assert plan(batch=8, d_inner=4096)[0] == "one chunk"
    # few channels and a short sequence: the in-wave scan at chunks of 128
    for d_inner, seqlen in ((64, 256), (1000, 1024), (1, 65)):
        p, K, _ = plan(batch=1, d_inner=d_inner, seqlen=seqlen)
        assert p.startswith("in-wave") and K == min(128, seqlen), (d_inner, seqlen, p)
    # few channels, longer sequences: chunks on separate workgroups
    assert plan(batch=1, d_inner=64, seqlen=1040)[0].startswith("two passes")
    assert plan(batch=1, d_inner=512, seqlen=65536)[0].startswith("two passes")
    # asked for explicitly, at any channel count, also with zero-order hold
    for k in (128, 256):
        p, K, _ = plan(chunk_size=k)
        assert p.startswith("in-wave") and K == k
        assert plan(chunk_size=k, flags=ssm.SSM_FLAG_ZOH)[0].startswith("in-wave")
    assert plan(chunk_size=512)[0].startswith("two passes")
    # d_state above 16: the group kernel
    assert not plan(d_state=17, chunk_size=256)[0].startswith("in-wave")


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), 2), (dict(seqlen=-5), 2), (dict(d_inner=-1), 2),
    (dict(d_state=0), 3), (dict(d_state=257), 3), (dict(io_dtype=7), 3),
    (dict(chunk_size=10), 2), (dict(chunk_size=-16), 2), (dict(seqlen=(1 << 25) + 1), 3),
])
def test_invalid_descriptors(lib, kw, status):
    d = desc(**kw)
    assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.ssm_scan_chunk_size(ctypes.byref(d)) == -1
    # validation fails before any pointer is looked at or anything is launched
    st = lib.ssm_scan_fwd(ctypes.byref(d), 16, 16, 16, 16, 16, None, None, None, 1, 16, None, None)
    assert st == status


def test_null_and_misaligned_arguments(lib):
    d = desc(chunk_size=512)                # 4 chunks: needs a workspace
    d.workspace, d.workspace_bytes = 4096, 1 << 30
    ok = 4096
    args = [ok, ok, ok, ok, ok, None, None, None, 1, ok, None, None]
    assert lib.ssm_scan_fwd(None, *args) == 1
    for i in (0, 1, 2, 3, 4, 9):          # u, delta, A, B, C, y
        bad = list(args)
        bad[i] = None
        assert lib.ssm_scan_fwd(ctypes.byref(d), *bad) == 1
    bad = list(args)
    bad[0] = 4098                           # u misaligned for float32
    assert lib.ssm_scan_fwd(ctypes.byref(d), *bad) == 4
    d.workspace, d.workspace_bytes = None, 0
    assert lib.ssm_scan_fwd(ctypes.byref(d), *args) == 5
    d.workspace, d.workspace_bytes = 4096, 16
    assert lib.ssm_scan_fwd(ctypes.byref(d), *args) == 5


def test_update_validation(lib):
    d = ssm.make_desc(4, 8, 16, 0, 0)
    ok = 4096
    assert lib.ssm_state_update(None, ok, ok, ok, ok, ok, ok, None, None, ok, None) == 1
    assert lib.ssm_state_update(ctypes.byref(d), None, ok, ok, ok, ok, ok, None, None, ok,
                                None) == 1
    d2 = ssm.make_desc(4, 8, 300, 0, 0)
    assert lib.ssm_state_update(ctypes.byref(d2), ok, ok, ok, ok, ok, ok, None, None, ok,
                                None) == 3
    d3 = ssm.make_desc(4, 8, 16, 0, 1)
    assert lib.ssm_state_update(ctypes.byref(d3), ok, 4097, ok, ok, ok, ok, None, None, ok,
                                None) == 4


def test_empty_problems_return_ok_without_launch(lib):
    d = desc(batch=0)
    assert lib.ssm_scan_fwd(ctypes.byref(d), None, None, None, None, None, None, None, None,
                            1, None, None, None) == 0
    d = ssm.make_desc(0, 8, 16, 0, 0)
    assert lib.ssm_state_update(ctypes.byref(d), None, None, None, None, None, None, None,
                                None, None, None) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="build the HIP library"):
        ssm.load_library(tmp_path / "libssm.so")


def test_packed_sequence_validation(lib):
    """ssm_scan_fwd_ex: packed sequences need batch == 1 and n_seqs >= 1, and
    the offset table and initial states must be 4-byte aligned; all checked
    before anything is launched."""
    ok = 4096
    def call(d, h0, cu, n):
        return lib.ssm_scan_fwd_ex(ctypes.byref(d), ok, ok, ok, ok, ok, None, None, None, 1,
                                   h0, cu, n, ok, None, None)
    d = desc(chunk_size=2048)                       # batch 2
    assert call(d, None, ok, 3) == 2
    d1 = desc(batch=1, chunk_size=2048)
    assert call(d1, None, ok, 0) == 2
    assert call(d1, None, ok + 2, 3) == 4
    assert call(d1, ok + 1, ok, 3) == 4
    assert call(d, ok + 1, None, 0) == 4
    # empty problem: nothing to do, nothing launched
    d0 = desc(batch=1, d_inner=0)
    assert call(d0, None, ok, 3) == 0


def test_conv_validation(lib):
    """ssm_scan_fwd_conv: the width must be 1..4 and the weights present."""
    ok = 4096
    d = desc(chunk_size=2048)
    def call(width, weight):
        return lib.ssm_scan_fwd_conv(ctypes.byref(d), ok, weight, None, width, 1, None, ok, ok,
                                     ok, ok, None, None, None, 1, None, None, 0, ok, None, None,
                                     None)
    assert call(0, ok) == 3
    assert call(5, ok) == 3
    assert call(4, None) == 1
    assert call(3, ok + 2) == 4
    assert lib.ssm_scan_fwd_conv(None, ok, ok, None, 4, 1, None, ok, ok, ok, ok, None, None,
                                 None, 1, None, None, 0, ok, None, None, None) == 1


def test_flags_validation(lib):
    """Unknown flag bits and a nonzero reserved field are rejected."""
    ok = 4096
    for flags, reserved, status in ((4, 0, 3), (1 << 31, 0, 3), (1, 1, 3)):
        d = desc(chunk_size=2048)
        d.flags, d.reserved = flags, reserved
        assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) == 0
        assert lib.ssm_scan_fwd(ctypes.byref(d), ok, ok, ok, ok, ok, None, None, None, 1, ok,
                                None, None) == status
        du = ssm.make_desc(4, 8, 16, 0, 0, 0, flags)
        du.reserved = reserved
        assert lib.ssm_state_update(ctypes.byref(du), ok, ok, ok, ok, ok, ok, None, None, ok,
                                    None) == status
    d = desc(chunk_size=2048, flags=ssm.SSM_FLAG_ZOH)
    assert lib.ssm_scan_chunk_size(ctypes.byref(d)) == 2048


def test_backward_state_groups_side_by_side_plan(lib):
    """d_state > 16: groups of 16 states run side by side (one chunk each, du,
    ddelta and dz written to a workspace slot per group and summed at the
    end) when one group's 16-channel blocks fill under half of the 2048
    wavefront slots (1024 with ZOH), P <= 4 groups fill at least three
    quarters, no chunk length is given and the slots take at most 8 GiB;
    otherwise one group per launch.  Seen through the workspace size."""
    def need(**kw):
        return lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc(**kw)))
    slots = lambda P, b, d, L: 3 * P * _al(b * d * L * 4)
    # 512 blocks: four groups side by side (the N = 256 layer's shape)
    assert need(batch=4, d_inner=2048, d_state=256, seqlen=4096) >= slots(4, 4, 2048, 4096)
    assert need(batch=1, d_inner=8192, d_state=80, seqlen=96) >= slots(4, 1, 8192, 96)
    # three groups: three side by side
    assert need(batch=2, d_inner=4096, d_state=48, seqlen=64) >= slots(3, 2, 4096, 64)
    # ZOH: 1024 slots, two groups of 512 blocks
    assert need(batch=1, d_inner=8192, d_state=32, seqlen=64,
                flags=ssm.SSM_FLAG_ZOH) >= slots(2, 1, 8192, 64)
    # a slot per group: five groups, five slots
    assert need(batch=1, d_inner=8192, d_state=80, seqlen=96) >= slots(5, 1, 8192, 96)
    # a chunk length given: one group per launch, no slots
    one = need(batch=1, d_inner=8192, d_state=64, seqlen=128, chunk_size=64)
    assert 0 < one < slots(4, 1, 8192, 128) <= need(batch=1, d_inner=8192, d_state=64,
                                                    seqlen=128)
    # slots beyond 8 GiB (16 groups x 3 x 2 GiB): one group per launch
    big = need(batch=1, d_inner=8192, d_state=256, seqlen=65536)
    assert 0 < big < slots(16, 1, 8192, 65536)
    assert need(batch=1, d_inner=8192, d_state=256, seqlen=1024) >= slots(16, 1, 8192, 1024)


def test_backward_plan_strings(lib):
    """ssm_scan_bwd_plan: with the forward's checkpoints and more 16-channel
    blocks than one round of wavefront slots (2048; 1024 with ZOH), a whole
    round of blocks runs as one chunk and the rest in chunks; otherwise, as
    without checkpoints."""
    p = ssm.scan_bwd_plan
    split = "the blocks of a whole round in one chunk, the rest in chunks"
    chunks = "chunks joined by reverse chunk aggregates"
    assert p(8, 5120, 16, 2048, 1, with_ckpt=True) == split          # the Mamba-2.8B layer
    assert p(8, 5120, 16, 2048, 1) == chunks
    assert p(3, 12288, 16, 256, 0, with_ckpt=True) == split
    assert p(2, 24576, 16, 128, 0, with_ckpt=True) == split
    assert p(3, 6144, 16, 128, 0, zoh=True, with_ckpt=True) == split
    # a chunk length given; blocks within one round; a single chunk
    assert p(8, 5120, 16, 2048, 1, chunk_size=512, with_ckpt=True) == chunks
    assert p(2, 64, 16, 2048, 0, with_ckpt=True) == chunks
    assert p(4, 8192, 16, 300, 0, with_ckpt=True) == "one chunk"
    # d_state above 16 (never with checkpoints)
    assert p(4, 2048, 256, 4096, 0) == "groups of 16 states side by side, one chunk each"
    assert p(2, 40, 48, 300, 0) == "groups of 16 states one per launch"
    assert p(4, 2048, 256, 4096, 0, with_ckpt=True) == "invalid"
    assert p(2, 40, 257, 300, 0) == "invalid"


def test_backward_plan_and_validation(lib):
    """ssm_scan_bwd: any d_state up to 256 (Euler or ZOH, same workspace;
    above 16 in groups of 16 states, without packed sequences or forward
    checkpoints); workspace sized for at most 32 chunks; null and misaligned
    arguments rejected before any launch."""
    d = desc(d_state=257)
    assert lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d)) == 0
    assert lib.ssm_scan_bwd(ctypes.byref(d), *([4096] * 5), None, None, None, 1, None, 4096,
                            None, *([4096] * 5), None, None, None, None, None) == 3
    d17 = desc(d_state=17)
    assert lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d17)) > \
        lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc())) > 0
    ok = 4096
    d17.workspace, d17.workspace_bytes = ok, 1 << 40
    base = [ok, ok, ok, ok, ok, None, None, None, 1, None]
    # d_state > 16: no packed sequences, no forward checkpoints
    assert lib.ssm_scan_bwd_ex(ctypes.byref(d17), *base, ok, 1, None, ok, None,
                               *([ok] * 5), None, None, None, None, None) == 3
    assert lib.ssm_scan_bwd_ex(ctypes.byref(d17), *base, None, 0, ok, ok, None,
                               *([ok] * 5), None, None, None, None, None) == 3
    assert (lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc(flags=ssm.SSM_FLAG_ZOH))) ==
            lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc())) > 0)
    d = desc(chunk_size=16)              # 128 chunks asked: the backward uses at most 32
    need16 = lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d))
    d64 = desc(chunk_size=64)            # exactly 32 chunks
    assert need16 == lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(d64)) > 0
    ok = 4096
    d.workspace, d.workspace_bytes = ok, 1 << 40
    args = [ok, ok, ok, ok, ok, None, None, None, 1, None, ok, None] + [ok] * 5 + [None] * 4
    for i in (0, 1, 2, 3, 4, 10, 12, 13, 14, 15, 16):
        bad = list(args)
        bad[i] = None
        assert lib.ssm_scan_bwd(ctypes.byref(d), *bad, None) == 1, i
    bad = list(args)
    bad[7] = ok + 2                      # delta_bias misaligned
    assert lib.ssm_scan_bwd(ctypes.byref(d), *bad, None) == 4
    bad = list(args)
    bad[6] = ok                          # z without dz
    assert lib.ssm_scan_bwd(ctypes.byref(d), *bad, None) == 1
    d.workspace, d.workspace_bytes = ok, 16
    assert lib.ssm_scan_bwd(ctypes.byref(d), *args, None) == 5
    # packed sequences: batch 1 and at least one sequence, an aligned table
    d.workspace, d.workspace_bytes = ok, 1 << 40
    # (..., softplus, initial_state, cu_seqlens, n_seqs, ckpt, dy, dlast, ...)
    ex = args[:10] + [ok, 3, None] + args[10:]
    assert len(ex) == 24
    assert lib.ssm_scan_bwd_ex(ctypes.byref(d), *ex, None) == 2          # batch 2
    d1 = desc(batch=1, chunk_size=16)
    d1.workspace, d1.workspace_bytes = ok, 1 << 40
    bad = list(ex)
    bad[11] = 0
    assert lib.ssm_scan_bwd_ex(ctypes.byref(d1), *bad, None) == 2        # no sequences
    bad = list(ex)
    bad[10] = ok + 2
    assert lib.ssm_scan_bwd_ex(ctypes.byref(d1), *bad, None) == 4        # misaligned table
    bad = list(ex)
    bad[12] = ok + 4
    assert lib.ssm_scan_bwd_ex(ctypes.byref(d1), *bad, None) == 4        # misaligned checkpoints


def test_checkpoint_plan_and_validation(lib):
    """ssm_scan_ckpt_bytes: 16 floats per 8-token tile per (batch, channel)
    row, d_state <= 16 only; ssm_scan_fwd_ckpt rejects a missing, misaligned
    or d_state > 16 checkpoint array before any launch."""
    d = desc(seqlen=2050)
    assert lib.ssm_scan_ckpt_bytes(ctypes.byref(d)) == 2 * 64 * 257 * 16 * 4
    assert lib.ssm_scan_ckpt_bytes(ctypes.byref(desc(d_state=17))) == 0
    ok = 4096
    d = desc(chunk_size=2048)
    base = [ok, ok, ok, ok, ok, None, None, None, 1, None, None, 0, ok, None]
    assert lib.ssm_scan_fwd_ckpt(ctypes.byref(d), *base, None, None) == 1           # no ckpt
    assert lib.ssm_scan_fwd_ckpt(ctypes.byref(d), *base, ok + 4, None) == 4        # misaligned
    d17 = desc(d_state=17, chunk_size=2048)
    assert lib.ssm_scan_fwd_ckpt(ctypes.byref(d17), *base, ok, None) == 3          # N > 16


def test_forward_auto_chunking(lib):
    """The forward's own chunk length (chunk_size 0).  With 1024 to 8192
    channels (d_state <= 16) the in-wave scan runs chunks of 256 tokens (up
    to 2048 channels, two wavefronts per SIMD) or 128 (three per SIMD).
    Otherwise, two-pass chunks (under 1024 tokens, d_state <= 16) are chosen
    so that the busiest SIMD scans the fewest tokens over both passes, with
    1024 SIMDs.  For d_state > 16 the group path keeps 2048 wavefronts in
    flight: 4 x 2048 channels x 4096 tokens, N = 256 are 4096 wavefronts, one
    chunk."""
    def K(**kw):
        return lib.ssm_scan_chunk_size(ctypes.byref(desc(**kw)))
    assert K(batch=2, d_inner=1536, seqlen=2048) == 128
    assert K(batch=1, d_inner=2048, seqlen=65536, io_dtype=1) == 256
    assert K(batch=1, d_inner=1024, seqlen=65536) == 256
    assert K(batch=4, d_inner=2048, seqlen=2048) == 128
    # past 8192 channels: two-pass chunks (4 x 2560 channels: 640 wavefronts
    # per chunk)
    d = desc(batch=4, d_inner=2560, seqlen=2048)
    assert lib.ssm_scan_plan(ctypes.byref(d)).decode().startswith("two passes")
    # 8 x 5120 channels: 2560 blocks of 16, 2.5 per SIMD: the 512 past the
    # second whole round run as two chunks, cut at 1/2.8 of the sequence
    d = desc(batch=8, d_inner=5120, seqlen=2048, io_dtype=1)
    assert lib.ssm_scan_plan(ctypes.byref(d)).decode().startswith("one chunk, the blocks past")
    assert K(batch=8, d_inner=5120, seqlen=2048, io_dtype=1) == 736
    assert lib.ssm_scan_workspace_bytes(ctypes.byref(d)) >= 2560 * 2 * 8
    # a whole number of rounds: one chunk
    assert K(batch=8, d_inner=4096, seqlen=2048, io_dtype=1) == 2048
    assert K(batch=4, d_inner=2048, d_state=256, seqlen=4096) == 4096
    # few channels and at most 1024 tokens: the in-wave scan's chunks of 128
    assert K(batch=1, d_inner=64, seqlen=256) == 128
    assert K(batch=1, d_inner=16, seqlen=65) == 65
    # one wavefront per chunk: the minimum chunk length, or one chunk when the
    # sequence is no longer than it
    assert K(batch=1, d_inner=16, seqlen=16) == 16
    assert K(batch=1, d_inner=16, seqlen=64) == 64
    assert K(batch=1, d_inner=16, seqlen=1100) == 64
    assert K(batch=1, d_inner=16, seqlen=1) == 1
    # the choice is a minimum of the cost over the candidate chunk counts
    def cost(k, waves, L):
        nj = -(-L // k)
        return k * (5 * -(-waves * nj // 1024) + 4 * -(-waves * (nj - 1) // 1024))
    for b, dI, L in ((1, 768, 4096), (1, 1000, 3000), (4, 2560, 2048), (1, 16, 3000)):
        waves = b * -(-dI // 16)
        got = K(batch=b, d_inner=dI, seqlen=L)
        J0 = -(-2048 // waves)
        cands = {min(L, max(64, -(-(-(-L // J)) // 16) * 16)) for J in range(J0, 2 * J0 + 1)}
        assert got in cands and cost(got, waves, L) == min(cost(k, waves, L) for k in cands), (b, dI, L)


def test_backward_auto_chunking(lib):
    """The backward's own chunk plan, seen through its workspace size (which
    depends on the chunk count): one round of two wavefronts per SIMD when a
    chunk's wavefronts fit (2 x 1536 channels: 10 chunks of 208 tokens, not the
    forward's 16 of 128; 1 x 2048 channels x 64 Ki tokens: 16 of 4096), else
    the fewest rounds x chunk length (8 x 5120 channels: 4 chunks of 512)."""
    def ws(**kw):
        return lib.ssm_scan_bwd_workspace_bytes(ctypes.byref(desc(**kw)))
    c1 = dict(batch=2, d_inner=1536, seqlen=2048)
    assert ws(**c1) == ws(chunk_size=208, **c1) != ws(chunk_size=192, **c1)
    c2 = dict(batch=8, d_inner=5120, seqlen=2048, io_dtype=1)
    assert ws(**c2) == ws(chunk_size=512, **c2) != ws(chunk_size=2048, **c2)
    c3 = dict(batch=1, d_inner=2048, seqlen=65536, io_dtype=1)
    assert ws(**c3) == ws(chunk_size=4096, **c3) != ws(chunk_size=2048, **c3)
    tiny = dict(batch=1, d_inner=64, seqlen=256)     # 4 wavefronts a chunk: 4 chunks of 64
    assert ws(**tiny) == ws(chunk_size=64, **tiny) != ws(chunk_size=256, **tiny)
