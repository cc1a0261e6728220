"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ssd.h declares, and rejects bad arguments before any
HIP call."""
import ctypes
import os
import re

import pytest

import mamba_ssd_scan_chunked_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

# fake, 256-byte aligned device addresses: validation must fail before they are used
A = 0x10000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ssd.load_library()
    names = declared_functions()
    assert {"ssd_forward", "ssd_validate", "ssd_workspace_size", "ssd_strerror", "ssd_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    assert ssd.version() == 5
    lib = ssd.load_library()
    for code in range(0, 10):
        assert lib.ssd_strerror(code)
    assert b"unknown" in lib.ssd_strerror(99)


def prob(**kw):
    base = dict(batch=4, seqlen=4096, nheads=80, headdim=64, dstate=128, ngroups=1, chunk_len=256, nseqs=None,
                dtype=ssd.DTYPE_BF16, flags=0)
    base.update(kw)
    return ssd.problem(**base)


def test_validate_accepts_the_measured_shapes():
    assert ssd.validate(prob()) == 0
    assert ssd.validate(prob(batch=8, seqlen=2048, nheads=24)) == 0
    for n in (64, 128, 256):
        assert ssd.validate(prob(batch=1, seqlen=16384, nheads=32, dstate=n)) == 0
    assert ssd.validate(prob(batch=1, seqlen=8192, nheads=48, ngroups=8, nseqs=16)) == 0
    assert ssd.validate(prob(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, chunk_len=32,
                             dtype=ssd.DTYPE_F32)) == 0
    for q in (16, 32, 64, 128, 256, 320):                       # chunk lengths the pages' sweeps use
        assert ssd.validate(prob(chunk_len=q)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), 2), (dict(seqlen=-5), 2), (dict(nheads=0), 2), (dict(headdim=0), 2),
    (dict(ngroups=3), 2), (dict(chunk_len=0), 2), (dict(nseqs=-1), 2),
    (dict(chunk_len=48), 3), (dict(chunk_len=8), 3), (dict(chunk_len=100), 3),
    (dict(headdim=48), 3), (dict(dstate=96), 3), (dict(dstate=16), 3), (dict(dtype=7), 3), (dict(flags=8), 3),
    (dict(flags=ssd.FLAG_DT_SCALES_X | ssd.FLAG_ZOH), 3),
    (dict(dtype=ssd.DTYPE_F32, dstate=256), 3),
    # limits: dimensions below 2^31, and one block of tokens addressable with 32-bit byte offsets
    (dict(batch=1 << 31, nseqs=1 << 31), 2), (dict(seqlen=1 << 31), 2),
    (dict(nheads=1 << 20), 3),                        # 64 tokens x 2^20 heads x 64 channels x 4 bytes = 2^34
    (dict(nheads=1 << 16, ngroups=1 << 16), 3),       # 64 tokens x 2^16 groups x 128 x 4 bytes = 2^31
    (dict(batch=1 << 20, nseqs=1 << 20, seqlen=1, nheads=1 << 11), 2),   # 2^31 (row, head) workgroups
])
def test_validate_rejects(kw, code):
    assert ssd.validate(prob(**kw)) == code


def test_workspace_size():
    # enough (row, head) items: one pass per row, intermediates on chip
    assert ssd.workspace_size(prob()) == 0
    assert ssd.workspace_size(prob(headdim=48)) == 0            # invalid problem
    assert ssd.workspace_size(prob(seqlen=0)) == 0
    # 32 items and 256 blocks of 64 tokens: 16 segments per row, 15 segment states
    # (fp32 64 x 128) and decays per (row, head), each region 256-byte aligned
    p = prob(batch=1, seqlen=16384, nheads=32)
    n = 32 * 15
    assert ssd.workspace_size(p) == n * 64 * 128 * 4 + ((n * 4 + 255) // 256) * 256


def test_workspace_size_follows_forced_segments():
    p = prob(batch=1, seqlen=1000, nheads=2, headdim=32, dstate=64, chunk_len=64, segments=1)   # 16 blocks
    assert ssd.workspace_size(p) == 0
    p = prob(batch=1, seqlen=1000, nheads=2, headdim=32, dstate=64, chunk_len=64, segments=5)
    n = 2 * 3                                    # 4 blocks per segment -> 4 segments
    assert ssd.workspace_size(p) == n * 32 * 64 * 4 + 256
    assert ssd.workspace_size(prob(batch=1, seqlen=1000, nheads=2, headdim=32, dstate=64, chunk_len=64)) > 0


def test_segments_and_reserved_fields_are_checked():
    assert ssd.validate(prob(segments=-1)) == 2                 # SSD_ERR_BAD_SHAPE
    p = prob()
    p.reserved = 1
    assert ssd.validate(p) == 3                                 # SSD_ERR_UNSUPPORTED
    assert ssd.validate(prob(segments=7)) == 0
    assert ctypes.sizeof(ssd.Problem) == 80


def _forward(p, **ptrs):
    lib = ssd.load_library()
    names = ["x", "dt", "A_log", "B", "C", "D", "init", "seq", "y", "fin"]
    vals = {n: A + 0x1000000 * (i + 1) for i, n in enumerate(names)}
    vals.update({"D": None, "init": None, "seq": None, "dt_bias": None})
    ws = ptrs.pop("ws", A + 0x40000000)
    wsb = ptrs.pop("wsb", ssd.workspace_size(p))
    vals.update(ptrs)
    order = ["x", "dt", "dt_bias"] + names[2:]
    return lib.ssd_forward(ctypes.byref(p), *[vals[n] for n in order], ws, wsb, None)


def small():
    return prob(batch=1, seqlen=64, nheads=2, headdim=32, dstate=64, chunk_len=64)


def test_forward_rejects_null_pointers():
    for n in ("x", "dt", "A_log", "B", "C", "y"):
        assert _forward(small(), **{n: None}) == 1, n


def test_forward_rejects_misalignment():
    assert _forward(small(), x=A + 0x1000000 + 2) == 4
    assert _forward(small(), y=A + 0x9000000 + 8) == 4
    assert _forward(small(), ws=A + 0x40000000 + 16) == 4


def test_forward_rejects_aliasing():
    assert _forward(small(), y=A + 0x1000000) == 6          # y on top of x
    assert _forward(small(), y=A + 0x4000000) == 6          # y on top of B
    assert _forward(small(), fin=A + 0x3000000) == 6        # final on top of A_log
    assert _forward(small(), fin=A + 0x5000000) == 6        # final on top of C


def test_in_place_state_carry_only_where_it_is_safe():
    """final_state == init_state is accepted for rows scanned in one piece without
    sequence ids, and rejected (ALIAS) where the scan reads an initial state after
    another wave or workgroup may have written the final one: packed sequences, and
    rows split into concurrently scanned segments."""
    st = A + 0x20000000
    torch = pytest.importorskip("torch")
    no_dev = not torch.cuda.is_available()
    if no_dev:
        assert _forward(small(), init=st, fin=st) == 8                   # passes every check
    packed = prob(batch=1, seqlen=64, nheads=2, headdim=32, dstate=64, chunk_len=64, nseqs=3)
    assert _forward(packed, seq=A + 0x8000000, init=st, fin=st) == 6
    # a long row of few heads: 16 segments per row; buffers 1 GiB apart, so that
    # only the state buffers can overlap
    split = prob(batch=1, seqlen=16384, nheads=32)
    assert ssd.workspace_size(split) > 0
    far = {n: A + (i + 1) * (1 << 30) for i, n in enumerate(["x", "dt", "A_log", "B", "C", "y"])}
    st = A + 8 * (1 << 30)
    ws = A + 9 * (1 << 30)
    assert _forward(split, ws=ws, init=st, fin=st, **far) == 6
    assert _forward(split, ws=ws, init=st, fin=st + 256, **far) == 6    # shifted overlap, as before
    if no_dev:
        assert _forward(split, ws=ws, init=st, fin=A + 10 * (1 << 30), **far) == 8   # separate buffers


def test_forward_checks_dt_bias():
    assert _forward(small(), dt_bias=A + 0x30000000 + 2) == 4            # misaligned
    assert _forward(small(), dt_bias=A + 0x9000000) == 6                 # y on top of dt_bias
    assert _forward(small(), dt_bias=A + 0xA000000) == 6                 # final on top of dt_bias


@pytest.mark.parametrize("flags", [0, 1, 2, 4, 1 | 2, 2 | 4])
def test_validate_accepts_step_size_and_scaling_flags(flags):
    assert ssd.validate(prob(flags=flags)) == 0


def test_forward_requires_seq_idx_for_packed_nseqs():
    assert _forward(prob(batch=1, seqlen=64, nheads=2, headdim=32, dstate=64, chunk_len=64, nseqs=3)) == 2


def test_forward_without_device_reports_no_device():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    assert _forward(small()) == 8
    # no workspace is needed, so a NULL one passes every argument check
    assert _forward(small(), ws=None, wsb=0) == 8


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, 2, 32, dtype=torch.bfloat16)
    B = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ssd.forward(x, torch.zeros(1, 64, 2), torch.zeros(2), B, B)


def _step(p, **ptrs):
    lib = ssd.load_library()
    names = ["x", "dt", "A_log", "B", "C", "D", "state", "y"]
    vals = {n: A + 0x1000000 * (i + 1) for i, n in enumerate(names)}
    vals.update({"D": None, "dt_bias": None})
    vals.update(ptrs)
    order = ["x", "dt", "dt_bias"] + names[2:]
    return lib.ssd_step(ctypes.byref(p), *[vals[n] for n in order], None)


def test_step_rejects_bad_arguments():
    one = prob(batch=2, seqlen=1, nheads=4, headdim=64, dstate=128)
    assert _step(prob(batch=2, seqlen=2, nheads=4)) == 2                  # one token only
    assert _step(prob(batch=2, seqlen=1, nheads=4, nseqs=3)) == 2         # no packed sequences
    assert _step(prob(batch=2, seqlen=1, nheads=4, headdim=48)) == 3      # unsupported shape
    for n in ("x", "dt", "A_log", "B", "C", "state", "y"):
        assert _step(one, **{n: None}) == 1, n
    assert _step(one, state=A + 0x7000000 + 8) == 4                      # misaligned state
    assert _step(one, y=A + 0x1000000) == 6                               # y on top of x
    assert _step(one, state=A + 0x4000000) == 6                           # state on top of B
    assert _step(one, y=A + 0x7000000) == 6                               # y on top of the state
    assert _step(one, y=A + 0x30000000, dt_bias=A + 0x30000000) == 6      # y on top of dt_bias
    assert _step(one, dt_bias=A + 0x30000000 + 1) == 4                    # misaligned dt_bias
    assert _step(prob(batch=2, seqlen=1, nheads=4, flags=1 | 4)) == 3      # Euler and hold together


def test_step_without_device_reports_no_device():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    assert _step(prob(batch=2, seqlen=1, nheads=4, headdim=64, dstate=128)) == 8


def _backward(p, **ptrs):
    lib = ssd.load_library()
    names = ["x", "dt", "dt_bias", "A_log", "B", "C", "D", "init", "seq", "dy", "dfinal",
             "dx", "ddt", "dA_log", "dB", "dC", "dD", "dinit", "ddt_bias"]
    vals = {n: A + 0x2000000 * (i + 1) for i, n in enumerate(names)}
    vals.update({"dt_bias": None, "D": None, "init": None, "seq": None, "dfinal": None, "dD": None, "dinit": None,
                 "ddt_bias": None})
    ws = ptrs.pop("ws", A + 0x60000000)
    wsb = ptrs.pop("wsb", ssd.backward_workspace_size(p))
    vals.update(ptrs)
    return lib.ssd_backward(ctypes.byref(p), *[vals[n] for n in names], ws, wsb, None)


def small_bwd(**kw):
    base = dict(batch=1, seqlen=64, nheads=2, headdim=32, dstate=64, chunk_len=64)
    base.update(kw)
    return prob(**base)


def test_backward_workspace_sizes():
    # a per-token scalar and dt, each 64-token block's incoming state (bf16), per-row sums, the
    # sequence table, and per-head dB, dC when 80 heads share one group
    p = prob(ngroups=1)
    bth, bh = 4 * 4096 * 80, 4 * 80
    r = lambda v: (v + 255) // 256 * 256
    # (320 items: rows cut into 4 segments, states and gradients at 3 edges per row)
    hin = 80 * (4 * 64 + 4) * 64 * 128 * 2      # (H, b * blocks + nseqs slots, P, N)
    edges = 4 * 80 * 3
    assert ssd.backward_workspace_size(p) == (2 * r(bth * 4) + r(hin) + r(4 * 4 * 80 * 12) + r(4 * 32)
                                              + 2 * (r(edges * 64 * 128 * 4) + r(edges * 4))
                                              + 2 * r(bth * 128 * 2))
    # one head per group (dB, dC written directly); 32 (row, head) items: rows cut into
    # 16 segments of 256 tokens, with the states and gradients at 15 segment edges
    p = prob(nheads=8, ngroups=8)
    edges = 4 * 8 * 15
    assert ssd.backward_workspace_size(p) == (2 * r(4 * 4096 * 8 * 4) + r(8 * 260 * 64 * 128 * 2) + r(64 * 8 * 12)
                                              + r(4 * 32) + 2 * (r(edges * 64 * 128 * 4) + r(edges * 4)))
    assert ssd.backward_workspace_size(prob(headdim=48)) == 0


def test_backward_rejects_bad_arguments():
    assert _backward(small_bwd(dtype=ssd.DTYPE_F32, dstate=256)) == 3    # no fp32 N = 256 build
    for n in ("x", "dt", "A_log", "B", "C", "dy", "dx", "ddt", "dA_log", "dB", "dC"):
        assert _backward(small_bwd(), **{n: None}) == 1, n
    assert _backward(small_bwd(), ws=None) == 5
    assert _backward(small_bwd(), wsb=16) == 5
    assert _backward(small_bwd(), dy=A + 0x14000000 + 4) == 4            # misaligned dy
    assert _backward(small_bwd(), dB=A + 0x1E000000 + 8) == 4            # misaligned dB
    assert _backward(small_bwd(), dx=A + 0x2000000) == 6                 # dx on top of x
    assert _backward(small_bwd(), dB=A + 0x1A000000) == 6                # dB on top of ddt
    assert _backward(small_bwd(), dinit=A + 0x14000000) == 6             # dinit on top of dy
    assert _backward(small_bwd(), dA_log=A + 0x60000000) == 6            # dA_log in the workspace


def test_packed_sequences_need_at_least_one_sequence():
    # seq_idx with tokens but nseqs = 0: no sequence to clamp the ids to
    p = small_bwd(nseqs=0)
    assert _backward(p, seq=A + 0x8000000) == 2
    q = prob(batch=1, seqlen=64, nheads=2, headdim=32, dstate=64, chunk_len=64, nseqs=0)
    assert _forward(q, seq=A + 0x8000000) == 2


def test_backward_without_device_reports_no_device():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: this call would launch on fake pointers")
    assert _backward(small_bwd()) == 8


def test_binding_checks_caller_outputs_and_workspace():
    """The raw entry points take caller-owned outputs; the binding checks their
    shape, dtype and contiguity and the workspace's size before the library is
    called (a short buffer would be written past its end on the device)."""
    torch = pytest.importorskip("torch")
    p = ssd.problem(1, 64, 2, 32, 64, 1, 64, 1, ssd.DTYPE_BF16, 0)
    x = torch.zeros(1, 64, 2, 32, dtype=torch.bfloat16)
    B = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    dt, A_log = torch.zeros(1, 64, 2), torch.zeros(2)
    fin = torch.zeros(1, 2, 32, 64)
    bad_y = [torch.zeros(1, 64, 2, 16),                            # short
             torch.zeros(1, 64, 2, 32, dtype=torch.bfloat16),      # wrong dtype
             torch.zeros(1, 64, 2, 64)[..., :32]]                  # strided
    for y in bad_y:
        with pytest.raises((ValueError, TypeError)):
            ssd.forward_into(p, x, dt, A_log, B, B, None, None, None, y, fin)
    y = torch.zeros(1, 64, 2, 32)
    with pytest.raises(ValueError):
        ssd.forward_into(p, x, dt, A_log, B, B, None, None, None, y, torch.zeros(1, 2, 32, 32))
    # a split problem needs its workspace, of at least ssd_workspace_size bytes
    q = ssd.problem(1, 16384, 32, 64, 128, 1, 256, 1, ssd.DTYPE_BF16, 0)
    need = ssd.workspace_size(q)
    assert need > 0
    with pytest.raises(ValueError):
        ssd._check_workspace(None, need, torch.device("cpu"))
    with pytest.raises(ValueError):
        ssd._check_workspace(torch.zeros(need - 1, dtype=torch.uint8), need, torch.device("cpu"))
    with pytest.raises(ValueError):
        ssd._check_workspace(torch.zeros(need // 4 + 1, dtype=torch.float32), need, torch.device("cpu"))
    ssd._check_workspace(torch.zeros(need, dtype=torch.uint8), need, torch.device("cpu"))
    # backward outputs
    outs = {"dx": torch.zeros(1, 64, 2, 32), "ddt": torch.zeros(1, 64, 2), "dA_log": torch.zeros(2),
            "dB": torch.zeros(1, 64, 1, 64), "dC": torch.zeros(1, 64, 1, 32)}      # dC short
    ws = torch.zeros(ssd.backward_workspace_size(p), dtype=torch.uint8)
    with pytest.raises(ValueError):
        ssd.backward_into(p, x, dt, None, A_log, B, B, None, None, y, None, outs, ws)


def _forward_noalloc(p, **ptrs):
    lib = ssd.load_library()
    names = ["x", "dt", "dt_bias", "A_log", "B", "C", "D", "init", "seq", "y", "fin"]
    vals = {n: A + (i + 1) * (1 << 30) for i, n in enumerate(names)}
    vals.update({"dt_bias": None, "D": None, "init": None, "seq": None})
    vals.update(ptrs)
    return lib.ssd_forward_noalloc(ctypes.byref(p), *[vals[n] for n in names], None)


def test_noalloc_entry_point_checks_and_limit(monkeypatch):
    """ssd_forward_noalloc runs the argument checks of ssd_forward (no workspace
    argument) and rejects, before any HIP call, a problem whose workspace would
    not fit its static scratch array."""
    assert ssd.noalloc_scratch_bytes() == 32 << 20
    torch = pytest.importorskip("torch")
    no_dev = not torch.cuda.is_available()
    split = prob(batch=1, seqlen=16384, nheads=32)                      # 15.7 MB of segment states
    assert 0 < ssd.workspace_size(split) <= ssd.noalloc_scratch_bytes()
    if no_dev:
        assert _forward_noalloc(split) == 8                             # passes every check
    assert _forward_noalloc(split, x=None) == 1
    assert _forward_noalloc(split, y=A + 1) == 4
    assert _forward_noalloc(split, y=A + 5 * (1 << 30)) == 6           # y on top of B
    st = A + 20 * (1 << 30)
    assert _forward_noalloc(split, init=st, fin=st) == 6               # in place on split rows
    # forced to 64 segments per row, 128 (row, head) items need 258 MB of states
    big = prob(batch=2, seqlen=16384, nheads=64, segments=64)
    assert ssd.workspace_size(big) > ssd.noalloc_scratch_bytes()
    assert _forward_noalloc(big) == 9
    assert b"scratch" in ssd.load_library().ssd_strerror(9)
