"""The C-ABI library on the CPU: it loads, exports every function the header declares,
and rejects malformed calls on the host before any launch (no GPU needed)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", "mamba2.h"), os.path.join(ROOT, "include", "mamba3.h")]


@pytest.fixture(scope="module")
def ops():
    from mamba2_selective_scan_causalconv1d_amd import _lib, build

    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    from mamba2_selective_scan_causalconv1d_amd import ops as o

    return o


def _declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \*]*?\b(mamba[23]_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function(ops):
    names = _declared_functions()
    assert len(names) >= 11, names
    lib = ctypes.CDLL(ops._lib.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    declared_py = {n for n, _, _ in ops._lib.SIGNATURES}
    assert declared_py == set(names)


def _dims(ops, **kw):
    base = dict(nheads=4, headdim=8, d_state=8, ngroups=2, conv_kernel=4, chunk_size=16, pool_slots=6,
                act="bf16")
    base.update(kw)
    return ops.make_dims(**base)


CASES = [
    ("ok", [3, 4], [0, 1], 7, False),
    ("slot_high", [3, 4], [0, 6], 7, False),
    ("slot_negative", [3, 4], [-1, 1], 7, False),
    ("slot_shared", [3, 4], [2, 2], 7, False),
    ("rows_not_covered", [3, 3], [0, 1], 7, False),
    ("rows_overrun", [3, 5], [0, 1], 7, False),
    ("zero_length", [0, 7], [0, 1], 7, False),
    ("negative_length", [-1, 8], [0, 1], 7, False),
    ("decode_ok", [1, 1], [0, 1], 2, True),
    ("decode_long_run", [1, 2], [0, 1], 3, True),
    ("empty", [], [], 0, False),
    ("empty_with_rows", [], [], 3, False),
]


@pytest.mark.parametrize("name,lens,slots,T,decode", CASES)
def test_validation_agrees_with_oracle_rules(ops, name, lens, slots, T, decode):
    """The library's host checks and the oracle's (written separately from the same page
    rules) give the same status for every case."""
    b = ops.RecurrentBatch(lens, slots, [0] * len(lens), device=None)
    b.c.num_rows = T
    got = ops.validate(b, _dims(ops), decode)
    want = oracle.check_batch(T, lens, slots, 6, decode)
    assert got == want, (name, got, want)


def test_entry_points_reject_before_launch(ops):
    """Malformed batches and unsupported dims return their status from every entry point
    on a machine with no GPU (nothing is launched, nothing is written).  The calls pass host
    pointers, so the test is kept off machines with a GPU: the same rejections are checked
    through the GPU path, with device buffers, by the gpu-marked tests."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("host-pointer rejection checks run on CPU-only machines")
    from mamba2_selective_scan_causalconv1d_amd import _lib

    d = _dims(ops)
    host = np.zeros(4096, dtype=np.float32)
    p = host.ctypes.data
    for lens, slots, code in (([3, 4], [2, 2], _lib.SLOT_SHARED), ([3, 4], [0, 9], _lib.SLOT_OUT_OF_RANGE),
                              ([3, 3], [0, 1], _lib.RUN_LENGTHS)):
        b = ops.RecurrentBatch(lens, slots, [0] * len(lens), device=None)
        b.c.num_rows = 7
        L = ops.LIB
        assert L.mamba2_conv1d(p, p, p, p, p, b.ref(), ctypes.byref(d), None) == code
        assert L.mamba2_scan_prefill(p, p, p, p, p, p, p, b.ref(), ctypes.byref(d), p, 1 << 20, None) == code
        assert L.mamba2_scan_decode(p, p, p, p, p, p, p, b.ref(), ctypes.byref(d), None) in (
            code, _lib.RUN_LENGTHS)
    assert not host.any()
    b = ops.RecurrentBatch([3, 4], [0, 1], [0, 0], device=None)
    L = ops.LIB
    # null pointers
    assert L.mamba2_conv1d(None, p, p, p, p, b.ref(), ctypes.byref(d), None) == _lib.INVALID_ARGUMENT
    # device buffers moved in 16-byte units must be 16-byte aligned
    assert p % 16 == 0
    q = p + 4
    assert L.mamba2_conv1d(p, q, p, p, p, b.ref(), ctypes.byref(d), None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_conv1d(p, p, p, p, q, b.ref(), ctypes.byref(d), None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_scan_prefill(p, q, p, p, p, p, p, b.ref(), ctypes.byref(d), p, 1 << 20, None) == \
        _lib.INVALID_ARGUMENT
    assert L.mamba2_scan_prefill(p, p, p, p, p, p, q, b.ref(), ctypes.byref(d), p, 1 << 20, None) == \
        _lib.INVALID_ARGUMENT
    assert L.mamba2_gated_rmsnorm(p, p, q, p, 2, 1e-5, 4, 64, 1, None) == _lib.INVALID_ARGUMENT
    # bad dims
    bad = _dims(ops, nheads=3)  # not a multiple of ngroups
    assert L.mamba2_validate(b.ref(), ctypes.byref(bad), 0) == _lib.INVALID_ARGUMENT
    bad = _dims(ops, act=5)
    assert L.mamba2_validate(b.ref(), ctypes.byref(bad), 0) == _lib.INVALID_ARGUMENT
    # unsupported conv kernel width / channel count
    k5 = _dims(ops, conv_kernel=5)
    assert L.mamba2_conv1d(p, p, p, p, p, b.ref(), ctypes.byref(k5), None) == _lib.NOT_IMPLEMENTED
    odd = _dims(ops, headdim=3, d_state=4, nheads=2, ngroups=1)  # Dc = 6 + 8 = 14
    assert L.mamba2_conv1d(p, p, p, p, p, b.ref(), ctypes.byref(odd), None) == _lib.NOT_IMPLEMENTED
    # workspace too small
    assert L.mamba2_scan_prefill(p, p, p, p, p, p, p, b.ref(), ctypes.byref(d), p, 16, None) == \
        _lib.WORKSPACE_TOO_SMALL
    # decode needs run lengths of 1
    assert L.mamba2_scan_decode(p, p, p, p, p, p, p, b.ref(), ctypes.byref(d), None) == _lib.RUN_LENGTHS
    # decode launches past the grid's limits (4096 requests x 65536 heads x 8 blocks = 2^31 items)
    wide = _dims(ops, nheads=65536, headdim=64, d_state=128, ngroups=1, pool_slots=4096)
    many = ops.RecurrentBatch([1] * 4096, list(range(4096)), [0] * 4096, device=None)
    assert L.mamba2_scan_decode(p, p, p, p, p, p, p, many.ref(), ctypes.byref(wide), None) == _lib.NOT_IMPLEMENTED
    # norm argument checks
    assert L.mamba2_gated_rmsnorm(p, p, p, p, 3, 1e-5, 4, 64, 1, None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_gated_rmsnorm(p, p, p, p, 2, -1.0, 4, 64, 1, None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_gated_rmsnorm(p, p, p, p, 16, 1e-5, 4, 64, 1, None) == _lib.NOT_IMPLEMENTED
    assert L.mamba2_gated_rmsnorm(p, p, p, p, 1, 1e-5, 0, 64, 1, None) == _lib.OK
    # snapshots, verify and commit: argument checks, then the batch, then what the kernels cover
    mf = _dims(ops, nheads=4, headdim=64, d_state=128, ngroups=1)  # the MFMA path's shape
    assert L.mamba2_snapshot_count(b.ref(), 2) == (3 - 1) // 2 + (4 - 1) // 2
    assert L.mamba2_snapshot_count(b.ref(), 0) == -1
    assert L.mamba2_conv1d_snap(p, p, p, p, p, p, 0, b.ref(), ctypes.byref(d), None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_conv1d_snap(p, p, p, p, p, None, 1, b.ref(), ctypes.byref(d), None) == \
        _lib.INVALID_ARGUMENT  # snapshots to write, no buffer
    assert L.mamba2_conv1d_snap(p, p, p, p, p, q, 1, b.ref(), ctypes.byref(d), None) == _lib.INVALID_ARGUMENT
    shared = ops.RecurrentBatch([3, 4], [2, 2], [0, 0], device=None)
    assert L.mamba2_conv1d_snap(p, p, p, p, p, p, 1, shared.ref(), ctypes.byref(d), None) == _lib.SLOT_SHARED
    assert L.mamba2_scan_prefill_snap(p, p, p, p, p, p, p, p, 96, b.ref(), ctypes.byref(mf), p, 1 << 20,
                                      None) == _lib.NOT_IMPLEMENTED  # 96 rows: not a multiple of 64
    c2 = _dims(ops, chunk_size=2)  # the fp32 path, segments of 2 rows
    assert L.mamba2_scan_prefill_snap(p, p, p, p, p, p, p, None, 2, b.ref(), ctypes.byref(c2), p, 1 << 20,
                                      None) == _lib.INVALID_ARGUMENT  # snapshots to write, no buffer
    assert L.mamba2_scan_prefill_snap_workspace_bytes(b.ref(), ctypes.byref(mf), 96) == 0
    assert L.mamba2_scan_prefill_snap_workspace_bytes(b.ref(), ctypes.byref(mf), 128) > 0
    dec = _dims(ops, nheads=4, headdim=64, d_state=128, ngroups=1)
    long_run = ops.RecurrentBatch([17, 1], [0, 1], [0, 0], device=None)
    assert L.mamba2_scan_verify(p, p, p, p, p, p, p, None, long_run.ref(), ctypes.byref(dec), None) == \
        _lib.RUN_LENGTHS
    assert L.mamba2_scan_verify(p, p, p, p, p, p, p, None, b.ref(), ctypes.byref(d), None) == \
        _lib.NOT_IMPLEMENTED  # 16 vectors per head state, as the decode scan
    assert L.mamba2_commit_snapshots(p, p, p, p, 0, p, b.ref(), ctypes.byref(d), None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_commit_snapshots(p, p, p, p, 1, None, b.ref(), ctypes.byref(d), None) == \
        _lib.INVALID_ARGUMENT
    assert L.mamba2_commit_snapshots(None, p, p, p, 1, p, b.ref(), ctypes.byref(d), None) == \
        _lib.INVALID_ARGUMENT
    assert L.mamba2_commit_snapshots(p, p, p, p, 1, p, shared.ref(), ctypes.byref(d), None) == _lib.SLOT_SHARED
    assert L.mamba2_commit_snapshots(p, p, None, None, 1, p, b.ref(), ctypes.byref(d), None) == _lib.OK
    # projections: sizes, dtype, alignment, then what the kernel covers
    assert L.mamba2_linear(p, p, p, 4, 0, 8, 1, None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_linear(p, p, q, 4, 8, 8, 1, None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_linear(p, p, p, 4, 12, 8, 1, None) == _lib.NOT_IMPLEMENTED  # out_features % 8
    assert L.mamba2_linear(p, p, p, 4, 8, 8, 0, None) == _lib.NOT_IMPLEMENTED  # fp32
    assert L.mamba2_linear(p, p, p, 0, 8, 8, 1, None) == _lib.OK
    # padded batches: the run finder agrees with the oracle's; pack / unpack check lengths first
    assert L.mamba2_pack_rows(p, p, 64, 3, 1, b.ref(), None) == _lib.RUN_LENGTHS  # a run of 4 > max_len 3
    assert L.mamba2_unpack_rows(p, p, 0, 8, 1, b.ref(), None) == _lib.INVALID_ARGUMENT
    assert L.mamba2_pack_rows(p, p, 64, 8, 2, b.ref(), None) == _lib.INVALID_ARGUMENT
    assert not host.any()


def test_state_size_closed_form(ops):
    """InfiniLM PR #575, 'Motivation': conv + fp32 SSM state of mamba2-130m (TP1, BF16) is about
    18.25 MiB per request -- the slot layout [K-1, Dc] act + [H, P, N] fp32 gives that figure."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "state_size_130m.json")))
    d = ops.make_dims(g["nheads"], g["headdim"], g["d_state"], g["ngroups"], g["conv_kernel"], 256, 1,
                      "bf16")
    per_layer = ops.ssm_slot_bytes(d) + ops.conv_slot_bytes(d)
    assert per_layer == g["bytes_per_layer"] == 797184
    assert round(per_layer * g["layers"] / 2 ** 20, 2) == g["mib_per_request_printed"]
    # the readings the figure rules out: K rows of conv state, or an fp32 conv state
    dk = ops.make_dims(g["nheads"], g["headdim"], g["d_state"], g["ngroups"], g["conv_kernel"] + 1, 256, 1,
                       "bf16")
    assert round((ops.ssm_slot_bytes(dk) + ops.conv_slot_bytes(dk)) * 24 / 2 ** 20, 2) != 18.25
    df = ops.make_dims(g["nheads"], g["headdim"], g["d_state"], g["ngroups"], g["conv_kernel"], 256, 1, "f32")
    assert round((ops.ssm_slot_bytes(df) + ops.conv_slot_bytes(df)) * 24 / 2 ** 20, 2) != 18.25


def test_workspace_size(ops):
    d = _dims(ops)
    b = ops.RecurrentBatch([30, 5], [0, 1], [1, 0], device=None)
    n = ops.scan_prefill_workspace_bytes(b, d)
    assert n > 0 and n % 256 == 0
    bad = ops.RecurrentBatch([30, 5], [0, 0], [1, 0], device=None)
    assert ops.scan_prefill_workspace_bytes(bad, d) == 0


def test_padded_runs_agree_with_oracle(ops):
    """The library's host run finder against the oracle's on random masks: left, right and
    no padding, gaps, empty rows, mixed sides."""
    rng = np.random.default_rng(92)
    for trial in range(60):
        B, Lmax = int(rng.integers(1, 6)), int(rng.integers(1, 12))
        lens = rng.integers(1, Lmax + 1, B)
        left = int(rng.integers(0, 2))
        m = np.zeros((B, Lmax), np.uint8)
        for i, L in enumerate(lens):
            if left:
                m[i, Lmax - L:] = 1
            else:
                m[i, :L] = 1
        if trial % 5 == 1:
            m[rng.integers(0, B), rng.integers(0, Lmax)] ^= 1  # a gap, an empty row or a longer run
        if trial % 7 == 2 and B > 1:
            m[0] = m[0][::-1]  # possibly the other side
        st_o, lens_o, left_o = oracle.padded_runs(m)
        got = np.zeros(B, np.int32)
        side = np.zeros(1, np.int32)
        st = ops.LIB.mamba2_padded_runs(m.ctypes.data, B, Lmax, got.ctypes.data, side.ctypes.data)
        assert st == st_o, (trial, m)
        if st == 0:
            assert np.array_equal(got, lens_o) and int(side[0]) == left_o


def test_mamba3_host_checks(ops):
    """The Mamba-3 entry's host checks, before any device access: run lengths, unsupported
    widths, too many rotary pairs; the workspace size is 0 for rejected arguments."""
    from mamba2_selective_scan_causalconv1d_amd import _lib

    d = ops.mamba3_dims(32, 128, 64, 32)
    ok = ops.Mamba3Batch([100, 300], device=None)
    assert ops.mamba3_workspace_bytes(ok, d) > 0
    fake = ctypes.c_void_p(256)
    args = [fake] * 16
    for lens, dims, code in (([100, 0], d, _lib.RUN_LENGTHS), ([5, 5], ops.mamba3_dims(32, 160, 64, 32),
                                                                _lib.NOT_IMPLEMENTED),
                             ([5, 5], ops.mamba3_dims(32, 128, 64, 65), _lib.INVALID_ARGUMENT),
                             ([5, 5], ops.mamba3_dims(32, 128, 72, 32), _lib.NOT_IMPLEMENTED)):
        b = ops.Mamba3Batch(lens, device=None)
        if lens == [100, 0]:
            b.c.num_rows = 100
        st = ops.LIB.mamba3_siso_forward(*args, b.ref(), ctypes.byref(dims), fake, 1 << 30, None)
        assert st == code, (lens, st)
        assert ops.mamba3_workspace_bytes(b, dims) == 0
    # a too-small workspace, and a sum of run lengths other than num_rows
    st = ops.LIB.mamba3_siso_forward(*args, ok.ref(), ctypes.byref(d), fake, 16, None)
    assert st == _lib.WORKSPACE_TOO_SMALL
    bad = ops.Mamba3Batch([100, 300], device=None)
    bad.c.num_rows = 401
    assert ops.LIB.mamba3_siso_forward(*args, bad.ref(), ctypes.byref(d), fake, 1 << 30, None) == _lib.RUN_LENGTHS
