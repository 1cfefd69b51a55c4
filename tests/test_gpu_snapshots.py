"""State snapshots and rollback through the C ABI against the oracle (GPU).

A snapshot at boundary b is the state a run of the sequence's first b rows would leave in
its slots ("feat(mamba2): integrate model loading and recurrent inference", section "Notes
for Reviewers", names prefix-state snapshots and speculative rollback as the variants that
adaptation leaves out).  Bars as the parity tests: bf16 outputs 2e-2 (1 + |ref|), SSM states
and snapshots 1e-3 (1 + |ref|), conv states and conv snapshots bit-exact.  As there, each op
is fed the same inputs on both sides (the scan gets the GPU's conv output).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mamba2_selective_scan_causalconv1d_amd import workloads as W
from _util import (F32_BAR, assert_close, bar_for, oracle_conv_snap, oracle_scan, oracle_scan_snap)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    import _gpu

    return _gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _gpu_conv_snap(gpu, wl, E, batch, p):
    ops = gpu.ops
    x = ops.to_device(wl.xbc)
    pool = ops.to_device(wl.conv_pool)
    n = ops.snapshot_count(batch, E)
    snaps = torch.zeros((max(n, 1), wl.shape.conv_kernel - 1, wl.shape.conv_dim), dtype=x.dtype, device="cuda")
    out = torch.empty_like(x)
    ops.conv1d_snap(out, x, p.conv_w, p.conv_b, pool, snaps, E, batch, gpu.dims_of(wl.shape))
    torch.cuda.synchronize()
    return ops.to_host(out), ops.to_host(pool), ops.to_host(snaps[:n])


def _gpu_scan_snap(gpu, wl, xa, E, batch, p):
    ops = gpu.ops
    sh = wl.shape
    x = ops.to_device(xa)
    pool = ops.to_device(wl.ssm_pool)
    n = ops.snapshot_count(batch, E)
    snaps = torch.zeros((max(n, 1), sh.nheads, sh.headdim, sh.d_state), dtype=torch.float32, device="cuda")
    y = torch.empty((x.shape[0], sh.d_inner), dtype=x.dtype, device="cuda")
    ops.scan_prefill_snap(y, x, ops.to_device(wl.dt), p.a_log, p.dt_bias, p.D, pool, snaps, E, batch,
                          gpu.dims_of(sh))
    torch.cuda.synchronize()
    return ops.to_host(y), ops.to_host(pool), ops.to_host(snaps[:n])


def _check_named_and_untouched(wl, got, ref, pristine, exact):
    for s in range(wl.shape.pool_slots):
        if s in set(int(v) for v in wl.slots):
            if exact:
                assert np.array_equal(got[s], ref[s]), "slot %d" % s
            else:
                assert_close(got[s], ref[s], F32_BAR, "slot %d" % s)
        else:
            assert got[s].tobytes() == pristine[s].tobytes(), "untouched slot %d" % s


TINY6 = W.Shape(**{**W.SHAPE_TINY.__dict__, "pool_slots": 6})
PREFILL_CASES = {
    # the packed varlen batch (8 runs of 100..4000 rows, half resuming) on the MFMA path,
    # snapshots every 256 rows: segments of 256 rows
    "varlen8_e256": (W.varlen_prefill, 256),
    # the same batch every 640 rows: segments of 640 / 5 = 128 rows
    "varlen8_e640": (W.varlen_prefill, 640),
    # the fp32 path (chunk 16): snapshots every 48 rows, runs shorter and longer than that
    "tiny_f32_e48": (lambda: W.random_prefill(81, TINY6, [130, 7, 48, 49, 200], fresh=[1, 0, 1, 0, 0],
                                              slots=[0, 3, 1, 4, 2]), 48),
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_snapshots(gpu, case):
    make, E = PREFILL_CASES[case]
    wl = make()
    sh = wl.shape
    bar = bar_for(sh.act)
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    n = oracle.snapshot_count(wl.run_lengths, E)
    say("[%s] T=%d S=%d E=%d snapshots=%d" % (case, wl.num_rows, len(wl.run_lengths), E, n))
    assert gpu.ops.snapshot_count(b, E) == n
    xa_g, cp_g, csn_g = _gpu_conv_snap(gpu, wl, E, b, p)
    xa_o, cp_o, csn_o = oracle_conv_snap(wl, E)
    assert_close(gpu.f32(xa_g), gpu.f32(xa_o), bar, "conv out")
    assert np.array_equal(csn_g, csn_o), "conv snapshots"
    _check_named_and_untouched(wl, cp_g, cp_o, wl.conv_pool, exact=True)
    y_g, sp_g, ssn_g = _gpu_scan_snap(gpu, wl, xa_g, E, b, p)
    y_o, sp_o, ssn_o = oracle_scan_snap(wl, xa_g, E)
    f = assert_close(gpu.f32(y_g), gpu.f32(y_o), bar, "scan y")
    fs = assert_close(ssn_g, ssn_o, F32_BAR, "ssm snapshots")
    _check_named_and_untouched(wl, sp_g, sp_o, wl.ssm_pool, exact=False)
    say("  y %.3g, ssm snapshots %.3g of bar; conv snapshots bit-exact" % (f, fs))


VERIFY_SHAPES = {
    "p64n128": W.Shape(nheads=48, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=256,
                       norm_groups=1, pool_slots=96, act="bf16"),
    "f32_p16n16": W.Shape(nheads=4, headdim=16, d_state=16, ngroups=2, conv_kernel=4, chunk_size=16,
                          norm_groups=2, pool_slots=96, act="f32"),
    "p32n64_k2": W.Shape(nheads=6, headdim=32, d_state=64, ngroups=3, conv_kernel=2, chunk_size=16,
                         norm_groups=3, pool_slots=96, act="bf16"),
}


@pytest.mark.parametrize("shape", list(VERIFY_SHAPES))
def test_verify_then_commit(gpu, shape):
    """64 sequences, runs of 1..16 draft rows (some fresh over dirty slots): the verify scan's
    y, per-row snapshots and final slots against the oracle, the conv snapshots bit-exact;
    then a commit of random accepted counts (0, 1..L, beyond L) on both sides."""
    sh = VERIFY_SHAPES[shape]
    bar = bar_for(sh.act)
    rng = np.random.default_rng(82)
    S = 64
    lens = rng.integers(1, 17, S)
    lens[:3] = [1, 16, 2]
    fresh = (rng.random(S) < 0.15).astype(np.uint8)
    slots = rng.permutation(sh.pool_slots)[:S]
    wl = W.random_prefill(83, sh, lens.tolist(), fresh=fresh, slots=slots)
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    ops = gpu.ops
    dims = gpu.dims_of(sh)
    xa_g, cp_g, csn_g = _gpu_conv_snap(gpu, wl, 1, b, p)
    xa_o, cp_o, csn_o = oracle_conv_snap(wl, 1)
    assert_close(gpu.f32(xa_g), gpu.f32(xa_o), bar, "conv out")
    assert np.array_equal(csn_g, csn_o), "conv snapshots"
    # verify scan
    x = ops.to_device(xa_g)
    spool = ops.to_device(wl.ssm_pool)
    n = ops.snapshot_count(b, 1)
    assert n == int(lens.sum()) - S
    ssn = torch.zeros((n, sh.nheads, sh.headdim, sh.d_state), dtype=torch.float32, device="cuda")
    y = torch.empty((x.shape[0], sh.d_inner), dtype=x.dtype, device="cuda")
    ops.scan_verify(y, x, ops.to_device(wl.dt), p.a_log, p.dt_bias, p.D, spool, ssn, b, dims)
    torch.cuda.synchronize()
    y_o, sp_o, ssn_o = oracle_scan_snap(wl, xa_g, 1)
    f = assert_close(gpu.f32(ops.to_host(y)), gpu.f32(y_o), bar, "verify y")
    fs = assert_close(ops.to_host(ssn), ssn_o, F32_BAR, "verify snapshots")
    _check_named_and_untouched(wl, ops.to_host(spool), sp_o, wl.ssm_pool, exact=False)
    say("  [%s] verify y %.3g, snapshots %.3g of bar" % (shape, f, fs))
    # commit: accepted 0, inside the run, the whole run, beyond it
    acc = np.array([int(rng.integers(0, L + 2)) for L in lens], dtype=np.int32)
    acc[:4] = [1, 9, 0, 40]
    cpool = ops.to_device(cp_g)
    ops.commit_snapshots(spool, cpool, ssn, ops.to_device(csn_g), 1,
                         torch.from_numpy(acc).to("cuda"), b, dims)
    torch.cuda.synchronize()
    sp_oc, cp_oc = sp_o.copy(), cp_o.copy()
    assert oracle.commit(sp_oc, cp_oc, ssn_o, csn_o, 1, acc, lens, slots) == 0
    # the oracle commit copies the oracle's snapshots: compare within the state bar
    _check_named_and_untouched(wl, ops.to_host(spool), sp_oc, wl.ssm_pool, exact=False)
    _check_named_and_untouched(wl, ops.to_host(cpool), cp_oc, wl.conv_pool, exact=True)


def test_verify_one_row_equals_decode(gpu):
    """Runs of one row: the verify scan gives the decode scan's y and states bit for bit."""
    sh = VERIFY_SHAPES["p64n128"]
    wl = W.random_prefill(84, sh, [1] * 40, fresh=[int(i % 5 == 0) for i in range(40)])
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    ops = gpu.ops
    dims = gpu.dims_of(sh)
    x, dt = ops.to_device(wl.xbc), ops.to_device(wl.dt)
    outs = []
    for verify in (False, True):
        pool = ops.to_device(wl.ssm_pool)
        y = torch.empty((40, sh.d_inner), dtype=x.dtype, device="cuda")
        if verify:
            ops.scan_verify(y, x, dt, p.a_log, p.dt_bias, p.D, pool, None, b, dims)
        else:
            ops.scan_decode(y, x, dt, p.a_log, p.dt_bias, p.D, pool, b, dims)
        torch.cuda.synchronize()
        outs.append((ops.to_host(y), ops.to_host(pool)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_snapshot_edge_cases(gpu):
    """A stride beyond every run (no snapshots, null snapshot pointers accepted), an empty
    batch, runs longer than 16 rows refused by the verify scan, and a stride the MFMA path
    cannot cut segments for refused by the prefill snapshots; nothing written on refusal."""
    from mamba2_selective_scan_causalconv1d_amd import _lib

    ops = gpu.ops
    sh = VERIFY_SHAPES["p64n128"]
    wl = W.random_prefill(85, sh, [5, 70], fresh=[0, 1], slots=[3, 7])
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    x, dt = ops.to_device(wl.xbc), ops.to_device(wl.dt)
    cp, sp = ops.to_device(wl.conv_pool), ops.to_device(wl.ssm_pool)
    xa = torch.empty_like(x)
    ops.conv1d_snap(xa, x, p.conv_w, p.conv_b, cp, None, 128, b, dims)  # 0 snapshots
    y = torch.full((75, sh.d_inner), 3.0, dtype=x.dtype, device="cuda")
    sp_before = sp.clone()
    with pytest.raises(ops.Mamba2Error) as e:
        ops.scan_verify(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, None, b, dims)
    assert e.value.status == _lib.RUN_LENGTHS
    with pytest.raises(ops.Mamba2Error) as e:
        ops.scan_prefill_snap(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, None, 96, b, dims)
    assert e.value.status == _lib.NOT_IMPLEMENTED
    torch.cuda.synchronize()
    assert (y == 3.0).all() and torch.equal(sp, sp_before)
    ops.scan_prefill_snap(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, None, 128, b, dims)  # 0 snapshots
    torch.cuda.synchronize()
    y_o, sp_o = oracle_scan(wl, ops.to_host(xa))
    assert_close(gpu.f32(ops.to_host(y)), gpu.f32(y_o), bar_for(sh.act), "y")
    empty = ops.RecurrentBatch([], [], [])
    e0 = torch.empty((0, sh.conv_dim), dtype=torch.bfloat16, device="cuda")
    ops.scan_verify(e0, e0, e0, p.a_log, p.dt_bias, p.D, sp, None, empty, dims)
    ops.commit_snapshots(sp, cp, None, None, 1, None, empty, dims)


@pytest.mark.parametrize("make", ["long_prefill", "decay_span_prefill"])
def test_long_snapshots_match_plain_run_and_oracle(gpu, make):
    """Snapshots every 1024 rows on the long shapes: the snapshot entry takes the plain
    prefill's 1024-row segments and kernels (a segment whose predecessor decays below e^-60
    recomputes that predecessor's local state; the others read the chained segment states), so
    y and the final slots agree with the plain run bit for bit; each snapshot, the state entering
    its boundary segment, is compared with the oracle's (the long prefill: every segment decays
    that much; the decay-span batch: mixed per head pair, two sequences resuming)."""
    wl = getattr(W, make)()
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    xa_g, _ = gpu.gpu_conv(wl, wl.xbc, wl.conv_pool, b, p)
    y_plain, sp_plain = gpu.gpu_scan(wl, xa_g, wl.dt, wl.ssm_pool, b, p)
    y_snap, sp_snap, ssn_g = _gpu_scan_snap(gpu, wl, xa_g, 1024, b, p)
    same_y = np.array_equal(y_plain, y_snap)
    same_states = np.array_equal(sp_plain, sp_snap)
    say("[%s] snapshot entry vs plain: y bit-identical %s, slots bit-identical %s" % (wl.name, same_y, same_states))
    assert same_y and same_states
    _, _, ssn_o = oracle_scan_snap(wl, xa_g, 1024)
    say("  %d ssm snapshots: %.3g of bar" % (len(ssn_o), assert_close(ssn_g, ssn_o, F32_BAR, "ssm snapshots")))
