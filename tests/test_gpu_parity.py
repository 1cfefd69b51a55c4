"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the seeded workloads.

Bars: bf16 outputs |err| <= 2e-2 (1 + |ref|); fp32 outputs and SSM states |err| <= 1e-3 (1 + |ref|);
conv states, written-slot sets, untouched slots and error behaviour bit-exact.
Per-op checks feed both sides the same inputs (the oracle's upstream outputs); the chained
checks run each side's own pipeline end to end.
"""
import sys

import numpy as np
import pytest
import torch

from mamba2_selective_scan_causalconv1d_amd import workloads as W
from _util import BF16_BAR, F32_BAR, assert_close, bar_for, oracle_conv, oracle_norm, oracle_scan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    import _gpu

    return _gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check_pools(wl, named, ssm_got, ssm_ref, conv_got=None, conv_ref=None):
    """Named slots: SSM within the fp32 bar, conv bit-exact; every other slot untouched."""
    M = wl.shape.pool_slots
    named = set(int(s) for s in named)
    for s in range(M):
        if s in named:
            assert_close(ssm_got[s], ssm_ref[s], F32_BAR, "ssm slot %d" % s)
            if conv_got is not None:
                assert np.array_equal(conv_got[s], conv_ref[s]), "conv slot %d" % s
        else:
            assert ssm_got[s].tobytes() == wl.ssm_pool[s].tobytes(), "untouched ssm slot %d" % s
            if conv_got is not None:
                assert conv_got[s].tobytes() == wl.conv_pool[s].tobytes(), "untouched conv slot %d" % s


def _chained(wl, xa_o, y_g, out_g, bar, what):
    """Print (never assert) how far the GPU's own end-to-end chain sits from the oracle's own
    chain (each side feeding its own rounded intermediates forward).  The per-op checks are the
    parity test; this figure only keeps regressions of the chain visible."""
    y_oo, _ = oracle_scan(wl, xa_o)
    out_oo = oracle_norm(wl, y_oo)
    import _util

    say("  chained (each side's own pipeline, not asserted): y %.3g, out %.3g of bar" % (
        _util.max_bar_fraction(W.act_to_f32(y_g), W.act_to_f32(y_oo), bar),
        _util.max_bar_fraction(W.act_to_f32(out_g), W.act_to_f32(out_oo), bar)))


def _prefill_parity(gpu, wl):
    """Each op of the GPU chain against the oracle run on the same inputs: the conv on the
    workload's rows, the scan on the GPU's conv output, the norm on the GPU's y.  (Comparing
    the two chains end to end would compare each side's own rounding of the intermediates,
    which the scan amplifies: one-ulp bf16 changes in its inputs move y by several bars; that
    figure is printed, not asserted.)"""
    sh = wl.shape
    bar = bar_for(sh.act)
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    say("[%s] T=%d S=%d H=%d P=%d N=%d act=%s" % (wl.name, wl.num_rows, len(wl.run_lengths), sh.nheads,
                                                sh.headdim, sh.d_state, sh.act))
    xa_o, cp_o = oracle_conv(wl)
    xa_g, cp_g = gpu.gpu_conv(wl, wl.xbc, wl.conv_pool, b, p)
    f = assert_close(gpu.f32(xa_g), gpu.f32(xa_o), bar, "conv out")
    say("  conv out: %.3g of bar" % f)
    y_o, sp_o = oracle_scan(wl, xa_g)
    y_g, sp_g = gpu.gpu_scan(wl, xa_g, wl.dt, wl.ssm_pool, b, p)
    f = assert_close(gpu.f32(y_g), gpu.f32(y_o), bar, "scan y")
    say("  scan y: %.3g of bar" % f)
    _check_pools(wl, wl.slots, sp_g, sp_o, cp_g, cp_o)
    out_o = oracle_norm(wl, y_g)
    out_g = gpu.gpu_norm(wl, y_g, wl.z)
    f = assert_close(gpu.f32(out_g), gpu.f32(out_o), bar, "norm out")
    say("  norm out: %.3g of bar" % f)
    _chained(wl, xa_o, y_g, out_g, bar, wl.name)


def test_tiny_fp32(gpu):
    _prefill_parity(gpu, W.tiny_fp32())


def test_130m_prefill(gpu):
    _prefill_parity(gpu, W.layer_130m_prefill())


def test_varlen_prefill(gpu):
    _prefill_parity(gpu, W.varlen_prefill())


def test_varlen_slow_decay(gpu):
    """Slow decay keeps resumed states and the state carried across chunks visible."""
    _prefill_parity(gpu, W.varlen_slow_decay())


def test_long_prefill(gpu):
    """4 x 16384 rows, 48 heads, norm over 8 groups, the launch configuration the bench times:
    every op against the oracle in full (all 48 heads, all rows, every slot)."""
    wl = W.long_prefill()
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    say("[%s] conv" % wl.name)
    xa_o, cp_o = oracle_conv(wl)
    xa_g, cp_g = gpu.gpu_conv(wl, wl.xbc, wl.conv_pool, b, p)
    say("  conv out: %.3g of bar" % assert_close(gpu.f32(xa_g), gpu.f32(xa_o), BF16_BAR, "conv out"))
    say("  scan (oracle on all heads)")
    y_o, sp_o = oracle_scan(wl, xa_g)
    y_g, sp_g = gpu.gpu_scan(wl, xa_g, wl.dt, wl.ssm_pool, b, p)
    say("  scan y: %.3g of bar" % assert_close(gpu.f32(y_g), gpu.f32(y_o), BF16_BAR, "scan y"))
    _check_pools(wl, wl.slots, sp_g, sp_o, cp_g, cp_o)
    del y_o
    out_o = oracle_norm(wl, y_g)  # the norm on the GPU's own y
    out_g = gpu.gpu_norm(wl, y_g, wl.z)
    say("  norm out: %.3g of bar" % assert_close(gpu.f32(out_g), gpu.f32(out_o), BF16_BAR, "norm out"))
    del out_o
    _chained(wl, xa_o, y_g, out_g, BF16_BAR, wl.name)


def _chunk_log_decays(wl, h):
    """Host-side sums of the log-decays -exp(A_log) softplus(dt + dt_bias) of head h over the
    64-row chunks of each run (in double, from the workload's bf16 dt)."""
    dt = (wl.dt[:, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = dt + float(wl.dt_bias[h])
    dtp = np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))
    a = -np.exp(float(wl.a_log[h])) * dtp
    sums, r0 = [], 0
    for L in wl.run_lengths:
        for c in range(0, int(L), 64):
            sums.append(a[r0 + c:r0 + min(c + 64, int(L))].sum())
        r0 += int(L)
    return np.array(sums)


def test_decay_regimes_long(gpu):
    """4 x 16384 rows with A log-spaced over [1e-3, 30] across the 48 heads, two sequences
    resuming: chunks whose log-decay sum is near zero (state carried across the whole run), a few
    units (the carried state shrinks by 2^-20 over several chunks), tens (every chunk) and
    hundreds (the carried state negligible).  The scan on all 48 heads against the oracle, all
    rows, final states and untouched slots (eight heads spanning the range are counted and
    printed)."""
    wl = W.decay_span_prefill()
    sh = wl.shape
    heads = [0, 7, 14, 20, 26, 33, 40, 47]
    classes = np.zeros(4, dtype=np.int64)
    for h in heads:
        c = -_chunk_log_decays(wl, h)
        classes += [np.sum(c < 1.0), np.sum((c >= 1.0) & (c < 13.8)), np.sum((c >= 13.8) & (c <= 60.0)),
                    np.sum(c > 60.0)]
    say("[%s] chunks by -log-decay: <1 %d, 1..13.8 %d, 13.8..60 %d, >60 %d" % ((wl.name,) + tuple(classes)))
    assert np.all(classes >= 100), classes
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    xa_g, _ = gpu.gpu_conv(wl, wl.xbc, wl.conv_pool, b, p)
    y_o, sp_o = oracle_scan(wl, xa_g)
    y_g, sp_g = gpu.gpu_scan(wl, xa_g, wl.dt, wl.ssm_pool, b, p)
    P = sh.headdim
    for h in range(sh.nheads):
        cols = slice(h * P, (h + 1) * P)
        f = assert_close(gpu.f32(y_g[:, cols]), gpu.f32(y_o[:, cols]), BF16_BAR, "y head %d" % h)
        g = max(assert_close(sp_g[s, h], sp_o[s, h], F32_BAR, "state slot %d head %d" % (s, h)) for s in wl.slots)
        if h in heads:
            say("  head %d (A %.3g): y %.3g of bar, states %.3g" % (h, np.exp(wl.a_log[h]), f, g))
    _check_pools(wl, wl.slots, sp_g, sp_o)


@pytest.mark.parametrize("seed", range(3))
def test_random_ragged_batches(gpu, seed):
    """Seeded random batches on the MFMA path's shapes (8 heads x 64, d_state 128): 1 to 9
    sequences of 1 to 700 rows, random fresh flags and distinct slots of a 12-slot pool; every
    op against the oracle."""
    rng = np.random.default_rng(900 + seed)
    S = int(rng.integers(1, 10))
    lens = [int(v) for v in rng.integers(1, 701, S)]
    sh = W.Shape(nheads=8, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=256, norm_groups=2,
                 pool_slots=12, act="bf16")
    wl = W.random_prefill(910 + seed, sh, lens, fresh=[int(v) for v in rng.integers(0, 2, S)],
                          slots=[int(v) for v in rng.permutation(12)[:S]])
    _prefill_parity(gpu, wl)


@pytest.mark.parametrize("S", [256, 257, 300])
def test_many_sequences(gpu, S):
    """Batches of S sequences on the MFMA path's shapes, around the size up to which the
    chunk-sum launch builds the sequence and segment tables itself (256; beyond it the table
    kernel runs first): mostly 1 to 40 rows, five of 200 to 700 rows (several segments each),
    random fresh flags over dirty slots of a 320-slot pool; every op against the oracle."""
    rng = np.random.default_rng(950 + S)
    lens = [int(v) for v in rng.integers(1, 41, S)]
    for i in rng.permutation(S)[:5]:
        lens[int(i)] = int(rng.integers(200, 701))
    sh = W.Shape(nheads=8, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=256, norm_groups=2,
                 pool_slots=320, act="bf16")
    wl = W.random_prefill(960 + S, sh, lens, fresh=[int(v) for v in rng.integers(0, 2, S)],
                          slots=[int(v) for v in rng.permutation(320)[:S]])
    _prefill_parity(gpu, wl)


GENERIC_SHAPES = {
    # the VALU chunked scan (fp32, and bf16 shapes off the MFMA path) stages 64-wide tiles:
    # these cover several n tiles, several p tiles with a partial last one, N not a multiple
    # of 64, three heads per group, and chunks of 48 and 64 rows
    "f32_p64n128": W.Shape(nheads=4, headdim=64, d_state=128, ngroups=2, conv_kernel=4, chunk_size=64,
                           norm_groups=2, pool_slots=8, act="f32"),
    "f32_p96n200": W.Shape(nheads=2, headdim=96, d_state=200, ngroups=1, conv_kernel=3, chunk_size=48,
                           norm_groups=2, pool_slots=8, act="f32"),
    "bf16_3hpg": W.Shape(nheads=6, headdim=64, d_state=128, ngroups=2, conv_kernel=4, chunk_size=256,
                         norm_groups=2, pool_slots=8, act="bf16"),
    "bf16_p128n64": W.Shape(nheads=2, headdim=128, d_state=64, ngroups=1, conv_kernel=4, chunk_size=256,
                            norm_groups=1, pool_slots=8, act="bf16"),
}


@pytest.mark.parametrize("shape", list(GENERIC_SHAPES))
def test_generic_scan_shapes(gpu, shape):
    """The VALU chunked scan on shapes of several 64-wide tiles: runs of 1, 47, 64, 150 and 333
    rows (one chunk, a partial chunk, several chunks), fresh and resumed slots; every op against
    the oracle, final states and untouched slots."""
    sh = GENERIC_SHAPES[shape]
    wl = W.random_prefill(970 + len(shape), sh, [150, 1, 333, 47, 64], fresh=[1, 0, 0, 1, 0], slots=[5, 0, 7, 2, 3])
    _prefill_parity(gpu, wl)


def test_decode_64_steps(gpu):
    """256 one-row requests on 512 slots, 10% fresh over dirty slots, 64 successive steps.
    Each step: conv on the step's rows (both sides), the decode scan on the GPU's conv output,
    the norm on the GPU's y; each side carries its own conv and SSM pools across steps."""
    wl = W.decode_batch()
    sh = wl.shape
    p = gpu.Params(wl)
    fresh0 = wl.fresh
    cp_o, sp_o = wl.conv_pool.copy(), wl.ssm_pool.copy()
    cp_g, sp_g = gpu.ops.to_device(wl.conv_pool), gpu.ops.to_device(wl.ssm_pool)
    dims = gpu.dims_of(sh)
    worst = [0.0, 0.0, 0.0]
    for step, (xbc, z, dt) in enumerate(wl.steps):
        fresh = fresh0 if step == 0 else np.zeros_like(fresh0)
        b = gpu.batch_of(wl, fresh=fresh)
        x = gpu.ops.to_device(xbc)
        xa = torch.empty_like(x)
        gpu.ops.conv1d(xa, x, p.conv_w, p.conv_b, cp_g, b, dims)
        y = torch.empty((x.shape[0], sh.d_inner), dtype=x.dtype, device="cuda")
        gpu.ops.scan_decode(y, xa, gpu.ops.to_device(dt), p.a_log, p.dt_bias, p.D, sp_g, b, dims)
        out = torch.empty_like(y)
        gpu.ops.gated_rmsnorm(out, y, gpu.ops.to_device(z), p.norm_w, sh.norm_groups, sh.eps)
        torch.cuda.synchronize()
        xa_h, y_h, out_h = gpu.ops.to_host(xa), gpu.ops.to_host(y), gpu.ops.to_host(out)
        xa_o, cp_o = oracle_conv(wl, xbc=xbc, conv_pool=cp_o, fresh=fresh, inplace=True)
        y_o, sp_o = oracle_scan(wl, xa_h, dt=dt, ssm_pool=sp_o, fresh=fresh, decode=True, inplace=True)
        out_o = oracle_norm(wl, y_h, z=z)
        fs = (assert_close(gpu.f32(xa_h), gpu.f32(xa_o), BF16_BAR, "conv step %d" % step),
              assert_close(gpu.f32(y_h), gpu.f32(y_o), BF16_BAR, "y step %d" % step),
              assert_close(gpu.f32(out_h), gpu.f32(out_o), BF16_BAR, "out step %d" % step))
        worst = [max(a, c) for a, c in zip(worst, fs)]
        if step % 16 == 0:
            say("  step %d: conv %.3g, y %.3g, out %.3g of bar" % ((step,) + fs))
    say("  decode worst: conv %.3g, y %.3g, out %.3g of bar" % tuple(worst))
    _check_pools(wl, wl.slots, gpu.ops.to_host(sp_g), sp_o, gpu.ops.to_host(cp_g), cp_o)


DECODE_SHAPES = {
    # float4s per head state: 64 (one 64-lane workgroup), 256 (one 256-lane workgroup),
    # 512 (one two-per-thread block), 2048 and 4096 (several blocks per head)
    "f32_p16n16": W.Shape(nheads=4, headdim=16, d_state=16, ngroups=2, conv_kernel=4, chunk_size=16,
                          norm_groups=2, pool_slots=10, act="f32"),
    "p64n16_k3": W.Shape(nheads=4, headdim=64, d_state=16, ngroups=1, conv_kernel=3, chunk_size=16,
                         norm_groups=1, pool_slots=10, act="bf16"),
    "p32n64_k2": W.Shape(nheads=6, headdim=32, d_state=64, ngroups=3, conv_kernel=2, chunk_size=16,
                         norm_groups=3, pool_slots=10, act="bf16"),
    "f32_p64n128": W.Shape(nheads=4, headdim=64, d_state=128, ngroups=2, conv_kernel=4, chunk_size=16,
                           norm_groups=4, pool_slots=10, act="f32"),
    "p128n128": W.Shape(nheads=2, headdim=128, d_state=128, ngroups=1, conv_kernel=4, chunk_size=16,
                        norm_groups=2, pool_slots=10, act="bf16"),
}


@pytest.mark.parametrize("shape", list(DECODE_SHAPES))
def test_decode_shapes(gpu, shape):
    """Three decode steps of 7 one-row sequences (3 fresh on step 0) for each block shape of the
    decode kernel; every op against the oracle on the same inputs, pools carried by each side."""
    sh = DECODE_SHAPES[shape]
    bar = bar_for(sh.act)
    R = 7
    wl = W.random_prefill(60, sh, [1] * R, fresh=[1, 0, 0, 1, 0, 1, 0])
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    cp_o, sp_o = wl.conv_pool.copy(), wl.ssm_pool.copy()
    cp_g, sp_g = gpu.ops.to_device(wl.conv_pool), gpu.ops.to_device(wl.ssm_pool)
    for step in range(3):
        src = wl if step == 0 else W.random_prefill(60 + step, sh, [1] * R, fresh=wl.fresh, slots=wl.slots)
        fresh = wl.fresh if step == 0 else np.zeros_like(wl.fresh)
        b = gpu.batch_of(wl, fresh=fresh)
        x = gpu.ops.to_device(src.xbc)
        xa = torch.empty_like(x)
        gpu.ops.conv1d(xa, x, p.conv_w, p.conv_b, cp_g, b, dims)
        y = torch.empty((R, sh.d_inner), dtype=x.dtype, device="cuda")
        gpu.ops.scan_decode(y, xa, gpu.ops.to_device(src.dt), p.a_log, p.dt_bias, p.D, sp_g, b, dims)
        out = torch.empty_like(y)
        gpu.ops.gated_rmsnorm(out, y, gpu.ops.to_device(src.z), p.norm_w, sh.norm_groups, sh.eps)
        torch.cuda.synchronize()
        xa_h, y_h, out_h = gpu.ops.to_host(xa), gpu.ops.to_host(y), gpu.ops.to_host(out)
        xa_o, cp_o = oracle_conv(wl, xbc=src.xbc, conv_pool=cp_o, fresh=fresh, inplace=True)
        y_o, sp_o = oracle_scan(wl, xa_h, dt=src.dt, ssm_pool=sp_o, fresh=fresh, decode=True, inplace=True)
        out_o = oracle_norm(wl, y_h, z=src.z)
        say("  [%s] step %d: conv %.3g, y %.3g, out %.3g of bar" % (
            shape, step, assert_close(gpu.f32(xa_h), gpu.f32(xa_o), bar, "conv step %d" % step),
            assert_close(gpu.f32(y_h), gpu.f32(y_o), bar, "y step %d" % step),
            assert_close(gpu.f32(out_h), gpu.f32(out_o), bar, "out step %d" % step)))
    _check_pools(wl, wl.slots, gpu.ops.to_host(sp_g), sp_o, gpu.ops.to_host(cp_g), cp_o)


def test_decode_past_grid_limit_and_unaligned_flags(gpu):
    """A decode step of 65,600 one-row requests in a tiny fp32 shape (more rows than a grid
    dimension holds: the conv step strides over its rows; the decode scan's item map deals
    262,400 items over the XCDs), with the fresh flags at an odd byte offset of a larger buffer;
    every op against the oracle on the same inputs, pools carried by each side."""
    sh = DECODE_SHAPES["f32_p16n16"]
    R = 65600
    sh = W.Shape(sh.nheads, sh.headdim, sh.d_state, sh.ngroups, sh.conv_kernel, sh.chunk_size, sh.norm_groups,
                 R + 7, sh.act)
    bar = bar_for(sh.act)
    wl = W.random_prefill(66, sh, [1] * R)
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    b = gpu.batch_of(wl)
    spill = torch.zeros(R + 3, dtype=torch.uint8, device="cuda")
    spill[3:] = b.dev_fresh
    b.c.dev_fresh = spill.data_ptr() + 3
    cp_g, sp_g = gpu.ops.to_device(wl.conv_pool), gpu.ops.to_device(wl.ssm_pool)
    x = gpu.ops.to_device(wl.xbc)
    xa = torch.empty_like(x)
    gpu.ops.conv1d(xa, x, p.conv_w, p.conv_b, cp_g, b, dims)
    y = torch.empty((R, sh.d_inner), dtype=x.dtype, device="cuda")
    gpu.ops.scan_decode(y, xa, gpu.ops.to_device(wl.dt), p.a_log, p.dt_bias, p.D, sp_g, b, dims)
    torch.cuda.synchronize()
    xa_h, y_h = gpu.ops.to_host(xa), gpu.ops.to_host(y)
    xa_o, cp_o = oracle_conv(wl)
    y_o, sp_o = oracle_scan(wl, xa_h, decode=True)
    say("  %d requests: conv %.3g, y %.3g of bar" % (
        R, assert_close(gpu.f32(xa_h), gpu.f32(xa_o), bar, "conv"), assert_close(gpu.f32(y_h), gpu.f32(y_o), bar, "y")))
    sp_h, cp_h = gpu.ops.to_host(sp_g), gpu.ops.to_host(cp_g)
    named = np.asarray(wl.slots)
    assert_close(sp_h[named], sp_o[named], F32_BAR, "ssm slots")
    assert np.array_equal(cp_h[named], cp_o[named]), "conv slots"
    rest = np.setdiff1d(np.arange(sh.pool_slots), named)
    assert sp_h[rest].tobytes() == wl.ssm_pool[rest].tobytes() and cp_h[rest].tobytes() == wl.conv_pool[rest].tobytes()


# ------------------------------------------------------------ invariants and edge cases

SMALL = W.Shape(nheads=4, headdim=8, d_state=8, ngroups=2, conv_kernel=4, chunk_size=16, norm_groups=2,
                pool_slots=6, act="bf16")
MFMA_SHAPE = W.Shape(nheads=4, headdim=64, d_state=128, ngroups=2, conv_kernel=4, chunk_size=256,
                     norm_groups=1, pool_slots=6, act="bf16")
SHAPES = {"small": SMALL, "p64n128": MFMA_SHAPE}


@pytest.mark.parametrize("shape", list(SHAPES))
def test_ragged_batch_with_short_runs(gpu, shape):
    """Runs of 1, 2 (shorter than the conv history), ragged multi-chunk runs, fresh and resumed."""
    sh = SHAPES[shape]
    lens = [1, 2, 3, 77, 300, 5, 129]
    wl = W.random_prefill(50, W.Shape(**{**sh.__dict__, "pool_slots": 9}), lens,
                          fresh=[1, 0, 0, 1, 0, 1, 0])
    _prefill_parity(gpu, wl)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_split_vs_whole(gpu, shape):
    """Conv outputs and states bit-exact between one call and a split {1, 2, L-3, ...};
    the scan within the bars."""
    sh = SHAPES[shape]
    L = 200
    wl = W.random_prefill(51, sh, [L], fresh=[1], slots=[2])
    p = gpu.Params(wl)
    whole_b = gpu.batch_of(wl)
    xa_w, cp_w = gpu.gpu_conv(wl, wl.xbc, wl.conv_pool, whole_b, p)
    y_w, sp_w = gpu.gpu_scan(wl, xa_w, wl.dt, wl.ssm_pool, whole_b, p)
    for split in ([1, 2, L - 3], [64, 1, 63, L - 128]):
        cp, sp = wl.conv_pool.copy(), wl.ssm_pool.copy()
        xs, ys = [], []
        r = 0
        for i, n in enumerate(split):
            b = gpu.batch_of(wl, run_lengths=[n], fresh=[1 if i == 0 else 0])
            xa, cp = gpu.gpu_conv(wl, np.ascontiguousarray(wl.xbc[r:r + n]), cp, b, p)
            y, sp = gpu.gpu_scan(wl, xa, np.ascontiguousarray(wl.dt[r:r + n]), sp, b, p)
            xs.append(xa)
            ys.append(y)
            r += n
        assert np.array_equal(np.concatenate(xs), xa_w)
        assert np.array_equal(cp, cp_w)
        assert_close(gpu.f32(np.concatenate(ys)), gpu.f32(y_w), BF16_BAR, "split y")
        assert_close(sp[2], sp_w[2], F32_BAR, "split state")


@pytest.mark.parametrize("shape", list(SHAPES))
def test_fresh_ignores_dirty_slot(gpu, shape):
    """NaN in the slots of fresh sequences changes nothing (bit for bit)."""
    sh = SHAPES[shape]
    wl = W.random_prefill(52, sh, [70, 9], fresh=[1, 1], slots=[0, 5])
    p = gpu.Params(wl)
    b = gpu.batch_of(wl)
    res = []
    for fill in (np.nan, 0.0):
        cp, sp = wl.conv_pool.copy(), wl.ssm_pool.copy()
        cp[[0, 5]] = W.to_act(np.full(cp[[0, 5]].shape, fill, np.float32), sh.act)
        sp[[0, 5]] = fill
        xa, cp2 = gpu.gpu_conv(wl, wl.xbc, cp, b, p)
        y, sp2 = gpu.gpu_scan(wl, xa, wl.dt, sp, b, p)
        res.append((xa, cp2, y, sp2))
    for a, c in zip(*res):
        assert np.array_equal(a, c)
    assert np.isfinite(gpu.f32(res[0][2])).all()


@pytest.mark.parametrize("shape", list(SHAPES))
def test_swapped_slots_match_solo(gpu, shape):
    sh = SHAPES[shape]
    la, lb = 90, 133
    wl = W.random_prefill(53, sh, [la, lb], fresh=[1, 0], slots=[1, 3])
    p = gpu.Params(wl)
    xa, _ = oracle_conv(wl)
    ya, pa = gpu.gpu_scan(wl, np.ascontiguousarray(xa[:la]), np.ascontiguousarray(wl.dt[:la]), wl.ssm_pool,
                          gpu.batch_of(wl, run_lengths=[la], slots=[1], fresh=[1]), p)
    yb, pb = gpu.gpu_scan(wl, np.ascontiguousarray(xa[la:]), np.ascontiguousarray(wl.dt[la:]), wl.ssm_pool,
                          gpu.batch_of(wl, run_lengths=[lb], slots=[3], fresh=[0]), p)
    sigma = wl.ssm_pool[3].copy()
    for sa, sb in ((1, 3), (3, 1)):
        pool = wl.ssm_pool.copy()
        pool[sb] = sigma
        pool[sa] = -5.0
        y, pp = gpu.gpu_scan(wl, xa, wl.dt, pool, gpu.batch_of(wl, slots=[sa, sb], fresh=[1, 0]), p)
        assert_close(gpu.f32(y[:la]), gpu.f32(ya), BF16_BAR, "a")
        assert_close(gpu.f32(y[la:]), gpu.f32(yb), BF16_BAR, "b")
        assert_close(pp[sa], pa[1], F32_BAR, "state a")
        assert_close(pp[sb], pb[3], F32_BAR, "state b")


@pytest.mark.parametrize("shape", list(SHAPES))
def test_head_to_group(gpu, shape):
    """Zeroing group 1's B and C: heads of group 1 give D*x with a zero state, group 0's heads
    are unchanged."""
    sh = SHAPES[shape]
    wl = W.random_prefill(54, sh, [150], fresh=[1], slots=[2])
    p = gpu.Params(wl)
    b = gpu.batch_of(wl)
    xa, _ = oracle_conv(wl)
    y0, _ = gpu.gpu_scan(wl, xa, wl.dt, wl.ssm_pool, b, p)
    xz = xa.copy()
    Di, GN, N, P = sh.d_inner, sh.ngroups * sh.d_state, sh.d_state, sh.headdim
    xz[:, Di + N:Di + 2 * N] = 0
    xz[:, Di + GN + N:Di + GN + 2 * N] = 0
    y1, s1 = gpu.gpu_scan(wl, xz, wl.dt, wl.ssm_pool, b, p)
    half = sh.nheads // 2
    assert_close(gpu.f32(y1[:, :half * P]), gpu.f32(y0[:, :half * P]), BF16_BAR, "group 0 heads")
    for h in range(half, sh.nheads):
        x = gpu.f32(xa[:, h * P:(h + 1) * P]).astype(np.float64)
        assert_close(gpu.f32(y1[:, h * P:(h + 1) * P]), np.float64(wl.D[h]) * x, BF16_BAR, "D*x head %d" % h)
        assert not s1[2, h].any()


def test_malformed_batches_through_gpu_abi(gpu):
    """Each rejected call leaves outputs and pools byte-identical (device buffers)."""
    from mamba2_selective_scan_causalconv1d_amd import _lib, ops

    wl = W.random_prefill(55, SMALL, [3, 4], fresh=[0, 0], slots=[0, 1])
    p = gpu.Params(wl)
    dims = gpu.dims_of(SMALL)
    x = ops.to_device(wl.xbc)
    dt = ops.to_device(wl.dt)
    out = torch.full_like(x, 7.0)
    y = torch.full((7, SMALL.d_inner), 5.0, dtype=x.dtype, device="cuda")
    cp, sp = ops.to_device(wl.conv_pool), ops.to_device(wl.ssm_pool)
    cases = [([3, 4], [0, 6], _lib.SLOT_OUT_OF_RANGE), ([3, 4], [2, 2], _lib.SLOT_SHARED),
             ([3, 3], [0, 1], _lib.RUN_LENGTHS), ([0, 7], [0, 1], _lib.RUN_LENGTHS)]
    for lens, slots, code in cases:
        b = ops.RecurrentBatch(lens, slots, [0, 0])
        b.c.num_rows = 7
        with pytest.raises(ops.Mamba2Error) as e:
            ops.conv1d(out, x, p.conv_w, p.conv_b, cp, b, dims)
        assert e.value.status == code
        with pytest.raises(ops.Mamba2Error) as e:
            ops.scan_prefill(y, x, dt, p.a_log, p.dt_bias, p.D, sp, b, dims)
        assert e.value.status == code
    with pytest.raises(ops.Mamba2Error) as e:
        ops.scan_decode(y, x, dt, p.a_log, p.dt_bias, p.D, sp, ops.RecurrentBatch([3, 4], [0, 1], [0, 0]), dims)
    assert e.value.status == _lib.RUN_LENGTHS
    torch.cuda.synchronize()
    assert (out == 7).all() and (y == 5).all()
    assert np.array_equal(ops.to_host(cp), wl.conv_pool) and np.array_equal(ops.to_host(sp), wl.ssm_pool)


def test_empty_batch_is_a_noop(gpu):
    from mamba2_selective_scan_causalconv1d_amd import ops

    wl = W.random_prefill(56, SMALL, [5], fresh=[0], slots=[0])
    p = gpu.Params(wl)
    dims = gpu.dims_of(SMALL)
    b = ops.RecurrentBatch([], [], [])
    cp, sp = ops.to_device(wl.conv_pool), ops.to_device(wl.ssm_pool)
    e = torch.empty((0, SMALL.conv_dim), dtype=torch.bfloat16, device="cuda")
    ops.conv1d(e, e, p.conv_w, p.conv_b, cp, b, dims)
    ops.scan_prefill(torch.empty((0, SMALL.d_inner), dtype=torch.bfloat16, device="cuda"), e,
                     torch.empty((0, 4), dtype=torch.bfloat16, device="cuda"), p.a_log, p.dt_bias, p.D, sp, b, dims)
    torch.cuda.synchronize()
    assert np.array_equal(ops.to_host(cp), wl.conv_pool) and np.array_equal(ops.to_host(sp), wl.ssm_pool)


@pytest.mark.parametrize("groups,act,Di", [(1, "bf16", 3072), (8, "bf16", 3072), (2, "f32", 3072), (48, "bf16", 3072),
                                           (1, "bf16", 8192), (3, "f32", 12288)])
def test_norm_group_widths(gpu, groups, act, Di):
    """Norm groups of 3072, 384, 1536 (fp32) and 64 columns (the row kernel and, for 48 groups,
    the per-group kernel), and groups wider than the per-group kernel holds in registers (one
    bf16 group of 8192 columns, three fp32 groups of 4096: the two-pass kernel); weight ~ N(1, 0.1)."""
    rng = np.random.default_rng(57)
    y = W.to_act(rng.standard_normal((33, Di), dtype=np.float32), act)
    z = W.to_act(rng.standard_normal((33, Di), dtype=np.float32), act)
    w = rng.normal(1, 0.1, Di).astype(np.float32)
    sh = W.Shape(Di // 64, 64, 128, 1, 4, 256, groups, 1, act)
    wl = W.Workload("norm", 57, sh, np.array([33], np.int32), np.array([0], np.int32), np.array([1], np.uint8),
                    None, None, None, None, None, w, None, None, z=z)
    out_o = oracle_norm(wl, y, z=z, weight=w, groups=groups)
    out_g = gpu.gpu_norm(wl, y, z, weight=w, groups=groups)
    assert_close(gpu.f32(out_g), gpu.f32(out_o), bar_for(act), "norm")
