"""Parity of the Mamba-3 SISO forward (mamba3_siso_forward, through the C ABI) with the oracle.

Bars: the bf16 output and the bf16 final angle |err| <= 2e-2 (1 + |ref|) (the angle measured
on the circle: a value just under 2 pi matches one just over 0); the fp32 final SSM and K
states |err| <= 1e-3 (1 + |ref|); the final V state (a copy of the last value) bit-exact.
Every input is checked unchanged after the call."""
import sys

import numpy as np
import pytest
import torch

from mamba2_selective_scan_causalconv1d_amd import workloads as W
from _util import BF16_BAR, F32_BAR, max_bar_fraction

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    import _gpu

    return _gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


INPUTS = ("q", "k", "v", "adt", "dt", "trap", "q_bias", "k_bias", "angles", "d", "z")


def run_gpu(ops, wl):
    T, H, DV = wl.v.shape
    DK, NA, S = wl.q.shape[1], wl.angles.shape[1], len(wl.run_lengths)
    dev = {n: ops.to_device(getattr(wl, n)) for n in INPUTS}
    out = torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda")
    fa = torch.empty((S, H, NA), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((S, H, DV, DK), dtype=torch.float32, device="cuda")
    fk = torch.empty((S, H, DK), dtype=torch.float32, device="cuda")
    fv = torch.empty((S, H, DV), dtype=torch.bfloat16, device="cuda")
    b = ops.Mamba3Batch(wl.run_lengths)
    dims = ops.mamba3_dims(H, DK, DV, NA)
    ops.mamba3_siso_forward(out, fa, fs, fk, fv, *[dev[n] for n in INPUTS], b, dims)
    torch.cuda.synchronize()
    for n in INPUTS:
        assert np.array_equal(ops.to_host(dev[n]), getattr(wl, n)), "input %s was written" % n
    return tuple(ops.to_host(t) for t in (out, fa, fs, fk, fv))


def compare(gpu, wl):
    import oracle

    say("[%s] T=%d S=%d lengths=%s H=%d DK=%d DV=%d NA=%d" % (wl.name, wl.num_rows, len(wl.run_lengths),
                                                             list(wl.run_lengths), wl.v.shape[1], wl.q.shape[1],
                                                             wl.v.shape[2], wl.angles.shape[1]))
    st, o_out, o_fa, o_fs, o_fk, o_fv = oracle.mamba3_forward(wl.q, wl.k, wl.v, wl.adt, wl.dt, wl.trap, wl.q_bias,
                                                              wl.k_bias, wl.angles, wl.d, wl.z, wl.run_lengths)
    assert st == 0
    g_out, g_fa, g_fs, g_fk, g_fv = run_gpu(gpu.ops, wl)
    f_out = max_bar_fraction(W.act_to_f32(g_out), W.act_to_f32(o_out), BF16_BAR)
    ra, ga = W.act_to_f32(o_fa).astype(np.float64), W.act_to_f32(g_fa).astype(np.float64)
    d = np.abs(ga - ra) % (2 * np.pi)
    d = np.minimum(d, 2 * np.pi - d)
    f_ang = float(np.max(d / (BF16_BAR * (1 + np.abs(ra))))) if d.size else 0.0
    f_ssm = max_bar_fraction(g_fs, o_fs, F32_BAR)
    f_k = max_bar_fraction(g_fk, o_fk, F32_BAR)
    say("  out %.3g, final angle %.3g, final ssm %.3g, final k %.3g of bar; final v bit-exact %s"
        % (f_out, f_ang, f_ssm, f_k, np.array_equal(g_fv, o_fv)))
    assert f_out <= 1.0 and f_ang <= 1.0 and f_ssm <= 1.0 and f_k <= 1.0
    assert np.array_equal(g_fv, o_fv)


def test_mamba3_varlen_default(gpu):
    """The seeded packed batch: 3-5 sequences of 3-15 chunks of 64 rows, never a multiple of
    64, 32 heads, Q/K width 128, V width 64, 32 rotary pairs."""
    compare(gpu, W.mamba3_varlen())


@pytest.mark.parametrize("seed", [8, 9])
def test_mamba3_varlen_seeds(gpu, seed):
    compare(gpu, W.mamba3_varlen(seed))


def test_mamba3_slow_decay(gpu):
    """Decay rates log-uniform over [1e-3, 1e-2]: the state carried across every chunk of a
    sequence, and the final states, depend on the whole sequence."""
    compare(gpu, W.mamba3_varlen(10, decay_range=(1e-3, 1e-2), name="mamba3_slow_decay"))


def test_mamba3_edges(gpu):
    """Sequences of 1 row, 63, 64 and 65 rows and one of 129 (chunk boundaries on and off the
    sequence's end), the smallest widths the tiles cover, three heads, no rotary pairs and all
    rotary pairs; one long sequence with 64 rotary pairs."""
    lens = [1, 63, 64, 65, 129]
    compare(gpu, W.mamba3_varlen(11, lengths=lens, H=3, DK=16, DV=16, NA=0, name="mamba3_edges_na0"))
    compare(gpu, W.mamba3_varlen(12, lengths=lens, H=3, DK=32, DV=16, NA=16, name="mamba3_edges_na_full"))
    compare(gpu, W.mamba3_varlen(13, lengths=[700], H=2, DK=128, DV=64, NA=64, name="mamba3_one_seq_64_pairs"))


def test_mamba3_many_chunks_per_workgroup(gpu):
    """Enough heads that each output workgroup walks several chunks of its head, crossing
    sequence ends, ragged chunks and one-row sequences on the way: 256 heads at the smallest
    widths (one workgroup per head takes all eight chunks) and 128 heads at the 128 / 64 widths
    with 32 rotary pairs (two workgroups per head, every other chunk each)."""
    compare(gpu, W.mamba3_varlen(15, lengths=[70, 5, 130, 64, 1], H=256, DK=16, DV=16, NA=4,
                                 name="mamba3_many_chunks_small"))
    compare(gpu, W.mamba3_varlen(16, lengths=[200, 65, 64, 1], H=128, DK=128, DV=64, NA=32,
                                 name="mamba3_many_chunks_128x64"))


@pytest.mark.parametrize("S", [256, 257, 300])
def test_mamba3_many_sequences(gpu, S):
    """Batches of S short sequences (1 to 20 rows, five of 65 to 200) around the size up to
    which the angle-totals launch builds the chunk tables itself (256; beyond it the table
    kernel runs first)."""
    rng = np.random.default_rng(1700 + S)
    lens = [int(v) for v in rng.integers(1, 21, S)]
    for i in rng.permutation(S)[:5]:
        lens[int(i)] = int(rng.integers(65, 201))
    compare(gpu, W.mamba3_varlen(1800 + S, lengths=lens, H=2, DK=16, DV=16, NA=4, name="mamba3_%d_seqs" % S))


def test_mamba3_rejections(gpu):
    """Misaligned outputs, a short workspace, a value width the tiles do not cover: refused
    before any launch, nothing written."""
    from mamba2_selective_scan_causalconv1d_amd import _lib

    ops = gpu.ops
    wl = W.mamba3_varlen(14, lengths=[70, 5], H=2, DK=16, DV=16, NA=4)
    dev = {n: ops.to_device(getattr(wl, n)) for n in INPUTS}
    T, H, DV = wl.v.shape
    out = torch.full((T * H * DV + 8,), 3.0, dtype=torch.bfloat16, device="cuda")
    fa = torch.zeros((2, H, 4), dtype=torch.bfloat16, device="cuda")
    fs = torch.zeros((2, H, DV, 16), dtype=torch.float32, device="cuda")
    fk = torch.zeros((2, H, 16), dtype=torch.float32, device="cuda")
    fv = torch.zeros((2, H, DV), dtype=torch.bfloat16, device="cuda")
    b = ops.Mamba3Batch(wl.run_lengths)
    dims = ops.mamba3_dims(H, 16, DV, 4)
    with pytest.raises(ops.Mamba2Error) as e:  # value width not a multiple of 16
        ops.mamba3_siso_forward(out, fa, fs, fk, fv, *[dev[n] for n in INPUTS], b, ops.mamba3_dims(H, 16, 8, 4))
    assert e.value.status == _lib.NOT_IMPLEMENTED
    with pytest.raises(ops.Mamba2Error) as e:
        ops.mamba3_siso_forward(out[1:], fa, fs, fk, fv, *[dev[n] for n in INPUTS], b, dims)
    assert e.value.status == _lib.INVALID_ARGUMENT
    with pytest.raises(ops.Mamba2Error) as e:
        ops.mamba3_siso_forward(out, fa, fs, fk, fv, *[dev[n] for n in INPUTS], b, dims,
                                workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == _lib.WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert (out == 3).all() and not fs.any() and not fk.any()
