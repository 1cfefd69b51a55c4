"""Helpers shared by the tests: run the oracle on a workload, and the parity bars."""
from __future__ import annotations

import numpy as np

import oracle
from mamba2_selective_scan_causalconv1d_amd import workloads as W

# Parity bars (per element): bf16 outputs |err| <= 2e-2 (1 + |ref|); fp32 results
# (SSM states, and the fp32 outputs of the tiny fp32 shape) |err| <= 1e-3 (1 + |ref|).
BF16_BAR = 2e-2
F32_BAR = 1e-3


def bar_for(act: str) -> float:
    return F32_BAR if act == "f32" else BF16_BAR


def max_bar_fraction(got, ref, bar) -> float:
    """max |got - ref| / (bar (1 + |ref|)); <= 1 passes.  NaN anywhere -> inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError("shape %s != %s" % (got.shape, ref.shape))
    if got.size == 0:
        return 0.0
    if not (np.isfinite(got).all() and np.isfinite(ref).all()):
        return float("inf")
    return float(np.max(np.abs(got - ref) / (bar * (1.0 + np.abs(ref)))))


def assert_close(got, ref, bar, what=""):
    f = max_bar_fraction(got, ref, bar)
    assert f <= 1.0, "%s: max error is %.3g x the bar %.1e(1+|ref|)" % (what, f, bar)
    return f


def oracle_conv(wl: W.Workload, xbc=None, conv_pool=None, run_lengths=None, slots=None,
                fresh=None, inplace=False):
    xbc = wl.xbc if xbc is None else xbc
    pool = wl.conv_pool if conv_pool is None else conv_pool
    pool = pool if inplace else pool.copy()
    out = np.zeros_like(xbc)
    st = oracle.conv1d(out, xbc, wl.conv_w, wl.conv_b, pool,
                       wl.run_lengths if run_lengths is None else run_lengths,
                       wl.slots if slots is None else slots, wl.fresh if fresh is None else fresh)
    assert st == 0, st
    return out, pool


def oracle_scan(wl: W.Workload, xa, dt=None, ssm_pool=None, run_lengths=None, slots=None,
                fresh=None, head_mask=None, decode=False, inplace=False):
    sh = wl.shape
    pool = wl.ssm_pool if ssm_pool is None else ssm_pool
    pool = pool if inplace else pool.copy()
    y = np.zeros((xa.shape[0], sh.d_inner), dtype=xa.dtype)
    st = oracle.scan(y, xa, wl.dt if dt is None else dt, wl.a_log, wl.dt_bias, wl.D, pool,
                     wl.run_lengths if run_lengths is None else run_lengths,
                     wl.slots if slots is None else slots, wl.fresh if fresh is None else fresh,
                     sh.ngroups, head_mask=head_mask, decode=decode)
    assert st == 0, st
    return y, pool


def oracle_norm(wl: W.Workload, y, z=None, weight=None, groups=None):
    sh = wl.shape
    out = np.zeros_like(y)
    st = oracle.gated_rmsnorm(out, y, wl.z if z is None else z,
                              wl.norm_w if weight is None else weight,
                              sh.norm_groups if groups is None else groups, sh.eps)
    assert st == 0, st
    return out


def oracle_conv_snap(wl: W.Workload, snap_every, xbc=None, conv_pool=None, run_lengths=None, slots=None,
                     fresh=None):
    """oracle conv with conv-state snapshots every `snap_every` rows: (out, pool, snaps)."""
    xbc = wl.xbc if xbc is None else xbc
    pool = (wl.conv_pool if conv_pool is None else conv_pool).copy()
    rl = wl.run_lengths if run_lengths is None else run_lengths
    n = oracle.snapshot_count(rl, snap_every)
    snaps = np.zeros((n, wl.shape.conv_kernel - 1, wl.shape.conv_dim), dtype=xbc.dtype)
    out = np.zeros_like(xbc)
    st = oracle.conv1d_snap(out, xbc, wl.conv_w, wl.conv_b, pool, snaps, snap_every, rl,
                            wl.slots if slots is None else slots, wl.fresh if fresh is None else fresh)
    assert st == 0, st
    return out, pool, snaps


def oracle_scan_snap(wl: W.Workload, xa, snap_every, dt=None, ssm_pool=None, run_lengths=None, slots=None,
                     fresh=None):
    """oracle scan with SSM-state snapshots every `snap_every` rows: (y, pool, snaps)."""
    sh = wl.shape
    pool = (wl.ssm_pool if ssm_pool is None else ssm_pool).copy()
    rl = wl.run_lengths if run_lengths is None else run_lengths
    n = oracle.snapshot_count(rl, snap_every)
    snaps = np.zeros((n, sh.nheads, sh.headdim, sh.d_state), dtype=np.float32)
    y = np.zeros((xa.shape[0], sh.d_inner), dtype=xa.dtype)
    st = oracle.scan_snap(y, xa, wl.dt if dt is None else dt, wl.a_log, wl.dt_bias, wl.D, pool, snaps,
                          snap_every, rl, wl.slots if slots is None else slots,
                          wl.fresh if fresh is None else fresh, sh.ngroups)
    assert st == 0, st
    return y, pool, snaps
