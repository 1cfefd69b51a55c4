"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a worked example printed
on the pages (``tests/golden``), a closed form, a textbook or library routine, an invariant
the pages state, or a brute force on tiny inputs.  Sources:
  * "feat(backend): Mamba2 ops, with CPU reference implementations" (gllm PR #85), sections
    "Ops", "CPU reference" and "Testing";
  * "feat(mamba2): integrate model loading and recurrent inference" (InfiniLM PR #575),
    sections "Motivation" and "Notes for Reviewers" (prefix-state snapshots and speculative
    rollback, which that adaptation leaves out: a snapshot at boundary b is the state a run of
    the first b rows leaves in the slot, pinned below against such runs);
  * "Granite Mamba2 Inference Optimization" (variable-length padded batches through the
    layer's attention mask; the layer's projections around the path).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from mamba2_selective_scan_causalconv1d_amd import workloads as W
from _util import oracle_conv, oracle_conv_snap, oracle_norm, oracle_scan, oracle_scan_snap

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _silu64(v):
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


SMALL = W.Shape(nheads=4, headdim=8, d_state=8, ngroups=2, conv_kernel=4, chunk_size=16,
                norm_groups=2, pool_slots=6, act="f32")


def _small(seed, lens, fresh=None, slots=None, act="f32", a_log_range=(1.0, 16.0), shape=SMALL):
    sh = W.Shape(**{**shape.__dict__, "act": act})
    return W.random_prefill(seed, sh, lens, fresh=fresh, slots=slots, a_log_range=a_log_range)


# ------------------------------------------------------------ worked examples


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_conv_worked_example(orc, act):
    """gllm PR #85 'Testing': pre-activations 0.5+3*1, 0.5+2*1+3*2 fix that w[K-1] multiplies
    the current token; the slot then holds the last K-1 inputs."""
    g = _golden("conv_worked_example.json")
    assert g["pre_activations"][:2] == [0.5 + 3 * 1, 0.5 + 2 * 1 + 3 * 2]
    x = W.to_act(np.array(g["inputs"], dtype=np.float32).reshape(-1, 1), act)
    w = np.array(g["weight"], dtype=np.float32).reshape(1, -1)
    b = np.array([g["bias"]], dtype=np.float32)
    pool = W.to_act(np.full((1, g["kernel"] - 1, 1), 7.0, dtype=np.float32), act)  # dirty, fresh
    out = np.zeros_like(x)
    assert oracle.conv1d(out, x, w, b, pool, [len(g["inputs"])], [0], [1]) == 0
    want = W.to_act(_silu64(g["pre_activations"]).astype(np.float32).reshape(-1, 1), act)
    assert np.array_equal(out, want)
    assert np.array_equal(pool.reshape(-1), W.to_act(np.array(g["new_state"], np.float32), act))


def test_scan_worked_example(orc):
    """gllm PR #85 'Testing': with dt such that softplus(dt) = 1, the two outputs are 7 and
    2/e + 2.5 (inputs reconstructed in the golden file)."""
    g = _golden("scan_worked_example.json")
    dt = np.full((2, 1), math.log(math.e - 1.0), dtype=np.float32)
    xbc = np.array([[g["x"][0], g["B"][0], g["C"][0]], [g["x"][1], g["B"][1], g["C"][1]]],
                   dtype=np.float32)
    pool = np.full((1, 1, 1, 1), 123.0, dtype=np.float32)  # dirty; the sequence is fresh
    y = np.zeros((2, 1), dtype=np.float32)
    st = oracle.scan(y, xbc, dt, np.array([g["a_log"]], np.float32), np.array([g["dt_bias"]], np.float32),
                     np.array([g["D"]], np.float32), pool, [2], [0], [1], 1)
    assert st == 0
    want = np.array([7.0, 2.0 / math.e + 2.5])
    # dt is stored in fp32, so softplus is 1 within 2e-8; the outputs are one fp32 rounding away.
    assert np.allclose(y[:, 0], want, rtol=3e-7, atol=0)
    assert abs(pool[0, 0, 0, 0] - (2.0 / math.e + 2.0)) <= 3e-7 * 3


# ------------------------------------------------------------ exactness invariants


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_split_vs_whole_exact(orc, act):
    """gllm PR #85 'CPU reference'/'Testing': cutting one run into several calls changes no bit
    of the outputs or the states, also when a call holds a single row (fewer rows than the
    conv keeps as history)."""
    L = 40
    wl = _small(11, [L], fresh=[1], slots=[2], act=act)
    xa_w, cpool_w = oracle_conv(wl)
    y_w, spool_w = oracle_scan(wl, xa_w)
    for split in ([1, 2, L - 3], [15, 17, L - 32], [1, 1, 1, L - 3]):
        cpool = wl.conv_pool.copy()
        spool = wl.ssm_pool.copy()
        xa_parts, y_parts = [], []
        r = 0
        for i, n in enumerate(split):
            rows = slice(r, r + n)
            xa, cpool = oracle_conv(wl, xbc=np.ascontiguousarray(wl.xbc[rows]), conv_pool=cpool,
                                    run_lengths=[n], fresh=[1 if i == 0 else 0])
            y, spool = oracle_scan(wl, xa, dt=np.ascontiguousarray(wl.dt[rows]), ssm_pool=spool,
                                   run_lengths=[n], fresh=[1 if i == 0 else 0])
            xa_parts.append(xa)
            y_parts.append(y)
            r += n
        assert np.array_equal(np.concatenate(xa_parts), xa_w)
        assert np.array_equal(np.concatenate(y_parts), y_w)
        assert np.array_equal(cpool, cpool_w)
        assert np.array_equal(spool, spool_w)


def test_resume_from_saved_state_exact(orc):
    """gllm PR #85 'Testing': a scan restarted from the state saved part-way through a run
    gives the remaining outputs and the final state exactly."""
    L, t0 = 48, 21
    wl = _small(12, [L], fresh=[1], slots=[0])
    xa, _ = oracle_conv(wl)
    y_w, spool_w = oracle_scan(wl, xa)
    y_a, spool_a = oracle_scan(wl, np.ascontiguousarray(xa[:t0]), dt=np.ascontiguousarray(wl.dt[:t0]),
                               run_lengths=[t0])
    saved = spool_a[0].copy()
    # resume in a different pool slot, after the original slot was overwritten
    pool = wl.ssm_pool.copy()
    pool[0] = np.nan
    pool[4] = saved
    y_b, spool_b = oracle_scan(wl, np.ascontiguousarray(xa[t0:]), dt=np.ascontiguousarray(wl.dt[t0:]),
                               ssm_pool=pool, run_lengths=[L - t0], slots=[4], fresh=[0])
    assert np.array_equal(np.concatenate([y_a, y_b]), y_w)
    assert np.array_equal(spool_b[4], spool_w[0])


def test_swapped_slots_match_solo_runs(orc):
    """gllm PR #85 'Testing': a fresh and a resuming sequence in one batch, on slots (a, b) and
    then (b, a), give what each gives when run alone."""
    la, lb = 13, 22
    wl = _small(13, [la, lb], fresh=[1, 0], slots=[1, 3])
    sigma_ssm = wl.ssm_pool[3].copy()
    sigma_conv = wl.conv_pool[3].copy()
    xa, _ = oracle_conv(wl)  # the conv output is fixed input for the scan check
    xa_a, xa_b = np.ascontiguousarray(xa[:la]), np.ascontiguousarray(xa[la:])
    dt_a, dt_b = np.ascontiguousarray(wl.dt[:la]), np.ascontiguousarray(wl.dt[la:])
    ya, pa = oracle_scan(wl, xa_a, dt=dt_a, run_lengths=[la], slots=[1], fresh=[1])
    yb, pb = oracle_scan(wl, xa_b, dt=dt_b, run_lengths=[lb], slots=[3], fresh=[0])
    for sa, sb in ((1, 3), (3, 1)):
        pool = wl.ssm_pool.copy()
        pool[sb] = sigma_ssm
        pool[sa] = -5.0  # dirty, the fresh sequence must not read it
        y, p = oracle_scan(wl, xa, ssm_pool=pool, slots=[sa, sb], fresh=[1, 0])
        assert np.array_equal(y[:la], ya) and np.array_equal(y[la:], yb)
        assert np.array_equal(p[sa], pa[1]) and np.array_equal(p[sb], pb[3])
        # conv: same check on the conv states and outputs
        cpool = wl.conv_pool.copy()
        cpool[sb] = sigma_conv
        cpool[sa] = 9
        out, cp = oracle_conv(wl, conv_pool=cpool, slots=[sa, sb], fresh=[1, 0])
        out_a, cpa = oracle_conv(wl, xbc=np.ascontiguousarray(wl.xbc[:la]), run_lengths=[la],
                                 slots=[sa], fresh=[1])
        cp_b0 = wl.conv_pool.copy()
        cp_b0[sb] = sigma_conv
        out_b, cpb = oracle_conv(wl, xbc=np.ascontiguousarray(wl.xbc[la:]), conv_pool=cp_b0,
                                 run_lengths=[lb], slots=[sb], fresh=[0])
        assert np.array_equal(out, np.concatenate([out_a, out_b]))
        assert np.array_equal(cp[sa], cpa[sa]) and np.array_equal(cp[sb], cpb[sb])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_fresh_ignores_dirty_slot(orc, act):
    """gllm PR #85 'Ops'/'Testing': a fresh run starts from zero state and leaves its slot
    unread, so NaN planted in that slot must not reach any output."""
    wl = _small(14, [9, 17], fresh=[1, 1], slots=[0, 5], act=act)
    nan_c = wl.conv_pool.copy()
    nan_c[[0, 5]] = W.to_act(np.full(nan_c[[0, 5]].shape, np.nan, np.float32), act)
    zero_c = wl.conv_pool.copy()
    zero_c[[0, 5]] = 0
    out_n, cp_n = oracle_conv(wl, conv_pool=nan_c)
    out_z, cp_z = oracle_conv(wl, conv_pool=zero_c)
    assert np.array_equal(out_n, out_z) and np.isfinite(W.act_to_f32(out_n)).all()
    assert np.array_equal(cp_n, cp_z)
    nan_s = wl.ssm_pool.copy()
    nan_s[[0, 5]] = np.nan
    zero_s = wl.ssm_pool.copy()
    zero_s[[0, 5]] = 0
    y_n, sp_n = oracle_scan(wl, out_z, ssm_pool=nan_s)
    y_z, sp_z = oracle_scan(wl, out_z, ssm_pool=zero_s)
    assert np.array_equal(y_n, y_z) and np.isfinite(W.act_to_f32(y_n)).all()
    assert np.array_equal(sp_n, sp_z)


def test_head_to_group_mapping(orc):
    """gllm PR #85 'Testing' (head-to-group mapping): with 4 heads in 2 groups, B and C of group 1
    set to zero reduce heads 2 and 3 to y = D*x while heads 0 and 1 keep their outputs (head h
    reads group h / (heads/groups))."""
    wl = _small(15, [30], fresh=[1], slots=[2])
    sh = wl.shape
    xa, _ = oracle_conv(wl)
    y0, p0 = oracle_scan(wl, xa)
    xz = xa.copy()
    Di, GN = sh.d_inner, sh.ngroups * sh.d_state
    N = sh.d_state
    xz[:, Di + N:Di + 2 * N] = 0  # B of group 1
    xz[:, Di + GN + N:Di + GN + 2 * N] = 0  # C of group 1
    y1, p1 = oracle_scan(wl, xz)
    P = sh.headdim
    assert np.array_equal(y1[:, :2 * P], y0[:, :2 * P])
    assert np.array_equal(p1[2, :2], p0[2, :2])
    for h in (2, 3):
        x = xa[:, h * P:(h + 1) * P].astype(np.float64)
        want = (np.float64(wl.D[h]) * x).astype(np.float32)
        assert np.array_equal(y1[:, h * P:(h + 1) * P], want)
        assert not p1[2, h].any()
    assert not np.array_equal(y1[:, 2 * P:], y0[:, 2 * P:])


# ------------------------------------------------------------ error behaviour


def _malformed_cases(M):
    return [
        ("slot_out_of_range_high", [3, 4], [0, M], oracle.SLOT_OUT_OF_RANGE, 7),
        ("slot_out_of_range_neg", [3, 4], [-1, 1], oracle.SLOT_OUT_OF_RANGE, 7),
        ("slot_shared", [3, 4], [2, 2], oracle.SLOT_SHARED, 7),
        ("rows_not_covered", [3, 3], [0, 1], oracle.RUN_LENGTHS, 7),
        ("rows_overrun", [3, 5], [0, 1], oracle.RUN_LENGTHS, 7),
        ("zero_length", [0, 7], [0, 1], oracle.RUN_LENGTHS, 7),
        ("negative_length", [-1, 8], [0, 1], oracle.RUN_LENGTHS, 7),
    ]


def test_malformed_batches_rejected_without_writes(orc):
    """gllm PR #85 'Ops'/'Testing': batches with a slot outside the pool, two sequences on one
    slot, or run lengths whose sum differs from the rows are refused with no write."""
    wl = _small(16, [3, 4], fresh=[0, 0], slots=[0, 1])
    M = wl.shape.pool_slots
    for name, lens, slots, code, T in _malformed_cases(M):
        out = np.full_like(wl.xbc[:T], 77)
        cpool = wl.conv_pool.copy()
        st = oracle.conv1d(out, np.ascontiguousarray(wl.xbc[:T]), wl.conv_w, wl.conv_b, cpool, lens,
                           slots, [0, 0])
        assert st == code, name
        assert np.array_equal(cpool, wl.conv_pool) and (out == 77).all(), name
        y = np.full((T, wl.shape.d_inner), 55, dtype=np.float32)
        spool = wl.ssm_pool.copy()
        st = oracle.scan(y, np.ascontiguousarray(wl.xbc[:T]), np.ascontiguousarray(wl.dt[:T]), wl.a_log,
                         wl.dt_bias, wl.D, spool, lens, slots, [0, 0], wl.shape.ngroups)
        assert st == code, name
        assert np.array_equal(spool, wl.ssm_pool) and (y == 55).all(), name
    # decode: every run length must be 1
    assert oracle.check_batch(3, [1, 2], [0, 1], M, decode=True) == oracle.RUN_LENGTHS
    assert oracle.check_batch(2, [1, 1], [0, 1], M, decode=True) == oracle.OK
    # an empty batch is a no-op
    assert oracle.check_batch(0, [], [], M) == oracle.OK


def test_untouched_slots_bit_identical(orc):
    wl = _small(17, [5, 6], fresh=[0, 1], slots=[4, 1])
    xa, cp = oracle_conv(wl)
    _, sp = oracle_scan(wl, xa)
    for s in range(wl.shape.pool_slots):
        if s in (4, 1):
            continue
        assert cp[s].tobytes() == wl.conv_pool[s].tobytes()
        assert sp[s].tobytes() == wl.ssm_pool[s].tobytes()


# ------------------------------------------------------------ closed forms


def _softplus64(v):
    return np.logaddexp(0.0, v)  # log(1 + e^v), a library routine


def _unrolled_scan(wl, xa, h0):
    """y_t = sum_{j<=t} (C_t.B_j) exp(sum_{k=j+1..t} a_k) dt'_j x_j
             + exp(sum_{k<=t} a_k) C_t.h0 + D x_t,  a_k = -exp(A_log) dt'_k.
    The same recurrence written out as a sum (double, numpy), one head at a time."""
    sh = wl.shape
    H, P, N, G = sh.nheads, sh.headdim, sh.d_state, sh.ngroups
    Di = H * P
    X = W.act_to_f32(xa).astype(np.float64)
    dt = W.act_to_f32(wl.dt).astype(np.float64)
    T = X.shape[0]
    y = np.zeros((T, Di))
    final = np.zeros((H, P, N))
    for h in range(H):
        g = h // (H // G)
        B = X[:, Di + g * N:Di + (g + 1) * N]
        C = X[:, Di + G * N + g * N:Di + G * N + (g + 1) * N]
        x = X[:, h * P:(h + 1) * P]
        dtp = _softplus64(dt[:, h] + np.float64(wl.dt_bias[h]))
        a = -np.exp(np.float64(wl.a_log[h])) * dtp
        cs = np.concatenate([[0.0], np.cumsum(a)])  # cs[t+1] = sum_{k<=t} a_k
        for t in range(T):
            w = np.exp(cs[t + 1] - cs[1:t + 2]) * dtp[:t + 1] * (B[:t + 1] @ C[t])
            y[t, h * P:(h + 1) * P] = (w[:, None] * x[:t + 1]).sum(0) + np.exp(cs[t + 1]) * (
                h0[h] @ C[t]) + np.float64(wl.D[h]) * x[t]
        wT = np.exp(cs[T] - cs[1:]) * dtp
        final[h] = np.exp(cs[T]) * h0[h] + np.einsum("t,tp,tn->pn", wT, x, B)
    return y, final


@pytest.mark.parametrize("a_log_range", [(1.0, 16.0), (1e-3, 1e-2)])
def test_unrolled_closed_form(orc, a_log_range):
    """The per-token loop equals the unrolled sum of the recurrence (resumed state included)."""
    wl = _small(18, [40], fresh=[0], slots=[3], a_log_range=a_log_range)
    xa, _ = oracle_conv(wl)
    y, pool = oracle_scan(wl, xa)
    y_ref, fin = _unrolled_scan(wl, xa, wl.ssm_pool[3].astype(np.float64))
    # the oracle rounds the state to fp32 once per token: ~T fp32 roundings
    tol = 1e-5
    assert np.max(np.abs(y - y_ref) / (1 + np.abs(y_ref))) < tol
    assert np.max(np.abs(pool[3] - fin) / (1 + np.abs(fin))) < tol


def test_prefix_sum_limit(orc):
    """A_log = -40 makes every decay factor exactly 1 in double, so the state is a running sum:
    h_t = h_0 + sum_{j<=t} dt'_j x_j (x) B_j (numpy cumsum)."""
    wl = _small(19, [33], fresh=[0], slots=[1])
    wl.a_log[:] = -40.0
    xa, _ = oracle_conv(wl)
    y, pool = oracle_scan(wl, xa)
    sh = wl.shape
    H, P, N, G = sh.nheads, sh.headdim, sh.d_state, sh.ngroups
    Di = H * P
    X = xa.astype(np.float64)
    dt = wl.dt.astype(np.float64)
    for h in range(H):
        g = h // (H // G)
        B = X[:, Di + g * N:Di + (g + 1) * N]
        C = X[:, Di + G * N + g * N:Di + G * N + (g + 1) * N]
        x = X[:, h * P:(h + 1) * P]
        dtp = _softplus64(dt[:, h] + np.float64(wl.dt_bias[h]))
        hs = wl.ssm_pool[1, h].astype(np.float64) + np.cumsum(
            dtp[:, None, None] * x[:, :, None] * B[:, None, :], axis=0)
        yr = np.einsum("tpn,tn->tp", hs, C) + np.float64(wl.D[h]) * x
        assert np.max(np.abs(y[:, h * P:(h + 1) * P] - yr) / (1 + np.abs(yr))) < 1e-5
        assert np.max(np.abs(pool[1, h] - hs[-1]) / (1 + np.abs(hs[-1]))) < 1e-5


def test_vanishing_time_step(orc):
    """dt = -40: dt' ~ 1e-17, so the state stays h_0 and y = C.h_0 + D x."""
    wl = _small(20, [12], fresh=[0], slots=[2])
    wl.dt[:] = -40.0
    xa, _ = oracle_conv(wl)
    y, pool = oracle_scan(wl, xa)
    sh = wl.shape
    H, P, N, G = sh.nheads, sh.headdim, sh.d_state, sh.ngroups
    Di = H * P
    X = xa.astype(np.float64)
    for h in range(H):
        g = h // (H // G)
        C = X[:, Di + G * N + g * N:Di + G * N + (g + 1) * N]
        yr = C @ wl.ssm_pool[2, h].astype(np.float64).T + np.float64(wl.D[h]) * X[:, h * P:(h + 1) * P]
        assert np.max(np.abs(y[:, h * P:(h + 1) * P] - yr) / (1 + np.abs(yr))) < 1e-6
    assert np.allclose(pool[2], wl.ssm_pool[2], rtol=1e-6, atol=0)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_conv_equals_numpy_convolve(orc, K):
    """One fresh sequence: bias + numpy.convolve(in, w reversed) truncated to L, then SiLU."""
    sh = W.Shape(**{**SMALL.__dict__, "conv_kernel": K})
    wl = W.random_prefill(21, sh, [37], fresh=[1], slots=[0])
    out, pool = oracle_conv(wl)
    x = wl.xbc.astype(np.float64)
    L = x.shape[0]
    for c in range(sh.conv_dim):
        pre = np.float64(wl.conv_b[c]) + np.convolve(x[:, c], wl.conv_w[c, ::-1].astype(np.float64))[:L]
        ref = _silu64(pre)
        assert np.allclose(out[:, c], ref, rtol=2.4e-7, atol=1e-30)
    assert np.array_equal(pool[0], wl.xbc[L - (K - 1):])


# ------------------------------------------------------------ norm invariants


def _norm_inputs(seed, rows=9, Di=48, act="f32"):
    rng = np.random.default_rng(seed)
    y = W.to_act(rng.standard_normal((rows, Di), dtype=np.float32), act)
    z = W.to_act(rng.standard_normal((rows, Di), dtype=np.float32), act)
    return y, z


def test_norm_unit_weight_mean_square(orc):
    """With w = 1, each group's mean of out^2 equals ms / (ms + eps), ms the mean of g^2."""
    y, z = _norm_inputs(30)
    for R in (1, 2, 4):
        out = np.zeros_like(y)
        eps = 1e-2
        assert oracle.gated_rmsnorm(out, y, z, np.ones(48, np.float32), R, eps) == 0
        g = y.astype(np.float64) * _silu64(z)
        gs = 48 // R
        for q in range(R):
            sl = slice(q * gs, (q + 1) * gs)
            ms = (g[:, sl] ** 2).mean(1)
            got = (out[:, sl].astype(np.float64) ** 2).mean(1)
            assert np.allclose(got, ms / (ms + np.float32(eps)), rtol=1e-6)


def test_norm_scale_invariance(orc):
    """eps = 0: scaling y by 2 leaves out unchanged, bit for bit."""
    y, z = _norm_inputs(31)
    w = np.random.default_rng(3).normal(1, 0.1, 48).astype(np.float32)
    o1, o2 = np.zeros_like(y), np.zeros_like(y)
    assert oracle.gated_rmsnorm(o1, y, z, w, 2, 0.0) == 0
    assert oracle.gated_rmsnorm(o2, (y * 2).astype(np.float32), z, w, 2, 0.0) == 0
    assert np.array_equal(o1, o2)


def test_norm_groups_are_independent_slices(orc):
    """R groups equal R single-group norms on the column slices, bit for bit."""
    y, z = _norm_inputs(32, act="bf16")
    w = np.random.default_rng(4).normal(1, 0.1, 48).astype(np.float32)
    out = np.zeros_like(y)
    assert oracle.gated_rmsnorm(out, y, z, w, 4, 1e-5) == 0
    for q in range(4):
        sl = slice(q * 12, (q + 1) * 12)
        o = np.zeros((y.shape[0], 12), dtype=y.dtype)
        assert oracle.gated_rmsnorm(o, np.ascontiguousarray(y[:, sl]), np.ascontiguousarray(z[:, sl]),
                                    np.ascontiguousarray(w[sl]), 1, 1e-5) == 0
        assert np.array_equal(out[:, sl], o)


def test_norm_matches_formula(orc):
    """rmsnorm(y * silu(z)) * w with w ~ N(1, 0.1): gate before the norm, eps inside the root."""
    y, z = _norm_inputs(33)
    w = np.random.default_rng(5).normal(1, 0.1, 48).astype(np.float32)
    out = np.zeros_like(y)
    eps = np.float32(1e-3)
    assert oracle.gated_rmsnorm(out, y, z, w, 3, eps) == 0
    g = (y.astype(np.float64) * _silu64(z)).reshape(9, 3, 16)
    ref = (g / np.sqrt((g ** 2).mean(-1, keepdims=True) + np.float64(eps))).reshape(9, 48) * w
    assert np.allclose(out, ref, rtol=2.4e-7, atol=1e-30)


# ------------------------------------------------------------ determinism


def test_thread_count_does_not_change_results(orc):
    wl = _small(40, [20, 9, 31], fresh=[0, 1, 0], slots=[5, 0, 2], act="bf16")
    n0 = oracle.max_threads()
    try:
        res = []
        for n in (1, max(2, n0)):
            oracle.set_threads(n)
            xa, cp = oracle_conv(wl)
            y, sp = oracle_scan(wl, xa)
            out = oracle_norm(wl, y)
            res.append((xa, cp, y, sp, out))
        for a, b in zip(*res):
            assert np.array_equal(a, b)
    finally:
        oracle.set_threads(n0)


# ------------------------------------------------------------ snapshots and rollback


def test_snapshot_count_brute_force(orc):
    rng = np.random.default_rng(70)
    for _ in range(50):
        lens = rng.integers(1, 40, rng.integers(0, 6)).tolist()
        E = int(rng.integers(1, 12))
        want = sum(len([b for b in range(1, L) if b % E == 0]) for L in lens)
        assert oracle.snapshot_count(lens, E) == want


def _prefix_states(wl, s, b):
    """Slot states a run of only the first b rows of sequence s leaves (conv, ssm)."""
    r0 = int(np.sum(wl.run_lengths[:s]))
    rows = slice(r0, r0 + b)
    one = dict(run_lengths=[b], slots=[wl.slots[s]], fresh=[wl.fresh[s]])
    xa, cp = oracle_conv(wl, xbc=np.ascontiguousarray(wl.xbc[rows]), **one)
    _, sp = oracle_scan(wl, xa, dt=np.ascontiguousarray(wl.dt[rows]), **one)
    return cp[wl.slots[s]], sp[wl.slots[s]]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("E", [1, 3, 8])
def test_snapshots_equal_prefix_runs(orc, act, E):
    """A snapshot at boundary b equals, bit for bit, the slot state after a run of the first b
    rows of its sequence (conv: including history rows when b < K-1); the outputs and the final
    slots are those of the same call without snapshots."""
    wl = _small(71, [9, 1, 17, 4], fresh=[1, 0, 0, 1], slots=[5, 0, 2, 3], act=act)
    xa, cp, csn = oracle_conv_snap(wl, E)
    y, sp, ssn = oracle_scan_snap(wl, xa, E)
    xa0, cp0 = oracle_conv(wl)
    y0, sp0 = oracle_scan(wl, xa0)
    assert np.array_equal(xa, xa0) and np.array_equal(y, y0)
    assert np.array_equal(cp, cp0) and np.array_equal(sp, sp0)
    idx = 0
    for s, L in enumerate(wl.run_lengths):
        for b in range(E, L, E):
            c_ref, s_ref = _prefix_states(wl, s, b)
            assert np.array_equal(csn[idx], c_ref), (s, b)
            assert np.array_equal(ssn[idx], s_ref), (s, b)
            idx += 1
    assert idx == len(ssn) == len(csn)


@pytest.mark.parametrize("E", [1, 4])
def test_commit_rolls_back_to_accepted_prefix(orc, E):
    """After a verified run, committing accepted[s] = m puts the state of the first m rows in
    the slots when m is a boundary below L; m == L keeps the whole run's state; other values
    (0, beyond L, between boundaries) leave the slots as they are; other slots are untouched."""
    lens = [5, 8, 1, 9, 8]
    wl = _small(72, lens, fresh=[0, 1, 0, 0, 1], slots=[4, 1, 0, 5, 2], act="bf16")
    xa, cp, csn = oracle_conv_snap(wl, E)
    _, sp, ssn = oracle_scan_snap(wl, xa, E)
    accepted = [4, 8, 1, 7 if E == 1 else 6, 0]
    cp_c, sp_c = cp.copy(), sp.copy()
    assert oracle.commit(sp_c, cp_c, ssn, csn, E, accepted, lens, wl.slots) == 0
    for s, (L, m) in enumerate(zip(lens, accepted)):
        sl = wl.slots[s]
        if 1 <= m < L and m % E == 0:
            c_ref, s_ref = _prefix_states(wl, s, m)
        else:
            c_ref, s_ref = cp[sl], sp[sl]
        assert np.array_equal(cp_c[sl], c_ref), s
        assert np.array_equal(sp_c[sl], s_ref), s
    for sl in set(range(wl.shape.pool_slots)) - set(int(v) for v in wl.slots):
        assert np.array_equal(cp_c[sl], wl.conv_pool[sl]) and np.array_equal(sp_c[sl], wl.ssm_pool[sl])


# ------------------------------------------------------------ padded batches


def _mask(lens, Lmax, left):
    m = np.zeros((len(lens), Lmax), dtype=np.uint8)
    for b, L in enumerate(lens):
        if left:
            m[b, Lmax - L:] = 1
        else:
            m[b, :L] = 1
    return m


@pytest.mark.parametrize("left", [0, 1])
def test_padded_runs_match_mask_counts(orc, left):
    """Run lengths are the mask's row sums and the side is where the runs sit (numpy)."""
    rng = np.random.default_rng(90)
    lens = rng.integers(1, 30, 7)
    Lmax = int(lens.max()) + 3
    st, got, side = oracle.padded_runs(_mask(lens, Lmax, left))
    assert st == 0 and np.array_equal(got, lens) and side == left
    full = np.ones((3, 5), dtype=np.uint8)  # no padding: either side, reported as right
    assert oracle.padded_runs(full)[0] == 0


def test_padded_runs_reject_gaps_empty_rows_and_mixed_sides(orc):
    gap = _mask([4, 3], 6, 1)
    gap[0, 3] = 0
    assert oracle.padded_runs(gap)[0] == oracle.INVALID_ARGUMENT
    assert oracle.padded_runs(np.zeros((2, 4), np.uint8))[0] == oracle.INVALID_ARGUMENT
    mixed = np.array([[0, 1, 1], [1, 1, 0]], np.uint8)
    assert oracle.padded_runs(mixed)[0] == oracle.INVALID_ARGUMENT


@pytest.mark.parametrize("left", [0, 1])
def test_pack_unpack_round_trip(orc, left):
    """pack gathers exactly the masked rows in batch order (checked with numpy boolean
    indexing); unpack puts them back and zeroes the padding."""
    rng = np.random.default_rng(91)
    lens = np.array([5, 1, 9, 2], dtype=np.int32)
    Lmax = 11
    m = _mask(lens, Lmax, left).astype(bool)
    src = rng.integers(0, 2 ** 16, (4, Lmax, 6), dtype=np.uint16)
    packed = np.zeros((int(lens.sum()), 6), np.uint16)
    assert oracle.pack_rows(packed, src, lens, left) == 0
    assert np.array_equal(packed, src[m])
    back = np.full_like(src, 7)
    assert oracle.unpack_rows(back, packed, lens, left) == 0
    assert np.array_equal(back, np.where(m[:, :, None], src, 0))


# ------------------------------------------------------------ projections


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_linear_identity_and_rank_one(orc, act):
    """An identity weight returns x exactly; a rank-one product is K a_m b_n (closed form,
    exact in both types for small integers)."""
    rng = np.random.default_rng(96)
    x = W.to_act(rng.standard_normal((5, 16)).astype(np.float32), act)
    eye = W.to_act(np.eye(16, dtype=np.float32), act)
    out = np.zeros_like(x)
    assert oracle.linear(out, x, eye) == 0
    assert np.array_equal(out, x)
    a = rng.integers(-3, 4, 6).astype(np.float32)
    b = rng.integers(-3, 4, 9).astype(np.float32)
    xa = W.to_act(np.repeat(a[:, None], 8, axis=1), act)
    wb = W.to_act(np.repeat(b[:, None], 8, axis=1), act)
    out = np.zeros((6, 9), dtype=xa.dtype)
    assert oracle.linear(out, xa, wb) == 0
    assert np.array_equal(W.act_to_f32(out), 8 * np.outer(a, b))


def test_linear_matches_numpy_matmul(orc):
    """Against numpy's float64 matmul of the same bf16 values, rounded once to bf16 (another
    summation order: equal up to one bf16 rounding flip)."""
    rng = np.random.default_rng(97)
    x = W.to_act(rng.standard_normal((33, 200)).astype(np.float32), "bf16")
    w = W.to_act(rng.standard_normal((24, 200)).astype(np.float32), "bf16")
    out = np.zeros((33, 24), np.uint16)
    assert oracle.linear(out, x, w) == 0
    ref = W.act_to_f32(x).astype(np.float64) @ W.act_to_f32(w).astype(np.float64).T
    want = W.act_to_f32(W.to_act(ref.astype(np.float32), "bf16"))
    got = W.act_to_f32(out)
    assert np.max(np.abs(got - want) / (1 + np.abs(want))) <= 2 ** -8


# ------------------------------------------------------------ conditioning of the chain


def test_scan_output_moves_by_bars_under_one_ulp_input_changes(orc):
    """Why parity is judged op by op on shared inputs.  y sums terms that cancel, so the scan
    amplifies the last-bit differences that two correct implementations of the conv may leave
    in its input.  Here the oracle alone, on the packed variable-length batch: flipping the
    lowest bf16 bit of 5 % of the conv output's elements (a change of one unit in the last
    place, the size of one rounding difference) moves the oracle's own y, and the norm after
    it, by more than the 2e-2 (1 + |ref|) output bar.  An end-to-end comparison of two chains
    can therefore fail although each op of each chain is within its bar."""
    from _util import BF16_BAR, max_bar_fraction

    wl = W.varlen_prefill()
    xa, _ = oracle_conv(wl)
    y0, _ = oracle_scan(wl, xa)
    rng = np.random.default_rng(28)
    flip = rng.random(xa.shape) < 0.05
    xf = xa ^ (flip.astype(np.uint16))
    y1, _ = oracle_scan(wl, xf)
    fy = max_bar_fraction(W.act_to_f32(y1), W.act_to_f32(y0), BF16_BAR)
    o0, o1 = oracle_norm(wl, y0), oracle_norm(wl, y1)
    fo = max_bar_fraction(W.act_to_f32(o1), W.act_to_f32(o0), BF16_BAR)
    print("one-ulp changes in 5%% of the scan input: y moves %.3g bars, the norm output %.3g" % (fy, fo))
    assert fy > 1.0 and fo > 1.0
