"""The projections around the path (mamba2_linear) against the oracle (GPU).

dst = x . w^T in bf16 with fp32 accumulation against the oracle's double sum rounded once:
element by element within the bf16 bar 2e-2 (1 + |ref|), on ragged shapes for both tilings
(M, N not multiples of the 128 x 128 or 256 x 256 tile, K a multiple of 64 or not; narrow
outputs of 8 to 64 columns over long K) and, at
the long-prefill layer's in_proj and out_proj shapes (65536 rows, model width 1536), on
sampled rows.  The layer case
runs in_proj (three calls on row slices of one weight) -> conv -> scan -> norm -> out_proj,
each op against the oracle on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba2_selective_scan_causalconv1d_amd import workloads as W
from _util import BF16_BAR, assert_close, oracle_conv, oracle_norm, oracle_scan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    import _gpu

    return _gpu


def _bf16(rng, shape, scale=1.0):
    return W.to_act((rng.standard_normal(shape) * scale).astype(np.float32), "bf16")


@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (37, 48, 64), (130, 136, 200), (257, 264, 72), (128, 128, 1536),
                                   (300, 3328, 96), (300, 264, 128), (257, 520, 64), (1000, 3328, 1536),
                                   (512, 256, 3072), (37, 48, 1536), (1000, 64, 256), (1, 8, 128),
                                   (130, 24, 384), (4099, 56, 640)])
def test_linear_ragged_shapes(gpu, M, N, K):
    ops = gpu.ops
    rng = np.random.default_rng(100 + M)
    x, w = _bf16(rng, (M, K)), _bf16(rng, (N, K), K ** -0.5)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.linear(out, ops.to_device(x), ops.to_device(w))
    torch.cuda.synchronize()
    want = np.zeros((M, N), np.uint16)
    assert oracle.linear(want, x, w) == 0
    assert_close(gpu.f32(ops.to_host(out)), gpu.f32(want), BF16_BAR, "linear %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("seed", range(6))
def test_linear_random_shapes(gpu, seed):
    """Seeded random shapes across both tilings: M in [1, 700], N in [8, 800] and K in [8, 640]
    (multiples of 8), every third case with K a multiple of 64 and M, N >= 256."""
    ops = gpu.ops
    rng = np.random.default_rng(500 + seed)
    if seed % 3 == 0:
        M, N, K = int(rng.integers(256, 701)), 8 * int(rng.integers(32, 101)), 64 * int(rng.integers(1, 11))
    else:
        M, N, K = int(rng.integers(1, 701)), 8 * int(rng.integers(1, 101)), 8 * int(rng.integers(1, 81))
    x, w = _bf16(rng, (M, K)), _bf16(rng, (N, K), K ** -0.5)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.linear(out, ops.to_device(x), ops.to_device(w))
    torch.cuda.synchronize()
    want = np.zeros((M, N), np.uint16)
    assert oracle.linear(want, x, w) == 0
    assert_close(gpu.f32(ops.to_host(out)), gpu.f32(want), BF16_BAR, "linear %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("N,K", [(3328, 1536), (3072, 1536), (48, 1536), (1536, 3072)])
def test_linear_layer_shapes_sampled(gpu, N, K):
    """65536 rows (the long-prefill batch); 96 rows sampled, incl. the first and last."""
    ops = gpu.ops
    rng = np.random.default_rng(N + K)
    M = 65536
    x, w = _bf16(rng, (M, K)), _bf16(rng, (N, K), K ** -0.5)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops.linear(out, ops.to_device(x), ops.to_device(w))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 94)]))
    want = np.zeros((len(rows), N), np.uint16)
    assert oracle.linear(want, np.ascontiguousarray(x[rows]), w) == 0
    got = ops.to_host(out)[rows]
    assert_close(gpu.f32(got), gpu.f32(want), BF16_BAR, "linear rows")


def test_mixer_layer(gpu):
    """in_proj -> conv -> scan -> norm -> out_proj on a ragged batch (runs 150, 1, 300, one
    resuming), model width 256, 8 heads x 64, d_state 128: each op against the oracle."""
    ops = gpu.ops
    sh = W.Shape(nheads=8, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=256, norm_groups=2,
                 pool_slots=4, act="bf16")
    d_model = 256
    wl = W.random_prefill(101, sh, [150, 1, 300], fresh=[1, 1, 0], slots=[2, 0, 3])
    rng = np.random.default_rng(102)
    T = wl.num_rows
    hidden = _bf16(rng, (T, d_model))
    nproj = sh.d_inner + sh.conv_dim + sh.nheads
    w_in = _bf16(rng, (nproj, d_model), d_model ** -0.5)
    w_out = _bf16(rng, (d_model, sh.d_inner), sh.d_inner ** -0.5)
    d = ops.to_device
    hid, win, wout = d(hidden), d(w_in), d(w_out)
    z = torch.empty((T, sh.d_inner), dtype=torch.bfloat16, device="cuda")
    xbc = torch.empty((T, sh.conv_dim), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((T, sh.nheads), dtype=torch.bfloat16, device="cuda")
    Di, Dc = sh.d_inner, sh.conv_dim
    ops.linear(z, hid, win[:Di])
    ops.linear(xbc, hid, win[Di:Di + Dc])
    ops.linear(dt, hid, win[Di + Dc:])
    torch.cuda.synchronize()
    parts = [ops.to_host(t) for t in (z, xbc, dt)]
    full = np.zeros((T, nproj), np.uint16)
    assert oracle.linear(full, hidden, w_in) == 0
    for got, lo, hi, name in zip(parts, (0, Di, Di + Dc), (Di, Di + Dc, nproj), ("z", "xbc", "dt")):
        assert_close(gpu.f32(got), gpu.f32(full[:, lo:hi]), BF16_BAR, "in_proj " + name)
    # the path on the GPU's projections, each op against the oracle on the same inputs
    wl.z, wl.xbc, wl.dt = parts
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    cp, sp = d(wl.conv_pool), d(wl.ssm_pool)
    xa = torch.empty_like(xbc)
    ops.conv1d(xa, xbc, p.conv_w, p.conv_b, cp, b, dims)
    y = torch.empty_like(z)
    ops.scan_prefill(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, b, dims)
    nrm = torch.empty_like(z)
    ops.gated_rmsnorm(nrm, y, z, p.norm_w, sh.norm_groups, sh.eps)
    out = torch.empty((T, d_model), dtype=torch.bfloat16, device="cuda")
    ops.linear(out, nrm, wout)
    torch.cuda.synchronize()
    xa_h, y_h, n_h = ops.to_host(xa), ops.to_host(y), ops.to_host(nrm)
    assert_close(gpu.f32(xa_h), gpu.f32(oracle_conv(wl)[0]), BF16_BAR, "conv")
    assert_close(gpu.f32(y_h), gpu.f32(oracle_scan(wl, xa_h)[0]), BF16_BAR, "scan")
    assert_close(gpu.f32(n_h), gpu.f32(oracle_norm(wl, y_h)), BF16_BAR, "norm")
    want = np.zeros((T, d_model), np.uint16)
    assert oracle.linear(want, n_h, w_out) == 0
    assert_close(gpu.f32(ops.to_host(out)), gpu.f32(want), BF16_BAR, "out_proj")
