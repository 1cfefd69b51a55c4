"""The padded-batch front end through the C ABI against the oracle (GPU).

"Granite Mamba2 Inference Optimization": the layer takes hidden states [B, Lmax] with an
attention mask and must match across variable-length padded batches.  Pack and unpack are
byte copies: bit-exact against the oracle's.  The end-to-end case runs a left-padded batch
(fresh and resumed rows) through pack -> conv -> scan -> norm -> unpack and checks each op
against the oracle on the same inputs, and the padding rows of the output for zeros.
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


def _mask(lens, Lmax, left):
    m = np.zeros((len(lens), Lmax), dtype=np.uint8)
    for b, L in enumerate(lens):
        if left:
            m[b, Lmax - L:] = 1
        else:
            m[b, :L] = 1
    return m


@pytest.mark.parametrize("left", [0, 1])
@pytest.mark.parametrize("row,dtype", [((3328,), np.uint16), ((48,), np.uint16), ((3,), np.uint16),
                                       ((5, 4), np.float32), ((7,), np.uint8)])
def test_pack_unpack_bit_exact(gpu, left, row, dtype):
    ops = gpu.ops
    rng = np.random.default_rng(93)
    lens = np.array([37, 1, 200, 64, 5], dtype=np.int32)
    Lmax = 211
    got_lens, got_left = ops.padded_runs(_mask(lens, Lmax, left))
    assert np.array_equal(got_lens, lens) and got_left == left
    b = ops.RecurrentBatch(lens, list(range(5)), [1] * 5)
    if dtype == np.float32:
        src = rng.standard_normal((5, Lmax) + row).astype(np.float32)
        tsrc = torch.from_numpy(src).cuda()
    else:
        src = rng.integers(0, np.iinfo(dtype).max, (5, Lmax) + row, dtype=dtype)
        tsrc = torch.from_numpy(src.view(np.int16) if dtype == np.uint16 else src).cuda()
    packed = torch.empty((int(lens.sum()),) + row, dtype=tsrc.dtype, device="cuda")
    ops.pack_rows(packed, tsrc, left, b)
    back = torch.full_like(tsrc, 3)
    ops.unpack_rows(back, packed, left, b)
    torch.cuda.synchronize()
    want_p = np.zeros((int(lens.sum()),) + row, dtype=dtype)
    assert oracle.pack_rows(want_p, src, lens, left) == 0
    want_u = np.zeros_like(src)
    assert oracle.unpack_rows(want_u, want_p, lens, left) == 0
    gp, gu = packed.cpu().numpy(), back.cpu().numpy()
    if dtype == np.uint16:
        gp, gu = gp.view(np.uint16), gu.view(np.uint16)
    assert np.array_equal(gp, want_p) and np.array_equal(gu, want_u)


def test_padded_batch_through_the_path(gpu):
    """A left-padded batch of 5 rows (runs of 1..300, two without previous state) through
    pack -> conv -> scan -> norm -> unpack; every op against the oracle on the same inputs."""
    ops = gpu.ops
    sh = W.Shape(nheads=48, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=256, norm_groups=8,
                 pool_slots=8, act="bf16")
    lens = [300, 1, 77, 129, 256]
    Lmax = 300
    has_prev = [1, 0, 1, 1, 0]
    wl = W.random_prefill(94, sh, lens, fresh=[1 - h for h in has_prev], slots=[6, 1, 3, 0, 5])
    got_lens, left = ops.padded_runs(_mask(lens, Lmax, 1))
    assert left == 1 and list(got_lens) == lens
    # the padded inputs: the workload's packed rows placed at the end of each batch row, junk elsewhere
    rng = np.random.default_rng(95)

    def padded(a):
        out = rng.integers(0, 2 ** 16, (5, Lmax) + a.shape[1:], dtype=np.uint16)
        r = 0
        for i, L in enumerate(lens):
            out[i, Lmax - L:] = a[r:r + L]
            r += L
        return out

    d = ops.to_device
    xp, zp, dtp = d(padded(wl.xbc)), d(padded(wl.z)), d(padded(wl.dt))
    b = gpu.batch_of(wl)
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    T = wl.num_rows
    x = torch.empty((T, sh.conv_dim), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((T, sh.d_inner), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((T, sh.nheads), dtype=torch.bfloat16, device="cuda")
    for dst, src in ((x, xp), (z, zp), (dt, dtp)):
        ops.pack_rows(dst, src, left, b)
    torch.cuda.synchronize()
    assert np.array_equal(ops.to_host(x), wl.xbc) and np.array_equal(ops.to_host(dt), wl.dt)
    cp, sp = d(wl.conv_pool), d(wl.ssm_pool)
    xa = torch.empty_like(x)
    ops.conv1d(xa, x, p.conv_w, p.conv_b, cp, b, dims)
    y = torch.empty_like(z)
    ops.scan_prefill(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, b, dims)
    out = torch.empty_like(z)
    ops.gated_rmsnorm(out, y, z, p.norm_w, sh.norm_groups, sh.eps)
    outp = torch.full((5, Lmax, sh.d_inner), 1.0, dtype=torch.bfloat16, device="cuda")
    ops.unpack_rows(outp, out, left, b)
    torch.cuda.synchronize()
    xa_h, y_h, out_h = ops.to_host(xa), ops.to_host(y), ops.to_host(out)
    xa_o, _ = oracle_conv(wl)
    assert_close(gpu.f32(xa_h), gpu.f32(xa_o), BF16_BAR, "conv")
    y_o, _ = oracle_scan(wl, xa_h)
    assert_close(gpu.f32(y_h), gpu.f32(y_o), BF16_BAR, "scan")
    assert_close(gpu.f32(out_h), gpu.f32(oracle_norm(wl, y_h)), BF16_BAR, "norm")
    want = np.zeros((5, Lmax, sh.d_inner), np.uint16)
    assert oracle.unpack_rows(want, out_h, np.array(lens, np.int32), left) == 0
    assert np.array_equal(ops.to_host(outp), want)
