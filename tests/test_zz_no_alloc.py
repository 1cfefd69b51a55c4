"""mamba2_scan_prefill_static (no workspace, no allocation: the library's own fixed scratch)
against mamba2_scan_prefill through the C ABI, on two calls in a row, the second on a smaller
batch: y within the bf16 output bar and every named slot within the fp32 state bar, other
slots untouched.  The first batch (4 x 16384 rows, 48 heads) needs longer segments than the
usual ones to fit the scratch; the second (the packed varlen batch, resumed slots) fits at a
length of its own.  A batch too large for the scratch is refused before any launch."""
import numpy as np
import pytest
import torch

from mamba2_selective_scan_causalconv1d_amd import workloads as W
from _util import BF16_BAR, F32_BAR, assert_close

pytestmark = pytest.mark.gpu


def _both(gpu, wl, xa):
    ops = gpu.ops
    p = gpu.Params(wl)
    sh = wl.shape
    dims = gpu.dims_of(sh)
    b = gpu.batch_of(wl)
    x, dt = ops.to_device(xa), ops.to_device(wl.dt)
    res = []
    for static in (False, True):
        pool = ops.to_device(wl.ssm_pool)
        y = torch.empty((x.shape[0], sh.d_inner), dtype=x.dtype, device="cuda")
        if static:
            ops.scan_prefill_static(y, x, dt, p.a_log, p.dt_bias, p.D, pool, b, dims)
        else:
            ops.scan_prefill(y, x, dt, p.a_log, p.dt_bias, p.D, pool, b, dims)
        torch.cuda.synchronize()
        res.append((ops.to_host(y), ops.to_host(pool)))
    (y_r, p_r), (y_s, p_s) = res
    fy = assert_close(W.act_to_f32(y_s), W.act_to_f32(y_r), BF16_BAR, wl.name + " y")
    named = set(int(s) for s in wl.slots)
    fs = 0.0
    for s in range(sh.pool_slots):
        if s in named:
            fs = max(fs, assert_close(p_s[s], p_r[s], F32_BAR, "slot %d" % s))
        else:
            assert p_s[s].tobytes() == wl.ssm_pool[s].tobytes(), "untouched slot %d" % s
    print("  [%s] static vs workspace entry: y %.3g of bar, states %.3g, bit-identical y: %s"
          % (wl.name, fy, fs, np.array_equal(y_s, y_r)), flush=True)


def test_static_scratch_matches_workspace_entry():
    assert torch.cuda.is_available()
    import _gpu

    from _util import oracle_conv

    big = W.long_prefill()
    xa_big, _ = oracle_conv(big)
    _both(_gpu, big, xa_big)
    small = W.varlen_prefill()
    xa_small, _ = oracle_conv(small)
    _both(_gpu, small, xa_small)


def test_static_scratch_refuses_oversized_batches():
    """The fp32 path keeps its 64-row segments: 8 sequences of 40000 rows need more segment
    states than the scratch holds, so the call is refused and writes nothing."""
    assert torch.cuda.is_available()
    import _gpu
    from mamba2_selective_scan_causalconv1d_amd import _lib

    ops = _gpu.ops
    sh = W.Shape(nheads=8, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=64, norm_groups=1,
                 pool_slots=8, act="f32")
    dims = _gpu.dims_of(sh)
    b = ops.RecurrentBatch([40000] * 8, list(range(8)), [1] * 8)
    # the call is refused by its host checks, which read no device data: small stand-ins
    x = torch.zeros((4, sh.conv_dim), dtype=torch.float32, device="cuda")
    dt = torch.zeros((4, sh.nheads), dtype=torch.float32, device="cuda")
    y = torch.full((4, sh.d_inner), 3.0, dtype=torch.float32, device="cuda")
    pool = torch.full((8, sh.nheads, sh.headdim, sh.d_state), 5.0, dtype=torch.float32, device="cuda")
    pv = torch.zeros(sh.nheads, dtype=torch.float32, device="cuda")
    with pytest.raises(ops.Mamba2Error) as e:
        ops.scan_prefill_static(y, x, dt, pv, pv, pv, pool, b, dims)
    assert e.value.status == _lib.WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert (y == 3).all() and (pool == 5).all()
