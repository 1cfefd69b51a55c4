"""The path captured in a HIP graph (GPU).

The library allocates nothing, copies nothing and clears nothing with memsets, so a caller may
capture its launches.  Each test captures a few steps into a graph, then replays it several
times with eager work (pool resets, host copies) and synchronisations in between, and checks
every replay against the same steps run eagerly: outputs and pools bit for bit.
"""
import numpy as np
import pytest
import torch

from mamba2_selective_scan_causalconv1d_amd import ops
from mamba2_selective_scan_causalconv1d_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    import _gpu

    return _gpu


def _replays_match(run, outputs, reset, reps=4):
    """run(): the launches; outputs(): host copies to compare; reset(): restore the inputs."""
    reset()
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    want = outputs()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(reps):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert a.tobytes() == b.tobytes(), "replay %d, output %d differs from the eager run" % (rep, i)
    del g


def test_decode_steps_in_a_graph(gpu):
    """Four decode steps (conv step, one-row scan, norm) of 32 requests on the decode pool."""
    wl = W.decode_batch(steps=4, requests=32)
    sh = wl.shape
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    b0 = gpu.batch_of(wl)
    b1 = gpu.batch_of(wl, fresh=np.zeros_like(wl.fresh))
    steps = [tuple(ops.to_device(a) for a in s) for s in wl.steps]
    cp0, sp0 = ops.to_device(wl.conv_pool), ops.to_device(wl.ssm_pool)
    cp, sp = cp0.clone(), sp0.clone()
    R = len(wl.run_lengths)
    xa = torch.empty((R, sh.conv_dim), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((R, sh.d_inner), dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty_like(y) for _ in steps]

    def run():
        for i, (x, z, dt) in enumerate(steps):
            b = b0 if i == 0 else b1
            ops.conv1d(xa, x, p.conv_w, p.conv_b, cp, b, dims)
            ops.scan_decode(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, b, dims)
            ops.gated_rmsnorm(outs[i], y, z, p.norm_w, sh.norm_groups, sh.eps)

    def reset():
        cp.copy_(cp0)
        sp.copy_(sp0)
        for o in outs:
            o.zero_()

    _replays_match(run, lambda: [ops.to_host(t) for t in outs + [cp, sp]], reset)


def test_prefill_step_in_a_graph(gpu):
    """A ragged prefill (runs 300, 1, 700 and 64 rows, two resuming) on the MFMA path, with a
    workspace allocated before capture, then a verify step with snapshots and a commit."""
    sh = W.Shape(nheads=8, headdim=64, d_state=128, ngroups=1, conv_kernel=4, chunk_size=256, norm_groups=2,
                 pool_slots=6, act="bf16")
    wl = W.random_prefill(71, sh, [300, 1, 700, 64], fresh=[1, 0, 1, 0], slots=[4, 0, 2, 5])
    p = gpu.Params(wl)
    dims = gpu.dims_of(sh)
    b = gpu.batch_of(wl)
    d = ops.to_device
    x, z, dt = d(wl.xbc), d(wl.z), d(wl.dt)
    cp0, sp0 = d(wl.conv_pool), d(wl.ssm_pool)
    cp, sp = cp0.clone(), sp0.clone()
    T = wl.num_rows
    xa = torch.empty_like(x)
    y = torch.empty((T, sh.d_inner), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(y)
    ws = torch.empty(max(256, ops.scan_prefill_workspace_bytes(b, dims)), dtype=torch.uint8, device="cuda")
    # a verify step of 3 rows per sequence after the prefill, with per-row snapshots and a commit
    vb = ops.RecurrentBatch([3] * 4, wl.slots, [0] * 4, device="cuda")
    rng = np.random.default_rng(72)
    vx = d(W.to_act(rng.standard_normal((12, sh.conv_dim)).astype(np.float32), "bf16"))
    vdt = d(W.to_act(rng.standard_normal((12, sh.nheads)).astype(np.float32), "bf16"))
    vxa = torch.empty_like(vx)
    vy = torch.empty((12, sh.d_inner), dtype=torch.bfloat16, device="cuda")
    n = ops.snapshot_count(vb, 1)
    csn = torch.empty((n, sh.conv_kernel - 1, sh.conv_dim), dtype=torch.bfloat16, device="cuda")
    ssn = torch.empty((n, sh.nheads, sh.headdim, sh.d_state), dtype=torch.float32, device="cuda")
    accepted = torch.tensor([1, 2, 3, 2], dtype=torch.int32, device="cuda")

    def run():
        ops.conv1d(xa, x, p.conv_w, p.conv_b, cp, b, dims)
        ops.scan_prefill(y, xa, dt, p.a_log, p.dt_bias, p.D, sp, b, dims, workspace=ws)
        ops.gated_rmsnorm(out, y, z, p.norm_w, sh.norm_groups, sh.eps)
        ops.conv1d_snap(vxa, vx, p.conv_w, p.conv_b, cp, csn, 1, vb, dims)
        ops.scan_verify(vy, vxa, vdt, p.a_log, p.dt_bias, p.D, sp, ssn, vb, dims)
        ops.commit_snapshots(sp, cp, ssn, csn, 1, accepted, vb, dims)

    def reset():
        cp.copy_(cp0)
        sp.copy_(sp0)
        for t in (xa, y, out, vxa, vy):
            t.zero_()

    _replays_match(run, lambda: [ops.to_host(t) for t in (xa, y, out, vxa, vy, cp, sp)], reset)
