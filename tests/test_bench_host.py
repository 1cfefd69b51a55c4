"""Host-side parts of bench.py (no GPU): the one-GPU guard and the algorithmic byte counts the
rooflines divide by, against counts written out from the shapes."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mamba2_selective_scan_causalconv1d_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_long_prefill():
    """4 fresh x 16384 rows, 48 heads x 64, d_state 128, xBC 3328 channels, bf16."""
    wl = W.long_prefill()
    T = 4 * 16384
    # scan: x, B, C, dt in and y out (2 bytes each), plus the final states (no seeds read: fresh)
    scan_bytes, scan_flops = bench.kernel_bytes_flops("ssd_scan", wl, T)
    assert scan_bytes == T * (3328 + 48 + 3072) * 2 + 4 * 48 * 64 * 128 * 4
    assert abs(scan_bytes / 1e6 - 851.44) < 0.01
    # flops per row and head at the workload's chunk Q = 256: C B^T over the causal triangle
    # (shared by the 48 heads of the group), the masked product with x, the chunk state and the
    # state's output term (two flops per multiply-add each): 49,901 per row and head, 157.0 GFLOP
    assert scan_flops == T * 48 * (128 * 257 / 48 + 64 * 257 + 4 * 128 * 64)
    assert abs(scan_flops / 1e9 - 157.0) < 0.05
    alg, dense = bench.scan_flops(wl, T)
    assert alg == scan_flops
    assert abs(dense / (T * 48) - 66901.33) < 0.01
    # conv: rows in and out, plus the slot rows written (fresh: none read)
    conv_bytes, _ = bench.kernel_bytes_flops("conv1d_silu", wl, T)
    assert conv_bytes == 2 * T * 3328 * 2 + 4 * 3 * 3328 * 2
    # norm: y, z in and out, plus the weights
    norm_bytes, _ = bench.kernel_bytes_flops("gated_rmsnorm", wl, T)
    assert norm_bytes == 3 * T * 3072 * 2 + 3072 * 4


def test_algorithmic_bytes_decode_step():
    """256 one-row requests, all resuming: each state read and written once."""
    wl = W.decode_batch(steps=1)
    wl.fresh[:] = 0
    b, _ = bench.kernel_bytes_flops("scan_decode", wl, 256)
    assert b == 256 * (3328 + 48 + 3072) * 2 + 2 * 256 * 48 * 64 * 128 * 4
    assert abs(b / 1e6 - 808.6) < 0.1


def test_digest_sees_every_bit():
    """The digest the bench compares across timed calls changes when any one bit changes, and
    depends on the position of a value, not only on the multiset of values."""
    import numpy as np
    import torch

    t = torch.from_numpy(np.random.default_rng(1).standard_normal(100003).astype(np.float32))
    d0 = bench.digest(torch, [t])
    for i in (0, 5, 100002):
        u = t.clone()
        u.view(torch.int32)[i] ^= 1
        assert bench.digest(torch, [u]) != d0
    s = t.clone()
    s[[3, 4]] = s[[4, 3]]
    assert bench.digest(torch, [s]) != d0
    b = t.to(torch.bfloat16)
    assert bench.digest(torch, [b]) == bench.digest(torch, [b.clone()])


def test_mamba3_flop_count():
    """Per row and head at chunk 64, Q/K width 128, V width 64: q.k over the causal triangle
    128 * 65, the masked product with v 64 * 65, the state's output term and the chunk state
    2 * 128 * 64 each: 45,248 flops."""
    wl = W.mamba3_varlen()
    T, H = wl.num_rows, wl.nheads
    assert bench.mamba3_flops(wl) == T * H * (128 * 65 + 64 * 65 + 4 * 128 * 64)
    assert bench.mamba3_flops(wl) / (T * H) == 45248
