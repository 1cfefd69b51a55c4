"""Run the HIP path (through the C ABI) on a workload; host arrays in, host arrays out."""
from __future__ import annotations

import numpy as np
import torch

from mamba2_selective_scan_causalconv1d_amd import ops
from mamba2_selective_scan_causalconv1d_amd import workloads as W

DEV = "cuda"


def dims_of(sh: W.Shape) -> ops.Dims:
    return ops.make_dims(sh.nheads, sh.headdim, sh.d_state, sh.ngroups, sh.conv_kernel, sh.chunk_size,
                         sh.pool_slots, sh.act)


def batch_of(wl: W.Workload, run_lengths=None, slots=None, fresh=None) -> ops.RecurrentBatch:
    return ops.RecurrentBatch(wl.run_lengths if run_lengths is None else run_lengths,
                              wl.slots if slots is None else slots,
                              wl.fresh if fresh is None else fresh, device=DEV)


class Params:
    """Per-layer parameters of a workload on the device."""

    def __init__(self, wl: W.Workload):
        d = ops.to_device
        self.conv_w, self.conv_b = d(wl.conv_w), d(wl.conv_b)
        self.a_log, self.dt_bias, self.D = d(wl.a_log), d(wl.dt_bias), d(wl.D)
        self.norm_w = d(wl.norm_w)


def gpu_conv(wl, xbc, conv_pool, batch, p=None):
    p = p or Params(wl)
    x = ops.to_device(xbc)
    pool = ops.to_device(conv_pool)
    out = torch.empty_like(x)
    ops.conv1d(out, x, p.conv_w, p.conv_b, pool, batch, dims_of(wl.shape))
    torch.cuda.synchronize()
    return ops.to_host(out), ops.to_host(pool)


def gpu_scan(wl, xa, dt, ssm_pool, batch, p=None, decode=False):
    p = p or Params(wl)
    sh = wl.shape
    x = ops.to_device(xa)
    dtd = ops.to_device(dt)
    pool = ops.to_device(ssm_pool)
    y = torch.empty((x.shape[0], sh.d_inner), dtype=x.dtype, device=DEV)
    if decode:
        ops.scan_decode(y, x, dtd, p.a_log, p.dt_bias, p.D, pool, batch, dims_of(sh))
    else:
        ops.scan_prefill(y, x, dtd, p.a_log, p.dt_bias, p.D, pool, batch, dims_of(sh))
    torch.cuda.synchronize()
    return ops.to_host(y), ops.to_host(pool)


def gpu_norm(wl, y, z, weight=None, groups=None):
    sh = wl.shape
    yd, zd = ops.to_device(y), ops.to_device(z)
    w = ops.to_device(wl.norm_w if weight is None else weight)
    out = torch.empty_like(yd)
    ops.gated_rmsnorm(out, yd, zd, w, sh.norm_groups if groups is None else groups, sh.eps)
    torch.cuda.synchronize()
    return ops.to_host(out)


def f32(a):
    return W.act_to_f32(a)
