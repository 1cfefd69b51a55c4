"""Python face of the C ABI (``include/mamba2.h``), same names, on torch device tensors.

Argument marshalling only: every step runs in the HIP kernels of ``libmamba2.so``.
Importing this module loads the library and raises if it is missing (there is no CPU
fallback).  Tensors are torch tensors on the GPU: activations ``torch.float32`` or
``torch.bfloat16``; SSM state, weights and per-head parameters ``torch.float32``.
Each call enqueues on the current torch stream (or ``stream``) and returns at once.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import Dims, KernelTime, Mamba2Error, Mamba3Dims, Mamba3VarlenC, RecurrentBatchC  # noqa: F401

LIB = _lib.load()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def act_dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    if t.dtype == torch.float32:
        return _lib.DTYPE_F32
    raise TypeError("activations are float32 or bfloat16, got %s" % t.dtype)


def make_dims(nheads, headdim, d_state, ngroups, conv_kernel, chunk_size, pool_slots, act) -> Dims:
    code = act if isinstance(act, int) else {"f32": 0, "bf16": 1}[act]
    return Dims(nheads, headdim, d_state, ngroups, conv_kernel, chunk_size, pool_slots, code)


class RecurrentBatch:
    """Per-sequence run lengths, slots and fresh flags, with the device copies the
    kernels read (``cu_seqlens`` is the exclusive prefix sum of the run lengths)."""

    def __init__(self, run_lengths: Sequence[int], slots: Sequence[int], fresh: Sequence[int],
                 device="cuda"):
        self.run_lengths = np.ascontiguousarray(run_lengths, dtype=np.int32)
        self.slots = np.ascontiguousarray(slots, dtype=np.int32)
        self.fresh = np.ascontiguousarray(fresh, dtype=np.uint8)
        n = len(self.run_lengths)
        if len(self.slots) != n or len(self.fresh) != n:
            raise ValueError("run_lengths, slots and fresh must have one entry per sequence")
        cu = np.zeros(n + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.run_lengths, dtype=np.int64).astype(np.int32)
        self.num_rows = int(self.run_lengths.astype(np.int64).sum())
        if device is not None:
            self.dev_cu = torch.from_numpy(cu).to(device)
            self.dev_slots = torch.from_numpy(self.slots.copy()).to(device)
            self.dev_fresh = torch.from_numpy(self.fresh.copy()).to(device)
            dptr = [self.dev_cu.data_ptr(), self.dev_slots.data_ptr(), self.dev_fresh.data_ptr()]
        else:  # host-only batch: validation without a device
            dptr = [1, 1, 1] if n > 0 else [0, 0, 0]
        self.c = RecurrentBatchC(n, self.num_rows, self.run_lengths.ctypes.data, self.slots.ctypes.data,
                                 self.fresh.ctypes.data, *dptr)

    @property
    def num_seqs(self) -> int:
        return len(self.run_lengths)

    def ref(self):
        return ctypes.byref(self.c)


def validate(batch: RecurrentBatch, dims: Dims, decode: bool = False) -> int:
    return LIB.mamba2_validate(batch.ref(), ctypes.byref(dims), 1 if decode else 0)


def conv1d(dst, x, weight, bias, conv_state, batch: RecurrentBatch, dims: Dims, stream=None):
    st = LIB.mamba2_conv1d(_ptr(dst), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), batch.ref(),
                           ctypes.byref(dims), _stream(stream))
    _lib.check(st, "mamba2_conv1d")


def scan_prefill_workspace_bytes(batch: RecurrentBatch, dims: Dims) -> int:
    return int(LIB.mamba2_scan_prefill_workspace_bytes(batch.ref(), ctypes.byref(dims)))


def scan_prefill(dst, xbc, dt, a_log, dt_bias, D, ssm_state, batch: RecurrentBatch, dims: Dims,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    if workspace is None:
        nbytes = scan_prefill_workspace_bytes(batch, dims)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=xbc.device)
    st = LIB.mamba2_scan_prefill(_ptr(dst), _ptr(xbc), _ptr(dt), _ptr(a_log), _ptr(dt_bias), _ptr(D),
                                 _ptr(ssm_state), batch.ref(), ctypes.byref(dims), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check(st, "mamba2_scan_prefill")
    return workspace


def scan_prefill_static(dst, xbc, dt, a_log, dt_bias, D, ssm_state, batch: RecurrentBatch, dims: Dims,
                        stream=None):
    """scan_prefill with the library's own fixed scratch: no workspace, no allocation."""
    st = LIB.mamba2_scan_prefill_static(_ptr(dst), _ptr(xbc), _ptr(dt), _ptr(a_log), _ptr(dt_bias), _ptr(D),
                                        _ptr(ssm_state), batch.ref(), ctypes.byref(dims), _stream(stream))
    _lib.check(st, "mamba2_scan_prefill_static")


def scan_decode(dst, xbc, dt, a_log, dt_bias, D, ssm_state, batch: RecurrentBatch, dims: Dims,
                stream=None):
    st = LIB.mamba2_scan_decode(_ptr(dst), _ptr(xbc), _ptr(dt), _ptr(a_log), _ptr(dt_bias), _ptr(D),
                                _ptr(ssm_state), batch.ref(), ctypes.byref(dims), _stream(stream))
    _lib.check(st, "mamba2_scan_decode")


def gated_rmsnorm(dst, x, z, weight, groups: int, eps: float, stream=None):
    rows, d_inner = x.shape
    st = LIB.mamba2_gated_rmsnorm(_ptr(dst), _ptr(x), _ptr(z), _ptr(weight), int(groups), float(eps),
                                  int(rows), int(d_inner), act_dtype_code(x), _stream(stream))
    _lib.check(st, "mamba2_gated_rmsnorm")


def snapshot_count(batch: RecurrentBatch, snap_every: int) -> int:
    return int(LIB.mamba2_snapshot_count(batch.ref(), int(snap_every)))


def conv1d_snap(dst, x, weight, bias, conv_state, conv_snaps, snap_every: int, batch: RecurrentBatch,
                dims: Dims, stream=None):
    st = LIB.mamba2_conv1d_snap(_ptr(dst), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state), _ptr(conv_snaps),
                                int(snap_every), batch.ref(), ctypes.byref(dims), _stream(stream))
    _lib.check(st, "mamba2_conv1d_snap")


def scan_prefill_snap_workspace_bytes(batch: RecurrentBatch, dims: Dims, snap_every: int) -> int:
    return int(LIB.mamba2_scan_prefill_snap_workspace_bytes(batch.ref(), ctypes.byref(dims), int(snap_every)))


def scan_prefill_snap(dst, xbc, dt, a_log, dt_bias, D, ssm_state, ssm_snaps, snap_every: int,
                      batch: RecurrentBatch, dims: Dims, workspace: Optional[torch.Tensor] = None, stream=None):
    if workspace is None:
        nbytes = scan_prefill_snap_workspace_bytes(batch, dims, snap_every)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=xbc.device)
    st = LIB.mamba2_scan_prefill_snap(_ptr(dst), _ptr(xbc), _ptr(dt), _ptr(a_log), _ptr(dt_bias), _ptr(D),
                                      _ptr(ssm_state), _ptr(ssm_snaps), int(snap_every), batch.ref(),
                                      ctypes.byref(dims), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check(st, "mamba2_scan_prefill_snap")
    return workspace


def scan_verify(dst, xbc, dt, a_log, dt_bias, D, ssm_state, ssm_snaps, batch: RecurrentBatch, dims: Dims,
                stream=None):
    st = LIB.mamba2_scan_verify(_ptr(dst), _ptr(xbc), _ptr(dt), _ptr(a_log), _ptr(dt_bias), _ptr(D),
                                _ptr(ssm_state), _ptr(ssm_snaps), batch.ref(), ctypes.byref(dims), _stream(stream))
    _lib.check(st, "mamba2_scan_verify")


def commit_snapshots(ssm_state, conv_state, ssm_snaps, conv_snaps, snap_every: int, accepted,
                     batch: RecurrentBatch, dims: Dims, stream=None):
    st = LIB.mamba2_commit_snapshots(_ptr(ssm_state), _ptr(conv_state), _ptr(ssm_snaps), _ptr(conv_snaps),
                                     int(snap_every), _ptr(accepted), batch.ref(), ctypes.byref(dims),
                                     _stream(stream))
    _lib.check(st, "mamba2_commit_snapshots")


def linear(dst, x, weight, stream=None):
    """dst [rows, out] = x [rows, in] . weight [out, in]^T (weight may be a row slice)."""
    rows, k = x.shape
    n = weight.shape[0]
    st = LIB.mamba2_linear(_ptr(dst), _ptr(x), _ptr(weight), int(rows), int(n), int(k), act_dtype_code(x),
                           _stream(stream))
    _lib.check(st, "mamba2_linear")


def padded_runs(mask: np.ndarray):
    """(run lengths [B] int32, left_padded) of a host mask [B, Lmax] (nonzero = a real row)."""
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    B, Lmax = m.shape
    lens = np.zeros(B, dtype=np.int32)
    left = np.zeros(1, dtype=np.int32)
    st = LIB.mamba2_padded_runs(m.ctypes.data, B, Lmax, lens.ctypes.data, left.ctypes.data)
    _lib.check(st, "mamba2_padded_runs")
    return lens, int(left[0])


def pack_rows(dst, src, left_padded: int, batch: RecurrentBatch, stream=None):
    """dst [T, ...] <- the real rows of src [B, Lmax, ...]."""
    row_bytes = src[0, 0].numel() * src.element_size()
    st = LIB.mamba2_pack_rows(_ptr(dst), _ptr(src), row_bytes, int(src.shape[1]), int(left_padded), batch.ref(),
                              _stream(stream))
    _lib.check(st, "mamba2_pack_rows")


def unpack_rows(dst, src, left_padded: int, batch: RecurrentBatch, stream=None):
    """dst [B, Lmax, ...] <- packed rows at their padded positions, zeros on padding."""
    row_bytes = dst[0, 0].numel() * dst.element_size()
    st = LIB.mamba2_unpack_rows(_ptr(dst), _ptr(src), row_bytes, int(dst.shape[1]), int(left_padded), batch.ref(),
                                _stream(stream))
    _lib.check(st, "mamba2_unpack_rows")


def ssm_slot_bytes(dims: Dims) -> int:
    return int(LIB.mamba2_ssm_slot_bytes(ctypes.byref(dims)))


def conv_slot_bytes(dims: Dims) -> int:
    return int(LIB.mamba2_conv_slot_bytes(ctypes.byref(dims)))


def timing_enable(capacity: int = 4096) -> None:
    _lib.check(LIB.mamba2_timing_enable(int(capacity)), "mamba2_timing_enable")


def timing_collect(max_records: int = 4096):
    """[(kernel name, ms)] for every kernel launched since the last collect."""
    buf = (KernelTime * max_records)()
    n = LIB.mamba2_timing_collect(buf, max_records)
    if n < 0:
        raise Mamba2Error(_lib.HIP_ERROR, "mamba2_timing_collect")
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]


# ------------------------------------------------------------------ Mamba-3 SISO forward


class Mamba3Batch:
    """Packed sequences of the Mamba-3 forward: host run lengths and the device cu_seqlens."""

    def __init__(self, run_lengths: Sequence[int], device="cuda"):
        self.run_lengths = np.ascontiguousarray(run_lengths, dtype=np.int32)
        n = len(self.run_lengths)
        cu = np.zeros(n + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.run_lengths, dtype=np.int64).astype(np.int32)
        self.num_rows = int(self.run_lengths.astype(np.int64).sum())
        self.dev_cu = torch.from_numpy(cu).to(device) if device is not None else None
        dptr = self.dev_cu.data_ptr() if self.dev_cu is not None else (1 if n > 0 else 0)
        self.c = Mamba3VarlenC(n, self.num_rows, self.run_lengths.ctypes.data, dptr)

    @property
    def num_seqs(self) -> int:
        return len(self.run_lengths)

    def ref(self):
        return ctypes.byref(self.c)


def mamba3_dims(nheads, qk_dim, v_dim, nangles) -> Mamba3Dims:
    return Mamba3Dims(nheads, qk_dim, v_dim, nangles)


def mamba3_workspace_bytes(batch: Mamba3Batch, dims: Mamba3Dims) -> int:
    return int(LIB.mamba3_siso_forward_workspace_bytes(batch.ref(), ctypes.byref(dims)))


def mamba3_siso_forward(out, final_angle, final_ssm, final_k, final_v, q, k, v, adt, dt, trap, q_bias, k_bias,
                        angles, d, z, batch: Mamba3Batch, dims: Mamba3Dims, workspace: Optional[torch.Tensor] = None,
                        stream=None):
    if workspace is None:
        workspace = torch.empty(max(mamba3_workspace_bytes(batch, dims), 256), dtype=torch.uint8, device=q.device)
    fa = _ptr(final_angle) if final_angle is not None and final_angle.numel() > 0 else None
    st = LIB.mamba3_siso_forward(_ptr(out), fa, _ptr(final_ssm), _ptr(final_k), _ptr(final_v), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(adt), _ptr(dt), _ptr(trap), _ptr(q_bias), _ptr(k_bias),
                                 _ptr(angles) if angles is not None and angles.numel() > 0 else None, _ptr(d), _ptr(z),
                                 batch.ref(), ctypes.byref(dims), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _lib.check(st, "mamba3_siso_forward")
    return workspace


# ------------------------------------------------------------------ host <-> device helpers


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Canonical host array (float32, or uint16 bf16 bits) -> device tensor, bits unchanged."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> canonical host array (float32, or uint16 bf16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
