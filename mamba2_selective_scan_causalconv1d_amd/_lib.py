"""ctypes declarations of the C ABI in ``include/mamba2.h`` (marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmamba2.so")

OK = 0
INVALID_ARGUMENT = 1
SLOT_OUT_OF_RANGE = 2
SLOT_SHARED = 3
RUN_LENGTHS = 4
WORKSPACE_TOO_SMALL = 5
NOT_IMPLEMENTED = 6
HIP_ERROR = 7

DTYPE_F32 = 0
DTYPE_BF16 = 1


class Dims(ctypes.Structure):
    _fields_ = [("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("conv_kernel", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("pool_slots", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32)]


class RecurrentBatchC(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("run_lengths", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("fresh", ctypes.c_void_p), ("dev_cu_seqlens", ctypes.c_void_p),
                ("dev_slots", ctypes.c_void_p), ("dev_fresh", ctypes.c_void_p)]


class Mamba3Dims(ctypes.Structure):
    _fields_ = [("nheads", ctypes.c_int32), ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32),
                ("nangles", ctypes.c_int32)]


class Mamba3VarlenC(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32), ("run_lengths", ctypes.c_void_p),
                ("dev_cu_seqlens", ctypes.c_void_p)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", ctypes.c_float)]


# (name, restype, argtypes) for every function the header declares
_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_pb, _pd = ctypes.POINTER(RecurrentBatchC), ctypes.POINTER(Dims)
_p3b, _p3d = ctypes.POINTER(Mamba3VarlenC), ctypes.POINTER(Mamba3Dims)
SIGNATURES = [
    ("mamba2_conv1d", _i32, [_vp, _vp, _vp, _vp, _vp, _pb, _pd, _vp]),
    ("mamba2_scan_prefill", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _pb, _pd, _vp, _sz, _vp]),
    ("mamba2_scan_prefill_workspace_bytes", _sz, [_pb, _pd]),
    ("mamba2_scan_prefill_static", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _pb, _pd, _vp]),
    ("mamba2_scan_decode", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _pb, _pd, _vp]),
    ("mamba2_gated_rmsnorm", _i32, [_vp, _vp, _vp, _vp, _i32, _f32, _i32, _i32, _i32, _vp]),
    ("mamba2_snapshot_count", ctypes.c_int64, [_pb, _i32]),
    ("mamba2_conv1d_snap", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _pb, _pd, _vp]),
    ("mamba2_scan_prefill_snap", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _pb, _pd, _vp, _sz, _vp]),
    ("mamba2_scan_prefill_snap_workspace_bytes", _sz, [_pb, _pd, _i32]),
    ("mamba2_scan_verify", _i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _pb, _pd, _vp]),
    ("mamba2_commit_snapshots", _i32, [_vp, _vp, _vp, _vp, _i32, _vp, _pb, _pd, _vp]),
    ("mamba2_linear", _i32, [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i32, _vp]),
    ("mamba2_padded_runs", _i32, [_vp, _i32, _i32, _vp, _vp]),
    ("mamba2_pack_rows", _i32, [_vp, _vp, ctypes.c_int64, _i32, _i32, _pb, _vp]),
    ("mamba2_unpack_rows", _i32, [_vp, _vp, ctypes.c_int64, _i32, _i32, _pb, _vp]),
    ("mamba2_validate", _i32, [_pb, _pd, _i32]),
    ("mamba2_ssm_slot_bytes", _sz, [_pd]),
    ("mamba2_conv_slot_bytes", _sz, [_pd]),
    ("mamba2_status_string", ctypes.c_char_p, [_i32]),
    ("mamba2_timing_enable", _i32, [_i32]),
    ("mamba2_timing_collect", _i32, [ctypes.POINTER(KernelTime), _i32]),
    ("mamba3_siso_forward", _i32, [_vp] * 16 + [_p3b, _p3d, _vp, _sz, _vp]),
    ("mamba3_siso_forward_workspace_bytes", _sz, [_p3b, _p3d]),
]

_lib = None


def load() -> ctypes.CDLL:
    """Load libmamba2.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmamba2.so is not built (%s); run "
                               "`python -m mamba2_selective_scan_causalconv1d_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


class Mamba2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        msg = load().mamba2_status_string(self.status).decode()
        super().__init__("%s: status %d (%s)" % (where, self.status, msg))


def check(status: int, where: str) -> None:
    if status != OK:
        raise Mamba2Error(status, where)
