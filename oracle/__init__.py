"""Python face of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg are the only callers.  The product path never imports this
package.  Arrays are numpy: fp32 activations as ``float32``, bf16 activations as
their raw bits in ``uint16``.  Every function returns the status code of the
call (0 on success) and writes its outputs into the arrays passed in, exactly
as the C functions do.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "oracle_mamba3.c")]
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1

OK, INVALID_ARGUMENT, SLOT_OUT_OF_RANGE, SLOT_SHARED, RUN_LENGTHS = 0, 1, 2, 3, 4


def build(force: bool = False) -> str:
    """Compile oracle.c and oracle_mamba3.c with gcc (no fast-math, no FP contraction)."""
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in _SRCS)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"] + _SRCS +
            ["-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.oracle_conv1d.argtypes = [vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, i32, i32, i32, i32]
        L.oracle_scan.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp,
                                  i32, i32, i32, i32, i32, i32, vp, i32]
        L.oracle_gated_rmsnorm.argtypes = [vp, vp, vp, vp, i32, f32, i32, i32, i32]
        L.oracle_conv1d_snap.argtypes = L.oracle_conv1d.argtypes + [vp, i32]
        L.oracle_scan_snap.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp,
                                       i32, i32, i32, i32, i32, i32, vp, i32]
        L.oracle_commit.argtypes = [vp, vp, vp, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32]
        L.oracle_linear.argtypes = [vp, vp, vp, i32, i32, i32, i32]
        L.oracle_linear.restype = ctypes.c_int
        L.oracle_padded_runs.argtypes = [vp, i32, i32, vp, vp]
        L.oracle_pack_rows.argtypes = [vp, vp, i32, i32, vp, i32, ctypes.c_size_t]
        L.oracle_unpack_rows.argtypes = [vp, vp, i32, i32, vp, i32, ctypes.c_size_t]
        for f in (L.oracle_padded_runs, L.oracle_pack_rows, L.oracle_unpack_rows):
            f.restype = ctypes.c_int
        L.oracle_snapshot_count.argtypes = [i32, vp, i32]
        L.oracle_snapshot_count.restype = ctypes.c_longlong
        L.oracle_check_batch.argtypes = [i32, i32, vp, vp, i32, i32]
        for f in (L.oracle_conv1d, L.oracle_scan, L.oracle_gated_rmsnorm, L.oracle_check_batch,
                  L.oracle_max_threads, L.oracle_conv1d_snap, L.oracle_scan_snap, L.oracle_commit):
            f.restype = ctypes.c_int
        L.oracle_mamba3_forward.argtypes = [vp] * 16 + [i32, i32, vp, i32, i32, i32, i32]
        L.oracle_mamba3_forward.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [i32]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous, "oracle arrays must be C-contiguous numpy"
    return a.ctypes.data_as(ctypes.c_void_p)


def _act_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("activations are float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _batch(run_lengths, slots, fresh):
    rl = np.ascontiguousarray(run_lengths, dtype=np.int32)
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    fr = np.ascontiguousarray(fresh, dtype=np.uint8)
    return rl, sl, fr


def conv1d(dst, x, weight, bias, conv_state, run_lengths, slots, fresh) -> int:
    """CausalConv1D: dst, x [T, Dc] act; weight [Dc, K] f32; bias [Dc] f32;
    conv_state [M, K-1, Dc] act (updated in place)."""
    rl, sl, fr = _batch(run_lengths, slots, fresh)
    Dc = x.shape[1]
    K = weight.shape[1]
    M = conv_state.shape[0]
    return lib().oracle_conv1d(_p(dst), _p(x), _p(weight), _p(bias), _p(conv_state), len(rl),
                               x.shape[0], _p(rl), _p(sl), _p(fr), Dc, K, M, _act_of(x))


def scan(y, xbc, dt, a_log, dt_bias, d, ssm_state, run_lengths, slots, fresh, ngroups,
         head_mask=None, decode=False) -> int:
    """SSMScan: y [T, H*P] act; xbc [T, H*P + 2*G*N] act; dt [T, H] act; a_log, dt_bias,
    d [H] f32; ssm_state [M, H, P, N] f32 (updated in place)."""
    rl, sl, fr = _batch(run_lengths, slots, fresh)
    M, H, P, N = ssm_state.shape
    hm = None if head_mask is None else np.ascontiguousarray(head_mask, dtype=np.uint8)
    return lib().oracle_scan(_p(y), _p(xbc), _p(dt), _p(a_log), _p(dt_bias), _p(d), _p(ssm_state),
                             len(rl), xbc.shape[0], _p(rl), _p(sl), _p(fr), H, P, N, ngroups, M,
                             _act_of(xbc), _p(hm), 1 if decode else 0)


def snapshot_count(run_lengths, snap_every) -> int:
    """Snapshots a batch holds at stride E: sum over sequences of floor((L - 1) / E)."""
    rl = np.ascontiguousarray(run_lengths, dtype=np.int32)
    return int(lib().oracle_snapshot_count(len(rl), _p(rl), int(snap_every)))


def conv1d_snap(dst, x, weight, bias, conv_state, snaps, snap_every, run_lengths, slots, fresh) -> int:
    """conv1d plus conv-state snapshots every E rows: snaps [count, K-1, Dc] act."""
    rl, sl, fr = _batch(run_lengths, slots, fresh)
    Dc = x.shape[1]
    K = weight.shape[1]
    M = conv_state.shape[0]
    return lib().oracle_conv1d_snap(_p(dst), _p(x), _p(weight), _p(bias), _p(conv_state), len(rl),
                                    x.shape[0], _p(rl), _p(sl), _p(fr), Dc, K, M, _act_of(x), _p(snaps),
                                    int(snap_every))


def scan_snap(y, xbc, dt, a_log, dt_bias, d, ssm_state, snaps, snap_every, run_lengths, slots, fresh,
              ngroups) -> int:
    """scan plus SSM-state snapshots every E rows: snaps [count, H, P, N] f32."""
    rl, sl, fr = _batch(run_lengths, slots, fresh)
    M, H, P, N = ssm_state.shape
    return lib().oracle_scan_snap(_p(y), _p(xbc), _p(dt), _p(a_log), _p(dt_bias), _p(d), _p(ssm_state),
                                  len(rl), xbc.shape[0], _p(rl), _p(sl), _p(fr), H, P, N, ngroups, M,
                                  _act_of(xbc), _p(snaps), int(snap_every))


def commit(ssm_state, conv_state, ssm_snaps, conv_snaps, snap_every, accepted, run_lengths, slots) -> int:
    """Rollback to the accepted prefix: slots take the snapshots at the accepted boundary."""
    rl = np.ascontiguousarray(run_lengths, dtype=np.int32)
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    M, H, P, N = ssm_state.shape
    K1, Dc = conv_state.shape[1], conv_state.shape[2]
    act = F32 if conv_state.dtype == np.float32 else BF16
    return lib().oracle_commit(_p(ssm_state), _p(conv_state), _p(ssm_snaps), _p(conv_snaps), int(snap_every),
                               _p(acc), len(rl), _p(rl), _p(sl), H, P, N, Dc, K1 + 1, act)


def linear(dst, x, w) -> int:
    """dst [M, N] = x [M, K] . w [N, K]^T in double, one rounding to the activation type."""
    M, K = x.shape
    N = w.shape[0]
    return lib().oracle_linear(_p(dst), _p(x), _p(w), M, N, K, _act_of(x))


def padded_runs(mask):
    """(status, run lengths [B] int32, left_padded) of a [B, Lmax] mask."""
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    B, Lmax = m.shape
    lens = np.zeros(B, dtype=np.int32)
    left = np.zeros(1, dtype=np.int32)
    st = lib().oracle_padded_runs(_p(m), B, Lmax, _p(lens), _p(left))
    return st, lens, int(left[0])


def pack_rows(dst, src, lens, left_padded) -> int:
    """dst [T, ...] <- the real rows of src [B, Lmax, ...] (any dtype; rows copied as bytes)."""
    B, Lmax = src.shape[0], src.shape[1]
    rl = np.ascontiguousarray(lens, dtype=np.int32)
    return lib().oracle_pack_rows(_p(dst), _p(src), B, Lmax, _p(rl), int(left_padded),
                                  src[0, 0].nbytes)


def unpack_rows(dst, src, lens, left_padded) -> int:
    """dst [B, Lmax, ...] <- packed rows at their padded positions, zeros on padding."""
    B, Lmax = dst.shape[0], dst.shape[1]
    rl = np.ascontiguousarray(lens, dtype=np.int32)
    return lib().oracle_unpack_rows(_p(dst), _p(src), B, Lmax, _p(rl), int(left_padded),
                                    dst[0, 0].nbytes)


def gated_rmsnorm(dst, x, z, weight, groups, eps) -> int:
    """GatedRMSNorm: dst, x, z [rows, Di] act; weight [Di] f32."""
    return lib().oracle_gated_rmsnorm(_p(dst), _p(x), _p(z), _p(weight), int(groups), float(eps),
                                      x.shape[0], x.shape[1], _act_of(x))


def check_batch(num_rows, run_lengths, slots, pool_slots, decode=False) -> int:
    rl, sl, _ = _batch(run_lengths, slots, np.zeros(len(run_lengths)))
    return lib().oracle_check_batch(len(rl), num_rows, _p(rl), _p(sl), pool_slots, 1 if decode else 0)


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def mamba3_forward(q, k, v, adt, dt, trap, q_bias, k_bias, angles, d, z, run_lengths):
    """Mamba-3 SISO forward over packed sequences (oracle_mamba3.c).  q, k [T, DK] bf16 bits;
    v, z [T, H, DV] bf16 bits; adt, dt [T, H] f32; trap [T, H] bf16 bits; q_bias, k_bias [H, DK]
    f32; angles [T, NA] bf16 bits; d [H] f32.  Returns (status, out [T, H, DV] bf16 bits,
    final angle [S, H, NA] bf16 bits, final SSM [S, H, DV, DK] f32, final K [S, H, DK] f32,
    final V [S, H, DV] bf16 bits)."""
    T, H, DV = v.shape
    DK = q.shape[1]
    NA = angles.shape[1]
    rl = np.ascontiguousarray(run_lengths, dtype=np.int32)
    S = len(rl)
    out = np.zeros((T, H, DV), dtype=np.uint16)
    fa = np.zeros((S, H, NA), dtype=np.uint16)
    fs = np.zeros((S, H, DV, DK), dtype=np.float32)
    fk = np.zeros((S, H, DK), dtype=np.float32)
    fv = np.zeros((S, H, DV), dtype=np.uint16)
    st = lib().oracle_mamba3_forward(_p(out), _p(fa), _p(fs), _p(fk), _p(fv), _p(q), _p(k), _p(v), _p(adt),
                                     _p(dt), _p(trap), _p(q_bias), _p(k_bias), _p(angles), _p(d), _p(z), S, T,
                                     _p(rl), H, DK, DV, NA)
    return st, out, fa, fs, fk, fv
