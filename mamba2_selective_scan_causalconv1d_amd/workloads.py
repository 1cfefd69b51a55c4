"""Seeded synthetic workloads for the Mamba2 mixer hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the GPU path (through the tests and the bench) and
the CPU oracle consume the arrays it returns, so both see identical bits.

Canonical host arrays are numpy: fp32 as ``float32``; bf16 as the raw bits in
``uint16`` (rounded from fp32 with round-to-nearest-even).

Workload recipe (distributions as the mixer's five benchmark shapes give them;
"N(0, s)" means standard deviation s):
  * structure first (run lengths, slots, fresh flags), then parameters
    (conv weight N(0,0.5) [Dc,K], conv bias N(0,0.1), dt_bias U(-1,1),
    A_log = log U(1,16), D N(0,1), norm weight 1), then the state pools (every
    slot dirty: SSM N(0,0.1) fp32, conv N(0,1) in the activation type), then
    the activations xBC, z, dt ~ N(0,1) (per step, in step order, for decode).
  * numpy PCG64 (``default_rng(seed)``), draws in float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# ------------------------------------------------------------------ storage


def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_act(a, act: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a if act == "f32" else f32_to_bf16_bits(a)


def act_to_f32(a) -> np.ndarray:
    return a.astype(np.float32) if a.dtype == np.float32 else bf16_bits_to_f32(a)


# ------------------------------------------------------------------ shapes


@dataclass(frozen=True)
class Shape:
    nheads: int
    headdim: int
    d_state: int
    ngroups: int
    conv_kernel: int
    chunk_size: int
    norm_groups: int
    pool_slots: int
    act: str  # "f32" | "bf16"
    eps: float = 1e-5

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.d_state


@dataclass
class Workload:
    name: str
    seed: int
    shape: Shape
    run_lengths: np.ndarray  # int32 [S]
    slots: np.ndarray  # int32 [S]
    fresh: np.ndarray  # uint8 [S]
    conv_w: np.ndarray  # f32 [Dc, K]
    conv_b: np.ndarray  # f32 [Dc]
    dt_bias: np.ndarray  # f32 [H]
    a_log: np.ndarray  # f32 [H]
    D: np.ndarray  # f32 [H]
    norm_w: np.ndarray  # f32 [Di]
    conv_pool: np.ndarray  # act [M, K-1, Dc]
    ssm_pool: np.ndarray  # f32 [M, H, P, N]
    xbc: Optional[np.ndarray] = None  # act [T, Dc]   (prefill)
    z: Optional[np.ndarray] = None  # act [T, Di]
    dt: Optional[np.ndarray] = None  # act [T, H]
    steps: List[tuple] = field(default_factory=list)  # decode: [(xbc, z, dt)] per step

    @property
    def num_rows(self) -> int:
        return int(self.run_lengths.sum())

    @property
    def decode(self) -> bool:
        return bool(self.steps)


def _normal(rng, shape, sigma=1.0):
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def _params(rng, sh: Shape, a_log_range=(1.0, 16.0)):
    Dc, K, H = sh.conv_dim, sh.conv_kernel, sh.nheads
    conv_w = _normal(rng, (Dc, K), 0.5)
    conv_b = _normal(rng, (Dc,), 0.1)
    dt_bias = rng.uniform(-1.0, 1.0, H).astype(np.float32)
    a_log = np.log(rng.uniform(a_log_range[0], a_log_range[1], H)).astype(np.float32)
    D = _normal(rng, (H,), 1.0)
    norm_w = np.ones(sh.d_inner, dtype=np.float32)
    return conv_w, conv_b, dt_bias, a_log, D, norm_w


def _pools(rng, sh: Shape):
    M, H, P, N = sh.pool_slots, sh.nheads, sh.headdim, sh.d_state
    ssm = _normal(rng, (M, H, P, N), 0.1)
    conv = to_act(_normal(rng, (M, sh.conv_kernel - 1, sh.conv_dim), 1.0), sh.act)
    return conv, ssm


def _acts(rng, sh: Shape, T: int):
    xbc = to_act(_normal(rng, (T, sh.conv_dim)), sh.act)
    z = to_act(_normal(rng, (T, sh.d_inner)), sh.act)
    dt = to_act(_normal(rng, (T, sh.nheads)), sh.act)
    return xbc, z, dt


def make_prefill(name, seed, sh: Shape, run_lengths, slots, fresh, a_log_range=(1.0, 16.0),
                 rng=None) -> Workload:
    rng = rng if rng is not None else np.random.default_rng(seed)
    conv_w, conv_b, dt_bias, a_log, D, norm_w = _params(rng, sh, a_log_range)
    conv_pool, ssm_pool = _pools(rng, sh)
    rl = np.asarray(run_lengths, dtype=np.int32)
    xbc, z, dt = _acts(rng, sh, int(rl.sum()))
    return Workload(name, seed, sh, rl, np.asarray(slots, dtype=np.int32),
                    np.asarray(fresh, dtype=np.uint8), conv_w, conv_b, dt_bias, a_log, D, norm_w,
                    conv_pool, ssm_pool, xbc, z, dt)


# ------------------------------------------------------------ the five shapes

SHAPE_TINY = Shape(4, 16, 16, 2, 4, 16, 2, 1, "f32")
SHAPE_130M = Shape(24, 64, 128, 1, 4, 256, 1, 1, "bf16")
SHAPE_VARLEN = Shape(48, 64, 128, 1, 4, 256, 1, 16, "bf16")
SHAPE_DECODE = Shape(48, 64, 128, 1, 4, 256, 1, 512, "bf16")
SHAPE_LONG = Shape(48, 64, 128, 1, 4, 256, 8, 4, "bf16")


def tiny_fp32() -> Workload:
    """Tiny fp32 mixer, one fresh sequence of 64 rows (4 heads x 16, N=16, 2 groups)."""
    return make_prefill("tiny_fp32_L64", 0, SHAPE_TINY, [64], [0], [1])


def layer_130m_prefill(length: int = 2048) -> Workload:
    """Mamba2-130m-shaped layer prefill, batch 1, all fresh."""
    return make_prefill("m130_prefill_L%d" % length, 1, SHAPE_130M, [length], [0], [1])


def varlen_prefill(seed: int = 2, a_log_range=(1.0, 16.0), name="varlen8_prefill") -> Workload:
    """8 packed sequences, lengths U[100, 4000] (never a multiple of 256), slots drawn from a
    16-slot pool, half of them resuming from the dirty slot contents."""
    rng = np.random.default_rng(seed)
    lens = []
    while len(lens) < 8:
        v = int(rng.integers(100, 4001))
        while v % 256 == 0:
            v = int(rng.integers(100, 4001))
        lens.append(v)
    slots = rng.permutation(16)[:8]
    resume = rng.permutation(8)[:4]
    fresh = np.ones(8, dtype=np.uint8)
    fresh[resume] = 0
    return make_prefill(name, seed, SHAPE_VARLEN, lens, slots, fresh, a_log_range, rng=rng)


def varlen_slow_decay() -> Workload:
    """Varlen shapes with slow decay (A_log = log U(1e-3, 1e-2)), so that the state carried across
    chunks and the resumed slot states stay visible over many chunks."""
    return varlen_prefill(seed=102, a_log_range=(1e-3, 1e-2), name="varlen8_slow_decay")


def decode_batch(steps: int = 64, requests: int = 256) -> Workload:
    """Batched decode: `requests` one-token requests on distinct slots of a 512-slot pool, 10%
    fresh over dirty slots on the first step, `steps` successive steps."""
    sh = SHAPE_DECODE
    rng = np.random.default_rng(3)
    slots = rng.permutation(sh.pool_slots)[:requests]
    nfresh = int(round(0.1 * requests))
    fresh = np.zeros(requests, dtype=np.uint8)
    fresh[rng.permutation(requests)[:nfresh]] = 1
    conv_w, conv_b, dt_bias, a_log, D, norm_w = _params(rng, sh)
    conv_pool, ssm_pool = _pools(rng, sh)
    st = [_acts(rng, sh, requests) for _ in range(steps)]
    return Workload("decode%d_x%d" % (requests, steps), 3, sh, np.ones(requests, dtype=np.int32),
                    slots.astype(np.int32), fresh, conv_w, conv_b, dt_bias, a_log, D, norm_w,
                    conv_pool, ssm_pool, steps=st)


def verify_batch(requests: int = 256, rows: int = 4) -> Workload:
    """Speculative verify: `requests` sequences of `rows` draft rows each on distinct slots of
    the decode workload's 512-slot pool (same shape and distributions), 10% fresh."""
    sh = SHAPE_DECODE
    rng = np.random.default_rng(5)
    slots = rng.permutation(sh.pool_slots)[:requests]
    fresh = np.zeros(requests, dtype=np.uint8)
    fresh[rng.permutation(requests)[:int(round(0.1 * requests))]] = 1
    return make_prefill("verify%d_x%d" % (requests, rows), 5, sh, [rows] * requests, slots, fresh, rng=rng)


def long_prefill(batch: int = 4, length: int = 16384) -> Workload:
    """Long prefill: `batch` fresh sequences of `length` rows, gated RMSNorm over 8 groups."""
    return make_prefill("long_prefill_%dx%d" % (batch, length), 4, SHAPE_LONG, [length] * batch,
                        list(range(batch)), [1] * batch)


def decay_span_prefill(batch: int = 4, length: int = 16384) -> Workload:
    """Long-prefill shapes with A = exp(A_log) log-spaced over [1e-3, 30] across the heads and
    every other sequence resuming from its slot: per 64-row chunk the log-decay sum runs from
    about -0.05 (state carried over whole runs) through a few units (the state entering a chunk
    scaled down by many orders over a few chunks) to hundreds (the carried state far below fp32
    resolution of the chunk's own contribution)."""
    sh = SHAPE_LONG
    rng = np.random.default_rng(6)
    wl = make_prefill("decay_span_%dx%d" % (batch, length), 6, sh, [length] * batch, list(range(batch)),
                      [(i + 1) % 2 for i in range(batch)], rng=rng)
    wl.a_log = np.log(np.geomspace(1e-3, 30.0, sh.nheads)).astype(np.float32)
    return wl


def by_index(i: int) -> Workload:
    return [tiny_fp32, layer_130m_prefill, varlen_prefill, decode_batch, long_prefill][i]()


def random_prefill(seed: int, sh: Shape, run_lengths, fresh=None, slots=None,
                   a_log_range=(1.0, 16.0)) -> Workload:
    """A small seeded prefill of any shape (for edge-case and invariant tests)."""
    rng = np.random.default_rng(seed)
    S = len(run_lengths)
    if slots is None:
        slots = rng.permutation(sh.pool_slots)[:S]
    if fresh is None:
        fresh = rng.integers(0, 2, S)
    return make_prefill("random_s%d" % seed, seed, sh, run_lengths, slots, fresh, a_log_range,
                        rng=rng)


# ------------------------------------------------------------ Mamba-3 SISO varlen forward


@dataclass
class Mamba3Workload:
    """Inputs of the Mamba-3 SISO forward over packed sequences.  bf16 tensors as raw bits
    (uint16): q, k [T, DK]; v, z [T, H, DV]; trap [T, H]; angles [T, NA].  fp32: adt, dt
    [T, H]; q_bias, k_bias [H, DK]; d [H]."""
    name: str
    seed: int
    run_lengths: np.ndarray  # int32 [S]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    adt: np.ndarray
    dt: np.ndarray
    trap: np.ndarray
    q_bias: np.ndarray
    k_bias: np.ndarray
    angles: np.ndarray
    d: np.ndarray
    z: np.ndarray

    @property
    def num_rows(self) -> int:
        return int(self.run_lengths.sum())

    @property
    def nheads(self) -> int:
        return int(self.v.shape[1])


def mamba3_varlen(seed: int = 7, lengths=None, H: int = 32, DK: int = 128, DV: int = 64, NA: int = 32,
                  decay_range=(0.05, 8.0), name=None) -> Mamba3Workload:
    """Packed Mamba-3 SISO batch: three to five sequences of 3..15 chunks of 64 rows, never a
    multiple of 64 rows (unless `lengths` is given).  Per head a decay rate A drawn log-uniform
    over decay_range; per token dt = softplus(N(0,1) - 1) and adt = -A dt (the log of the
    token's decay); q, k, v, z, trap, angles ~ N(0,1); q_bias, k_bias ~ N(0, 0.1); d ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        S = int(rng.integers(3, 6))
        lengths = [64 * (int(rng.integers(3, 16)) - 1) + int(rng.integers(1, 64)) for _ in range(S)]
    rl = np.asarray(lengths, dtype=np.int32)
    T = int(rl.sum())
    A = np.exp(rng.uniform(np.log(decay_range[0]), np.log(decay_range[1]), H)).astype(np.float32)
    q_bias = _normal(rng, (H, DK), 0.1)
    k_bias = _normal(rng, (H, DK), 0.1)
    d = _normal(rng, (H,), 1.0)
    q = to_act(_normal(rng, (T, DK)), "bf16")
    k = to_act(_normal(rng, (T, DK)), "bf16")
    v = to_act(_normal(rng, (T, H, DV)), "bf16")
    z = to_act(_normal(rng, (T, H, DV)), "bf16")
    trap = to_act(_normal(rng, (T, H)), "bf16")
    angles = to_act(_normal(rng, (T, NA)), "bf16")
    u = _normal(rng, (T, H)).astype(np.float64) - 1.0
    dt = np.log1p(np.exp(u)).astype(np.float32)
    adt = (-A[None, :].astype(np.float64) * dt.astype(np.float64)).astype(np.float32)
    return Mamba3Workload(name or "mamba3_varlen_s%d" % seed, seed, rl, q, k, v, adt, dt, trap, q_bias, k_bias,
                          angles, d, z)
