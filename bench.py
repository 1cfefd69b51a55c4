"""Benchmark of the Mamba2 mixer hot path on one MI355X.

One step = one pass of the whole prefill path (causal conv1d + SiLU, chunked selective
scan, gated RMSNorm) over the long-prefill batch: 4 fresh sequences x 16384 rows, 48 heads
x headdim 64, d_state 128, one B/C group, conv kernel 4, norm over 8 groups, bf16
activations, fp32 states.  ``value`` is prefill tokens/s.  The decode half of the metric is
timed on the batched-decode workload (256 one-row requests on a 512-slot pool, 64
successive steps of conv + decode scan + norm) and reported as ``decode_us_per_step``.

Inputs are seeded synthetic tensors resident in HBM before the timed region, and 40 warm-up
steps let the clocks settle first.  Per-kernel durations come from HIP events the library
records on the launch stream around every launch, in a second pass of the same steps (the
events cost a few us per launch, so they stay out of the timed pass); the roofline
object uses the dominant kernel's algorithmic bytes (or flops) per launch over its average
duration.  The two smaller prefill workloads (the packed variable-length batch and one
2048-row 130m-shaped layer) are timed the same way and reported under ``other_workloads``.  The
CPU oracle is timed on a bounded sample on the host cores as a reported baseline.  Prints ONE
JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "mamba2_selective_scan_causalconv1d_amd", "csrc")
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "traffic_long_prefill_4x16384.txt")
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32, matrix (MFMA) and vector alike (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="GPU time spent on untimed steps before the warm-up, so the clocks settle")
    ap.add_argument("--reps", type=int, default=20, help="individually timed and digested prefill steps")
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="the long prefill only (for counter runs)")
    ap.add_argument("--no-others", action="store_true", help="skip the smaller prefill workloads")
    ap.add_argument("--no-snapshots", action="store_true", help="skip the snapshot and verify workloads")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this many MB (calibrates traffic counters)")
    ap.add_argument("--cpu-sample-rows", type=int, default=16384)
    return ap.parse_args()


def kernel_bytes_flops(name, wl, nrows):
    """Algorithmic bytes (and flops) one launch of `name` must move on this workload."""
    sh = wl.shape
    a = 2 if sh.act == "bf16" else 4
    T, Dc, Di, H, P, N, G = nrows, sh.conv_dim, sh.d_inner, sh.nheads, sh.headdim, sh.d_state, sh.ngroups
    S = len(wl.run_lengths)
    resumed = int((wl.fresh == 0).sum())
    if name == "conv1d_silu":
        return 2 * T * Dc * a + (S + resumed) * (sh.conv_kernel - 1) * Dc * a, 0
    if name in ("ssd_scan", "ssd_generic_scan", "scan_op"):
        return T * (Dc + H + Di) * a + (S + resumed) * H * P * N * 4, scan_flops(wl, T)[0]
    if name in ("gated_rmsnorm", "gated_rmsnorm_unit", "gated_rmsnorm_wide"):
        return 3 * T * Di * a + Di * 4, 0
    if name == "scan_decode":
        return (T * (Dc + H + Di) * a + (S + resumed) * H * P * N * 4), 6 * T * H * P * N
    return None, None


def scan_flops(wl, T):
    """Algorithmic and dense-tile flops of the chunked scan over T rows at the workload's chunk
    length Q.  Per row and head: C B^T over the causal triangle N (Q + 1) / (H / G) (shared by
    the heads of a group), the masked product with x P (Q + 1), the chunk state 2 N P and the
    state's output term 2 N P.  Dense tiles (the upper triangle not skipped) double the two
    triangular terms' Q / 2 to Q."""
    sh = wl.shape
    H, P, N, G, Q = sh.nheads, sh.headdim, sh.d_state, sh.ngroups, sh.chunk_size
    alg = T * H * (N * (Q + 1) / (H // G) + P * (Q + 1) + 4 * N * P)
    dense = T * H * (2 * N * Q / (H // G) + 2 * P * Q + 4 * N * P)
    return alg, dense


SCAN_KERNELS = ("scan_setup", "chunk_sums", "ssd_state", "scan_pass", "ssd_scan", "ssd_generic_state", "ssd_generic_scan")


def digest(torch, tensors):
    """64-bit digest of the exact bits of device tensors: per tensor, two int64 sums of its
    32-bit words (plain, and weighted by a position pattern), combined on the host."""
    h = hashlib.sha1()
    for t in tensors:
        flat = t.contiguous().view(-1)
        if flat.element_size() == 2 and flat.numel() % 2:
            h.update(("tail:%d;" % int(flat[-1:].view(torch.int16).item())).encode())
            flat = flat[:-1]
        w = flat.view(torch.int32)
        n = w.numel()
        s1 = s2 = 0
        step = 1 << 24
        pat = (torch.arange(step, device=w.device, dtype=torch.int64) % 1021) + 1
        for i in range(0, n, step):
            c = w[i:i + step].to(torch.int64)
            s1 += int(c.sum().item())
            s2 += int((c * pat[: c.numel()]).sum().item())
        h.update(("%d:%d:%d;" % (n, s1, s2)).encode())
    return h.hexdigest()[:16]


def sources_sha1(names):
    h = hashlib.sha1()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the counter table (FETCH_SIZE / WRITE_SIZE runs),
    or None when the table has no entry or the kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_TABLE):
        return None
    for line in open(TRAFFIC_TABLE):
        if not line.startswith("kernel="):
            continue
        kv = dict(f.split("=", 1) for f in line.split())
        if kv["kernel"] != kernel:
            continue
        if sources_sha1(kv["sources"].split(",")) != kv["sha1"]:
            return None
        return float(kv["bytes"])
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: every box here has one MI355X and this path has no "
              "multi-GPU part (--gpus %d is not supported)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from mamba2_selective_scan_causalconv1d_amd import ops
    from mamba2_selective_scan_causalconv1d_amd import workloads as W

    dev = "cuda"
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    t_gen = time.time()
    wl = W.long_prefill()
    sh = wl.shape
    T = wl.num_rows
    dims = ops.make_dims(sh.nheads, sh.headdim, sh.d_state, sh.ngroups, sh.conv_kernel, sh.chunk_size,
                         sh.pool_slots, sh.act)
    d = ops.to_device
    conv_w, conv_b, a_log, dt_bias, D, norm_w = (d(wl.conv_w), d(wl.conv_b), d(wl.a_log), d(wl.dt_bias),
                                                 d(wl.D), d(wl.norm_w))
    xbc, z, dt = d(wl.xbc), d(wl.z), d(wl.dt)
    conv_pool, ssm_pool = d(wl.conv_pool), d(wl.ssm_pool)
    batch = ops.RecurrentBatch(wl.run_lengths, wl.slots, wl.fresh, device=dev)
    xa = torch.empty_like(xbc)
    y = torch.empty((T, sh.d_inner), dtype=xbc.dtype, device=dev)
    out = torch.empty_like(y)
    ws = torch.empty(max(256, ops.scan_prefill_workspace_bytes(batch, dims)), dtype=torch.uint8, device=dev)
    print("bench: inputs ready in %.1fs (T=%d, workspace %.1f MB)" % (time.time() - t_gen, T, ws.numel() / 1e6),
          file=sys.stderr, flush=True)

    def step():
        ops.conv1d(xa, xbc, conv_w, conv_b, conv_pool, batch, dims)
        ops.scan_prefill(y, xa, dt, a_log, dt_bias, D, ssm_pool, batch, dims, workspace=ws)
        ops.gated_rmsnorm(out, y, z, norm_w, sh.norm_groups, sh.eps)

    slots = torch.from_numpy(wl.slots.astype(np.int64)).to(dev)

    def step_digest():
        # every output of a step and the states it leaves in its slots (all-fresh batch: every
        # step recomputes the same bits)
        return digest(torch, [xa, y, out, conv_pool.index_select(0, slots), ssm_pool.index_select(0, slots)])

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the digest of a first (untimed) run: every timed step must reproduce it
    step()
    torch.cuda.synchronize()
    ref_digest = step_digest()

    # clock settling: untimed steps worth settle_ms of GPU time, reported on their own
    e0.record()
    step()
    e1.record()
    torch.cuda.synchronize()
    n_settle = max(1, int(args.settle_ms / max(e0.elapsed_time(e1), 1e-3)))
    e0.record()
    for _ in range(n_settle):
        step()
    e1.record()
    torch.cuda.synchronize()
    settle = {"steps": n_settle + 1, "ms": e0.elapsed_time(e1)}

    # the contract's timed region: W warm-up steps, then exactly K steps back to back
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # per-kernel durations: the same K steps again, straight after the timed region (same
    # clock state), with the library's HIP events recorded on the launch stream around every
    # kernel (they add a few us per launch, hence a pass of its own)
    ops.timing_enable(64 * max(1, args.steps))
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    recs = ops.timing_collect(64 * max(1, args.steps))
    ops.timing_enable(0)
    # every step rewrites the same bits, so the outputs and states left now are the timed
    # steps' ones too
    assert step_digest() == ref_digest, "timed output differs from the parity run"

    # repetitions: each step timed on its own with HIP events on the launch stream, then its
    # outputs and states digested (outside the timed span) and compared with the first run's
    rep_ms = []
    for _ in range(max(1, args.reps)):
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        rep_ms.append(e0.elapsed_time(e1))
        assert step_digest() == ref_digest, "a repetition's outputs or states differ from the parity run"
    reps = {"n": len(rep_ms), "median_ms": float(np.median(rep_ms)), "min_ms": float(np.min(rep_ms)),
            "max_ms": float(np.max(rep_ms)), "median_tokens_per_s": T / (float(np.median(rep_ms)) * 1e-3),
            "digest": ref_digest, "digests_matched": len(rep_ms) + 1}

    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    kernels = {k: {"avg_us": 1e3 * float(np.mean(v)), "launches_per_step": len(v) / args.steps}
               for k, v in per.items()}
    rooflines = {}
    for k, v in kernels.items():
        nbytes, flops = kernel_bytes_flops(k, wl, T)
        if nbytes is None:
            continue
        sec = v["avg_us"] * 1e-6
        r = {"achieved_GBs": nbytes / sec / 1e9, "frac_hbm": nbytes / sec / 1e9 / HBM_PEAK_GBS,
             "alg_bytes": nbytes}
        if flops:
            r["achieved_TFLOPs"] = flops / sec / 1e12
            r["frac_mfma"] = flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS
            r["alg_flops"] = flops
        rooflines[k] = r
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches_per_step"])
    dr = rooflines.get(dom, {})
    traffic = measured_traffic(dom)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": dr.get("achieved_GBs"), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": dr.get("frac_hbm"), "traffic": traffic,
                "traffic_source": None if traffic is None else
                "rocprofv3 FETCH_SIZE and WRITE_SIZE per launch, scaled by a plain copy's counts "
                "(profiles/traffic_long_prefill_4x16384.txt, taken on these kernel sources)",
                "avg_us": kernels[dom]["avg_us"],
                "alg_bytes_scope": "the whole scan op's algorithmic bytes (x, B, C, dt read; y written; states)"}
    # the scan op as a whole: every launch it makes, against its algorithmic bytes and flops
    scan_us = sum(v["avg_us"] * v["launches_per_step"] for k, v in kernels.items() if k in SCAN_KERNELS)
    sb, _ = kernel_bytes_flops("scan_op", wl, T)
    sf, sfd = scan_flops(wl, T)
    scan_op = {"kernels": [k for k in kernels if k in SCAN_KERNELS], "us_per_step": scan_us,
               "alg_bytes": sb, "achieved_GBs": sb / (scan_us * 1e-6) / 1e9,
               "frac_hbm": sb / (scan_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
               "alg_flops": sf, "dense_flops": sfd, "chunk_for_flops": sh.chunk_size,
               "achieved_TFLOPs": sf / (scan_us * 1e-6) / 1e12,
               "frac_mfma": sf / (scan_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}

    if args.copy_calibration_mb:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE give the counters' scale
        src = torch.empty(args.copy_calibration_mb * (1 << 20) // 2, dtype=torch.bfloat16, device=dev)
        src.fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- decode
    decode_us, dkern, dec_roof, R, dsh, dsteps, drep = None, None, None, None, None, [], None
    if not args.no_decode:
        decode_us, dkern, dec_roof, R, dsh, dsteps, drep = run_decode(args, torch, ops, W, dev, e0, e1)

    # ---------------------------------------------------------------- smaller prefills
    others = None if (args.no_others or args.no_decode) else run_other_prefills(args, torch, ops, W, dev)
    if others is not None:
        others["mamba3_siso_varlen"] = run_mamba3(args, torch, ops, W, dev)

    # ---------------------------------------------------------------- snapshots and verify
    snaps = None
    if not (args.no_snapshots or args.no_decode):
        def long_snap_step(E, snaps_c, snaps_s, ws_snap):
            ops.conv1d_snap(xa, xbc, conv_w, conv_b, conv_pool, snaps_c, E, batch, dims)
            ops.scan_prefill_snap(y, xa, dt, a_log, dt_bias, D, ssm_pool, snaps_s, E, batch, dims, workspace=ws_snap)
            ops.gated_rmsnorm(out, y, z, norm_w, sh.norm_groups, sh.eps)

        snaps = run_snapshots(args, torch, ops, W, dev, e0, e1, long_snap_step, batch, dims, sh, ms_per_step)
        snaps["padded"] = run_padded(torch, ops, W, dev, e0, e1)

    # ---------------------------------------------------------------- the whole layer
    layer = None
    if not (args.no_snapshots or args.no_decode):
        layer = run_layer(args, torch, ops, dev, e0, e1, xbc, z, dt, xa, y, out, conv_w, conv_b, a_log, dt_bias,
                          D, norm_w, conv_pool, ssm_pool, batch, dims, sh, ws)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, W, wl, sh)

    res = {
        "metric": "Mamba2 mixer prefill tokens/s + decode us/step; % of HBM/MFMA roofline",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settle,
        "ms_per_step": ms_per_step,
        "repetitions": reps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long_prefill_4x16384", "global_batch": 4, "seq_len": 16384, "nheads": 48,
                   "headdim": 64, "d_state": 128, "ngroups": 1, "conv_kernel": 4, "norm_groups": 8,
                   "parallelism": "single_gpu"},
        "decode_us_per_step": decode_us,
        "decode_config": None if args.no_decode else
        {"workload": "decode_256x64", "requests": R, "pool_slots": dsh.pool_slots, "steps": len(dsteps)},
        "decode_repetitions": drep,
        "roofline": roofline,
        "scan_op": scan_op,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "rooflines": rooflines,
        "decode_kernels": dkern,
        "decode_roofline": dec_roof,
        "other_workloads": others,
        "snapshots": snaps,
        "layer": layer,
    }
    print(json.dumps(res))


def run_decode(args, torch, ops, W, dev, e0, e1):
    """64 successive decode steps of 256 requests (conv step, decode scan, norm per step), timed
    as one span per repetition; the pools are restored from pristine copies outside the span.
    Each step writes its own output buffers, so after every repetition the outputs of all 64
    steps and the final pools are digested and compared with the first run's."""
    d = ops.to_device
    dwl = W.decode_batch()
    dsh = dwl.shape
    ddims = ops.make_dims(dsh.nheads, dsh.headdim, dsh.d_state, dsh.ngroups, dsh.conv_kernel, dsh.chunk_size,
                          dsh.pool_slots, dsh.act)
    dparams = [d(a) for a in (dwl.conv_w, dwl.conv_b, dwl.a_log, dwl.dt_bias, dwl.D, dwl.norm_w)]
    dsteps = [tuple(d(a) for a in s) for s in dwl.steps]
    pristine_conv, pristine_ssm = d(dwl.conv_pool), d(dwl.ssm_pool)
    cpool, spool = pristine_conv.clone(), pristine_ssm.clone()
    b0 = ops.RecurrentBatch(dwl.run_lengths, dwl.slots, dwl.fresh, device=dev)
    b1 = ops.RecurrentBatch(dwl.run_lengths, dwl.slots, np.zeros_like(dwl.fresh), device=dev)
    R = len(dwl.run_lengths)
    nS = len(dsteps)
    dxa = torch.empty((nS, R, dsh.conv_dim), dtype=torch.bfloat16, device=dev)
    dy = torch.empty((nS, R, dsh.d_inner), dtype=torch.bfloat16, device=dev)
    dout = torch.empty_like(dy)

    def decode_run():
        cw, cb, al, db, DD, nw = dparams
        for i, (x, zz, dd) in enumerate(dsteps):
            b = b0 if i == 0 else b1
            ops.conv1d(dxa[i], x, cw, cb, cpool, b, ddims)
            ops.scan_decode(dy[i], dxa[i], dd, al, db, DD, spool, b, ddims)
            ops.gated_rmsnorm(dout[i], dy[i], zz, nw, dsh.norm_groups, dsh.eps)

    def run_digest():
        return digest(torch, [dxa, dy, dout, cpool, spool])

    def restore():
        cpool.copy_(pristine_conv)
        spool.copy_(pristine_ssm)
        torch.cuda.synchronize()

    restore()
    decode_run()  # warm-up, and the reference digest
    torch.cuda.synchronize()
    dref = run_digest()
    times = []
    for _ in range(max(1, args.decode_reps)):
        restore()
        e0.record()
        decode_run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        assert run_digest() == dref, "a decode repetition differs from the first run"
    decode_us = 1e3 * float(np.median(times)) / nS
    drep = {"n": len(times), "median_us_per_step": decode_us, "min_us_per_step": 1e3 * float(np.min(times)) / nS,
            "max_us_per_step": 1e3 * float(np.max(times)) / nS, "digest": dref, "digests_matched": len(times) + 1}

    # the same 64 steps captured once in a HIP graph and replayed (the launch pattern of a
    # serving loop that captures its decode step); every replay is checked against the eager
    # run's digest, with eager work and synchronisations in between
    g = torch.cuda.CUDAGraph()
    restore()
    with torch.cuda.graph(g):
        decode_run()
    gtimes = []
    for _ in range(max(1, args.decode_reps)):
        restore()
        dout.zero_()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        gtimes.append(e0.elapsed_time(e1))
        assert run_digest() == dref, "graph replay differs from the eager run"
    graph_us = 1e3 * float(np.median(gtimes)) / nS
    del g
    # per-kernel durations: one more run with the library's HIP events around every launch
    restore()
    ops.timing_enable(4096)
    decode_run()
    torch.cuda.synchronize()
    drecs = ops.timing_collect(4096)
    ops.timing_enable(0)
    dper = {}
    for name, ms in drecs:
        dper.setdefault(name, []).append(ms)
    dkern = {k: {"avg_us": 1e3 * float(np.mean(v)), "launches_per_step": len(v) / nS}
             for k, v in dper.items()}
    # steps 1..63 read every slot (none fresh): algorithmic bytes of a resumed step
    dec_bytes = R * (dsh.conv_dim + dsh.nheads + dsh.d_inner) * 2 + 2 * R * dsh.nheads * dsh.headdim * dsh.d_state * 4
    # the whole step, fused-mixer count (inputs xBC, dt, z read, the output written, both states
    # read and written once): 3,204,704 bytes per request at this shape
    step_bytes = R * (2 * dsh.nheads * dsh.headdim * dsh.d_state * 4 + 2 * (dsh.conv_kernel - 1) * dsh.conv_dim * 2 +
                      (dsh.conv_dim + dsh.nheads + 2 * dsh.d_inner) * 2)
    skern = [k for k in dkern if k.startswith("scan_decode")]
    dec_roof = {"kernel": skern[0] if skern else None,
                "achieved_GBs": dec_bytes / (dkern[skern[0]]["avg_us"] * 1e-6) / 1e9 if skern else None,
                "step_alg_bytes": step_bytes, "step_GBs": step_bytes / (decode_us * 1e-6) / 1e9,
                "step_frac_hbm": step_bytes / (decode_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    if skern:
        dec_roof["frac_hbm"] = dec_roof["achieved_GBs"] / HBM_PEAK_GBS
    dec_roof["graph_us_per_step"] = graph_us
    return decode_us, dkern, dec_roof, R, dsh, dsteps, drep


def run_snapshots(args, torch, ops, W, dev, e0, e1, long_snap_step, long_batch, long_dims, long_sh,
                  long_ms):
    """State snapshots and speculative verify.  (1) The verify workload: 256 sequences of 4
    draft rows on the decode workload's 512-slot pool, one step = conv with per-row conv
    snapshots + the verify scan with per-row SSM snapshots + the norm, timed against the same
    step without snapshots; then the commit of random accepted counts.  (2) The long prefill
    with snapshots every 1024 rows against the plain prefill step."""
    d = ops.to_device
    vwl = W.verify_batch()
    sh = vwl.shape
    dims = ops.make_dims(sh.nheads, sh.headdim, sh.d_state, sh.ngroups, sh.conv_kernel, sh.chunk_size,
                         sh.pool_slots, sh.act)
    cw, cb, al, db, DD, nw = [d(a) for a in (vwl.conv_w, vwl.conv_b, vwl.a_log, vwl.dt_bias, vwl.D, vwl.norm_w)]
    x, z, dt = d(vwl.xbc), d(vwl.z), d(vwl.dt)
    pristine_c, pristine_s = d(vwl.conv_pool), d(vwl.ssm_pool)
    cp, sp = pristine_c.clone(), pristine_s.clone()
    b = ops.RecurrentBatch(vwl.run_lengths, vwl.slots, vwl.fresh, device=dev)
    T, R, rows = vwl.num_rows, len(vwl.run_lengths), int(vwl.run_lengths[0])
    n = ops.snapshot_count(b, 1)
    csn = torch.empty((n, sh.conv_kernel - 1, sh.conv_dim), dtype=torch.bfloat16, device=dev)
    ssn = torch.empty((n, sh.nheads, sh.headdim, sh.d_state), dtype=torch.float32, device=dev)
    xa = torch.empty_like(x)
    y = torch.empty((T, sh.d_inner), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(y)
    accepted = torch.from_numpy(np.random.default_rng(5).integers(1, rows + 1, R).astype(np.int32)).to(dev)

    def step(snap):
        if snap:
            ops.conv1d_snap(xa, x, cw, cb, cp, csn, 1, b, dims)
        else:
            ops.conv1d(xa, x, cw, cb, cp, b, dims)
        ops.scan_verify(y, xa, dt, al, db, DD, sp, ssn if snap else None, b, dims)
        ops.gated_rmsnorm(out, y, z, nw, sh.norm_groups, sh.eps)

    def timed(fn, reps=7):
        times = []
        for _ in range(reps):
            cp.copy_(pristine_c)
            sp.copy_(pristine_s)
            torch.cuda.synchronize()
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(times[1:]))

    us_snap = timed(lambda: step(True))
    us_plain = timed(lambda: step(False))
    step(True)
    torch.cuda.synchronize()
    t0 = []
    for _ in range(7):
        e0.record()
        ops.commit_snapshots(sp, cp, ssn, csn, 1, accepted, b, dims)
        e1.record()
        torch.cuda.synchronize()
        t0.append(e0.elapsed_time(e1) * 1e3)
    us_commit = float(np.median(t0[1:]))
    ops.timing_enable(64)
    cp.copy_(pristine_c)
    sp.copy_(pristine_s)
    step(True)
    ops.commit_snapshots(sp, cp, ssn, csn, 1, accepted, b, dims)
    torch.cuda.synchronize()
    kern = {k: round(1e3 * ms, 2) for k, ms in ops.timing_collect(64)}
    ops.timing_enable(0)
    H, P, N = sh.nheads, sh.headdim, sh.d_state
    resumed = int((vwl.fresh == 0).sum())
    vbytes = (resumed + R) * H * P * N * 4 + n * H * P * N * 4 + T * (sh.conv_dim + H + sh.d_inner) * 2
    verify = {"workload": "verify_%dx%d" % (R, rows), "requests": R, "rows_per_request": rows,
              "us_per_step": us_snap, "tokens_per_s": T / (us_snap * 1e-6), "us_per_step_no_snapshots": us_plain,
              "commit_us": us_commit, "kernels_us": kern, "scan_verify_alg_bytes": vbytes,
              "scan_verify_GBs": vbytes / (kern["scan_verify"] * 1e-6) / 1e9}

    # (2) long prefill, snapshots every 1024 rows
    E = 1024
    nl = ops.snapshot_count(long_batch, E)
    lc = torch.empty((nl, long_sh.conv_kernel - 1, long_sh.conv_dim), dtype=torch.bfloat16, device=dev)
    ls = torch.empty((nl, long_sh.nheads, long_sh.headdim, long_sh.d_state), dtype=torch.float32, device=dev)
    ws = torch.empty(max(256, ops.scan_prefill_snap_workspace_bytes(long_batch, long_dims, E)), dtype=torch.uint8,
                     device=dev)
    for _ in range(5):
        long_snap_step(E, lc, ls, ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        long_snap_step(E, lc, ls, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    prefill = {"workload": "long_prefill_4x16384", "snap_every": E, "snapshots": nl, "ms_per_step": ms,
               "overhead_vs_plain_step": ms / long_ms - 1.0,
               "snapshot_bytes": nl * (long_sh.nheads * long_sh.headdim * long_sh.d_state * 4 +
                                       (long_sh.conv_kernel - 1) * long_sh.conv_dim * 2)}
    del lc, ls, ws
    return {"verify": verify, "prefill": prefill}


def run_layer(args, torch, ops, dev, e0, e1, xbc, z, dt, xa, y, out, conv_w, conv_b, a_log, dt_bias, D, norm_w,
              conv_pool, ssm_pool, batch, dims, sh, ws):
    """The whole mixer layer on the long-prefill batch: in_proj (z, xBC and dt from model-width
    hidden states, three calls on row slices of one weight) -> the path -> out_proj, model
    width Di / 2 = 1536, random weights of that architecture (scaled by 1/sqrt(fan-in))."""
    T, Di, Dc, H = xbc.shape[0], sh.d_inner, sh.conv_dim, sh.nheads
    d_model = Di // 2
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    hid = torch.randn((T, d_model), generator=g, device=dev).to(torch.bfloat16)
    w_in = (torch.randn((Di + Dc + H, d_model), generator=g, device=dev) * d_model ** -0.5).to(torch.bfloat16)
    w_out = (torch.randn((d_model, Di), generator=g, device=dev) * Di ** -0.5).to(torch.bfloat16)
    res_out = torch.empty((T, d_model), dtype=torch.bfloat16, device=dev)

    def in_proj():
        ops.linear(z, hid, w_in[:Di])
        ops.linear(xbc, hid, w_in[Di:Di + Dc])
        ops.linear(dt, hid, w_in[Di + Dc:])

    def step():
        in_proj()
        ops.conv1d(xa, xbc, conv_w, conv_b, conv_pool, batch, dims)
        ops.scan_prefill(y, xa, dt, a_log, dt_bias, D, ssm_pool, batch, dims, workspace=ws)
        ops.gated_rmsnorm(out, y, z, norm_w, sh.norm_groups, sh.eps)
        ops.linear(res_out, out, w_out)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ops.timing_enable(64)
    step()
    torch.cuda.synchronize()
    recs = ops.timing_collect(64)
    ops.timing_enable(0)
    lin = [1e3 * t for name, t in recs if name == "linear"]  # z, xBC, dt, out_proj
    shapes = [(Di, d_model), (Dc, d_model), (H, d_model), (d_model, Di)]
    gemms = []
    for (n, k), us in zip(shapes, lin):
        fl = 2.0 * T * n * k
        by = 2.0 * (T * k + n * k + T * n)  # x, w and dst once
        gemms.append({"N": n, "K": k, "us": us, "TFLOPs": fl / (us * 1e-6) / 1e12, "GBs": by / (us * 1e-6) / 1e9,
                      "frac_mfma": fl / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS})
    tot_fl = sum(2.0 * T * n * k for n, k in shapes)
    tot_us = sum(lin)
    # the sums keep the work from being optimised out and show the output is finite
    assert torch.isfinite(res_out.float()).all()
    return {"workload": "long_prefill_4x16384_layer", "d_model": d_model, "ms_per_step": ms,
            "tokens_per_s": T / (ms * 1e-3), "gemms": gemms, "gemm_us": tot_us,
            "gemm_TFLOPs": tot_fl / (tot_us * 1e-6) / 1e12,
            "gemm_frac_mfma": tot_fl / (tot_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def run_padded(torch, ops, W, dev, e0, e1):
    """The padded-batch front end on the varlen batch laid out left-padded ([8, Lmax] rows):
    pack of the xBC, z and dt rows into the packed layout and unpack of the output."""
    vwl = W.varlen_prefill()
    sh = vwl.shape
    lens = vwl.run_lengths
    Lmax = int(lens.max())
    b = ops.RecurrentBatch(lens, vwl.slots, vwl.fresh, device=dev)
    T, B = vwl.num_rows, len(lens)
    bf = torch.bfloat16
    srcs = [torch.zeros((B, Lmax, c), dtype=bf, device=dev) for c in (sh.conv_dim, sh.d_inner, sh.nheads)]
    dsts = [torch.empty((T, c), dtype=bf, device=dev) for c in (sh.conv_dim, sh.d_inner, sh.nheads)]
    outp = torch.empty((B, Lmax, sh.d_inner), dtype=bf, device=dev)

    def pack():
        for dst, src in zip(dsts, srcs):
            ops.pack_rows(dst, src, 1, b)

    def unpack():
        ops.unpack_rows(outp, dsts[1], 1, b)

    res = {"workload": "varlen8_left_padded", "rows": T, "padded_rows": B * Lmax}
    for name, fn, nbytes in (("pack", pack, 2 * T * (sh.conv_dim + sh.d_inner + sh.nheads) * 2),
                             ("unpack", unpack, (T + B * Lmax) * sh.d_inner * 2)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 20 * 1e3
        res[name + "_us"] = us
        res[name + "_GBs"] = nbytes / (us * 1e-6) / 1e9
        # GPU time of the launches alone (HIP events around each launch): the calls above
        # include the host's per-call cost, which the short launches do not cover
        ops.timing_enable(64)
        per_call = []
        for _ in range(5):
            fn()
            torch.cuda.synchronize()
            per_call.append(1e3 * sum(ms for _, ms in ops.timing_collect(64)))
        ops.timing_enable(0)
        kus = float(np.median(per_call))
        res[name + "_kernel_us"] = kus
        res[name + "_kernel_GBs"] = nbytes / (kus * 1e-6) / 1e9
    return res


def run_other_prefills(args, torch, ops, W, dev):
    """The two smaller prefill workloads: the packed variable-length batch (8 sequences of
    100..4000 rows, half resuming from their slots) and one 2048-row layer of the 130m shape.
    Whole-step time (conv + scan + norm) and per-kernel HIP-event times; the pools are restored
    from pristine copies before each timed pass, outside it."""
    res = {}
    for wl in (W.varlen_prefill(), W.layer_130m_prefill()):
        sh = wl.shape
        T = wl.num_rows
        d = ops.to_device
        dims = ops.make_dims(sh.nheads, sh.headdim, sh.d_state, sh.ngroups, sh.conv_kernel, sh.chunk_size,
                             sh.pool_slots, sh.act)
        cw, cb, al, db, DD, nw = (d(a) for a in (wl.conv_w, wl.conv_b, wl.a_log, wl.dt_bias, wl.D, wl.norm_w))
        xbc, z, dt = d(wl.xbc), d(wl.z), d(wl.dt)
        cp0, sp0 = d(wl.conv_pool), d(wl.ssm_pool)
        cp, sp = cp0.clone(), sp0.clone()
        b = ops.RecurrentBatch(wl.run_lengths, wl.slots, wl.fresh, device=dev)
        xa = torch.empty_like(xbc)
        y = torch.empty((T, sh.d_inner), dtype=xbc.dtype, device=dev)
        out = torch.empty_like(y)
        ws = torch.empty(max(256, ops.scan_prefill_workspace_bytes(b, dims)), dtype=torch.uint8, device=dev)

        def step():
            ops.conv1d(xa, xbc, cw, cb, cp, b, dims)
            ops.scan_prefill(y, xa, dt, al, db, DD, sp, b, dims, workspace=ws)
            ops.gated_rmsnorm(out, y, z, nw, sh.norm_groups, sh.eps)

        for _ in range(args.warmup):
            step()
        cp.copy_(cp0)
        sp.copy_(sp0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        cp.copy_(cp0)
        sp.copy_(sp0)
        torch.cuda.synchronize()
        ops.timing_enable(64 * max(1, args.steps))
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        per = {}
        for name, t in ops.timing_collect(64 * max(1, args.steps)):
            per.setdefault(name, []).append(t)
        ops.timing_enable(0)
        res[wl.name] = {"rows": T, "sequences": len(wl.run_lengths), "us_per_step": 1e3 * ms,
                        "tokens_per_s": T / (ms * 1e-3),
                        "kernels_us": {k: 1e3 * float(np.mean(v)) * len(v) / args.steps for k, v in per.items()}}
    return res


def _oracle_prefill(oracle, wl, sub_rows=None):
    """conv -> scan -> norm of the oracle on a workload (or on the first sub_rows rows of every
    sequence); returns (rows, seconds)."""
    sh = wl.shape
    if sub_rows is not None:
        L = min(sub_rows, int(wl.run_lengths.min()))
        cu = np.concatenate([[0], np.cumsum(wl.run_lengths)])
        rows = np.concatenate([np.arange(cu[s], cu[s] + L) for s in range(len(wl.run_lengths))])
        lens = np.full(len(wl.run_lengths), L, np.int32)
        xbc, z, dt = (np.ascontiguousarray(a[rows]) for a in (wl.xbc, wl.z, wl.dt))
    else:
        lens, xbc, z, dt = wl.run_lengths, wl.xbc, wl.z, wl.dt
    T = int(lens.sum())
    t0 = time.perf_counter()
    oa = np.zeros_like(xbc)
    cp = wl.conv_pool.copy()
    assert oracle.conv1d(oa, xbc, wl.conv_w, wl.conv_b, cp, lens, wl.slots, wl.fresh) == 0
    oy = np.zeros((T, sh.d_inner), dtype=xbc.dtype)
    sp = wl.ssm_pool.copy()
    assert oracle.scan(oy, oa, dt, wl.a_log, wl.dt_bias, wl.D, sp, lens, wl.slots, wl.fresh, sh.ngroups) == 0
    oo = np.zeros_like(oy)
    assert oracle.gated_rmsnorm(oo, oy, z, wl.norm_w, sh.norm_groups, sh.eps) == 0
    return T, time.perf_counter() - t0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def mamba3_flops(wl, Q=64):
    """Algorithmic flops of the chunked Mamba-3 forward: per row and head, q.k over the causal
    triangle of its chunk DK (Q + 1), the masked product with v DV (Q + 1), and the state's
    output term and the chunk state 2 DK DV each."""
    T, H, DV = wl.v.shape
    DK = wl.q.shape[1]
    return T * H * (DK * (Q + 1) + DV * (Q + 1) + 4 * DK * DV)


def run_mamba3(args, torch, ops, W, dev):
    """The Mamba-3 SISO forward on its seeded packed batch (3-5 sequences of 3-15 chunks, 32
    heads): 20 calls timed one by one with HIP events, each call's outputs and final states
    digested and compared with the first call's; per-kernel times from one more call."""
    wl = W.mamba3_varlen()
    T, H, DV = wl.v.shape
    DK, NA, S = wl.q.shape[1], wl.angles.shape[1], len(wl.run_lengths)
    names = ("q", "k", "v", "adt", "dt", "trap", "q_bias", "k_bias", "angles", "d", "z")
    ins = [ops.to_device(getattr(wl, n)) for n in names]
    out = torch.empty((T, H, DV), dtype=torch.bfloat16, device=dev)
    fa = torch.empty((S, H, NA), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((S, H, DV, DK), dtype=torch.float32, device=dev)
    fk = torch.empty((S, H, DK), dtype=torch.float32, device=dev)
    fv = torch.empty((S, H, DV), dtype=torch.bfloat16, device=dev)
    b = ops.Mamba3Batch(wl.run_lengths, device=dev)
    dims = ops.mamba3_dims(H, DK, DV, NA)
    ws = torch.empty(max(256, ops.mamba3_workspace_bytes(b, dims)), dtype=torch.uint8, device=dev)

    def call():
        ops.mamba3_siso_forward(out, fa, fs, fk, fv, *ins, b, dims, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = digest(torch, [out, fa, fs, fk, fv])
    for _ in range(5):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(max(20, args.reps)):
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
        assert digest(torch, [out, fa, fs, fk, fv]) == ref, "a Mamba-3 call's outputs differ from the first"
    ops.timing_enable(64)
    call()
    torch.cuda.synchronize()
    kern = {}
    for name, ms in ops.timing_collect(64):
        kern[name] = kern.get(name, 0.0) + 1e3 * ms
    ops.timing_enable(0)
    us = float(np.median(times))
    fl = mamba3_flops(wl)
    return {"workload": "mamba3_siso_varlen_s7", "rows": T, "sequences": S, "lengths": [int(x) for x in wl.run_lengths],
            "heads": H, "qk_dim": DK, "v_dim": DV, "nangles": NA, "median_us": us, "min_us": float(np.min(times)),
            "tokens_per_s": T / (us * 1e-6), "kernels_us": kern, "alg_flops": fl,
            "achieved_TFLOPs": fl / (us * 1e-6) / 1e12,
            "frac_fp32_mfma_peak": fl / (us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS,
            "digest": ref, "digests_matched": len(times) + 1}


def cpu_baseline(args, W, wl, sh):
    """The oracle (as it stands) timed on the host cores, after the GPU work: the long-prefill
    batch (first cpu_sample_rows rows of every sequence; the whole batch by default) on all the
    threads the process may use, the tiny fp32 and 130m-shaped prefills on one thread as well,
    and a few decode steps of the 256-request batch."""
    import oracle

    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = oracle.max_threads()
    T, sec = _oracle_prefill(oracle, wl, args.cpu_sample_rows)
    cpu = {"value": T / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": "%d sequences x first %d rows of the long-prefill batch (48 heads, conv+scan+norm), "
                     "%.1f s wall on %d threads" % (len(wl.run_lengths), T // len(wl.run_lengths), sec, threads),
           "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": ncpu}
    small = {}
    for name, w in (("tiny_fp32", W.tiny_fp32()), ("m130_prefill", W.layer_130m_prefill())):
        for nt in (1, threads):
            oracle.set_threads(nt)
            t, sc = _oracle_prefill(oracle, w)
            small["%s_%dthr" % (name, nt)] = {"tokens_per_s": t / sc, "seconds": sc, "threads": nt}
    oracle.set_threads(threads)
    cpu["small_prefills"] = small
    # decode: the first few of the 64 steps (conv, scan, norm per step), on all threads
    dwl = W.decode_batch()
    dsh = dwl.shape
    cp, sp = dwl.conv_pool.copy(), dwl.ssm_pool.copy()
    nsteps = 4
    t0 = time.perf_counter()
    for i, (x, z, dt) in enumerate(dwl.steps[:nsteps]):
        fresh = dwl.fresh if i == 0 else np.zeros_like(dwl.fresh)
        oa = np.zeros_like(x)
        assert oracle.conv1d(oa, x, dwl.conv_w, dwl.conv_b, cp, dwl.run_lengths, dwl.slots, fresh) == 0
        oy = np.zeros((x.shape[0], dsh.d_inner), dtype=x.dtype)
        assert oracle.scan(oy, oa, dt, dwl.a_log, dwl.dt_bias, dwl.D, sp, dwl.run_lengths, dwl.slots, fresh,
                           dsh.ngroups, decode=True) == 0
        oo = np.zeros_like(oy)
        assert oracle.gated_rmsnorm(oo, oy, z, dwl.norm_w, dsh.norm_groups, dsh.eps) == 0
    cpu["decode_us_per_step"] = 1e6 * (time.perf_counter() - t0) / nsteps
    cpu["decode_sample"] = "first %d of the 64 steps of 256 requests, %d threads" % (nsteps, threads)
    return cpu


if __name__ == "__main__":
    main()
