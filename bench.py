#!/usr/bin/env python3
"""Benchmark of the Q4 verify GEMM on one MI355X.

One step = one q4_gemm_verify call at M = 16 verify rows on the fused MLP
gate+up projection of the 27B target (N = 34816 outputs, K = 5120 inputs,
100,270,080 packed weight bytes), the shape the pages' model spends most of
its weight bytes on.  The same shape is also timed at M = 1 (one decode row)
for the M=16/M=1 time ratio.

Protocol (the prediction-first page's order: stamp, count bytes, predict,
warm up, measure):
  * stamp: device, architecture, CU count, software versions, UTC time;
  * algorithmic bytes per call = 9NK/16 (weights) + 2MK (x) + 4MN (y), and
    the floor time at the 8 TB/s HBM peak, printed before measuring;
  * weights are rotated over >= 1.2 GB of distinct copies so that neither the
    L2 nor the 256 MB Infinity Cache can serve a repeated read;
  * W warm-up steps, then K timed back-to-back steps between two HIP events
    on the launch stream, bracketed by device synchronisations; the mean per
    call is both the step time and the launch duration of the roofline
    figure (the kernel-trace profile of the same command must agree).

Output: one JSON line on stdout.  `value` is the effective bandwidth of the
M = 16 step (algorithmic bytes / mean step time, inputs resident in HBM).
Every timed block reports the mean over all its calls and the median and
minimum over five equal sub-blocks (an event between sub-blocks), and is
followed, outside the timed region, by a parity verdict: the prepared call
on weight copy 0 runs once more and all of its outputs are compared with
the CPU oracle (max err / (2e-3 sum|x w| + 1e-5), pass when <= 1).
Besides the step: the planar entry point q4_gemm_verify; gate+up and down at
M in {1, 2, 4, 8, 16} through each entry point (`m_sweep`); the small
256 x 512 shape's per-call latency (`tiny`); every projection shape at
M = 1, 16, 32 (`shapes`); the LM head's sampling epilogue, the Gated
DeltaNet commit and the tree attention; the 64-layer pass; and a streaming
read probe at the GEMM's sizes (`stream_read_by_size`).
`roofline.traffic` comes from the committed rocprofv3 counter summary when
that summary was taken of the current kernel source, else null.
`cpu_baseline` times the CPU oracle (test infrastructure, never tuned) on the
host cores: its `value` on the whole gate+up matrix at M = 16, and
`per_config` the small, gate+up, down and LM-head shapes at M = 1 and 16 and
the 64-layer pass as the sum over its shapes of count x time per call.
"""
from __future__ import annotations

import argparse
import datetime
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("Q4 verify GEMM effective HBM GB/s (% of peak) and M=16/M=1 time "
          "ratio")
HBM_PEAK_GBPS = 8000.0
WORKLOADS = {
    "gate_up": (34816, 5120),
    "down": (5120, 17408),
    "lm_head": (248320, 5120),
    "attn_in": (14336, 5120),
    "o_proj": (5120, 6144),
    "gdn_in": (16640, 5120),
}
KERNEL_SOURCE = os.path.join(ROOT, "speculative_verify_gemm_q4_amd", "csrc",
                             "q4verify_kernels.hip")
KERNEL_NAMES = {0: "gemm_verify_kernel", 1: "gemm_tiled_kernel",
                2: "gemm_resident_kernel", 3: "gemm_kslice_kernel"}
def counters_file(entry, shape, M):
    N, K = WORKLOADS[shape]
    return os.path.join(ROOT, "profiles",
                        f"gemm_{entry}_{shape}_{N}x{K}_M{M}_counters.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(M, N, K):
    return 9 * N * K // 16 + 2 * M * K + 4 * M * N


def kernel_source_hash(path=None):
    with open(path or KERNEL_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def stamp(torch):
    p = torch.cuda.get_device_properties(0)
    return {
        "device": p.name,
        "arch": getattr(p, "gcnArchName", ""),
        "cus": p.multi_processor_count,
        "hbm_gib": round(p.total_memory / 2 ** 30, 1),
        "torch": torch.__version__,
        "hip": getattr(torch.version, "hip", None),
        "host": platform.node(),
        "utc": datetime.datetime.now(datetime.timezone.utc).isoformat(
            timespec="seconds"),
    }


def load_traffic(entry, shape, M):
    """Per-launch HBM bytes from the committed counter summary of this
    entry point, shape and M, if it was taken of the current kernel
    source (else None)."""
    path = counters_file(entry, shape, M)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as fh:
            rec = next(json.loads(line) for line in fh
                       if line.strip().startswith("{"))
    except (StopIteration, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    got = [k.get("hbm_bytes_per_dispatch") for k in rec.get("kernels", {}).values()
           if k.get("hbm_bytes_per_dispatch")]
    return got[0] if len(got) == 1 else None


def cpu_baseline(torch, W, x16, N, K, budget_s):
    import oracle
    import synth
    threads = min(16, len(os.sched_getaffinity(0)))
    W_host = W.cpu().numpy()
    x_bits = synth.bf16_bits(x16)
    M = x16.shape[0]
    # bounded sample: whole row blocks of the matrix until ~budget_s of work
    rows = N
    t0 = time.perf_counter()
    done = 0
    runs = 0
    while True:
        _, _, _, used = oracle.gemm(x_bits, W_host, N, K, threads=threads)
        runs += 1
        done += alg_bytes(M, N, K)
        if time.perf_counter() - t0 >= budget_s or runs >= 20:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt / 1e9, 4), "unit": "GB/s",
            "cores": used, "kind": "oracle",
            "sample": f"whole {N}x{K} matrix at M={M}, {runs} run(s), "
                      f"{dt:.1f} s, fp64 accumulation, {used} threads",
            "s_per_call": round(dt / runs, 4), "rows": rows}


def rotated_tiled(torch, synth, q4, N, K, rotate_gb, stream0, dev,
                  keep_first=False):
    """Distinct tiled copies of an N x K matrix, >= rotate_gb in total (at
    least two), each generated planar and repacked; with keep_first, also
    the planar bytes of copy 0 on the host (for the parity check)."""
    wbytes = 9 * N * K // 16
    copies = max(2, math.ceil(rotate_gb * 1e9 / wbytes))
    out = []
    first = None
    for i in range(copies):
        W = synth.q4_weights(N, K, seed=0, stream=stream0 + i, device=dev)
        Wt = torch.empty_like(W)
        q4.q4_repack(W, Wt, N, K)
        out.append(Wt)
        if keep_first and i == 0:
            first = W.cpu().numpy()
        del W
    torch.cuda.synchronize()
    return (out, first) if keep_first else out


def raw_calls(torch, q4, entry, x, Ws, y, M, N, K, ws=None):
    """One prepared zero-argument call of the C entry point per weight copy:
    the binding's argument checks are done here once, so the timed loop pays
    only the ctypes call (about 1-2 us of host time, below every kernel's
    duration, so launches queue ahead of the GPU)."""
    import functools
    lib = q4.load()
    fn = getattr(lib, entry)
    stream = torch.cuda.current_stream().cuda_stream
    out = []
    for W in Ws:
        # validate once through the public binding (raises on misuse)
        if entry == "q4_gemm_verify_tiled_ws":
            q4.q4_gemm_verify_tiled_ws(x, W, y, M, N, K, ws)
            args = (x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K,
                    None if ws is None else ws.data_ptr(),
                    0 if ws is None else ws.numel(), stream)
        else:
            getattr(q4, entry)(x, W, y, M, N, K)
            args = (x.data_ptr(), W.data_ptr(), y.data_ptr(), M, N, K, stream)
        f = functools.partial(fn, *args)
        if f() != 0:
            raise RuntimeError(f"{entry} failed on a prepared call")
        out.append(f)
    torch.cuda.synchronize()
    return out


# Least untimed warm-up per timed block.  Right after a repack, a block of
# 200 gate+up calls that followed 200 warm-up calls (4.5 ms) measured 23.0 us
# per call and every later block 20.6-21.0 us: the clocks take longer than
# that to settle under a sustained load.
MIN_WARM_S = 0.05


SUB_BLOCKS = 5


def time_stats(torch, fns, steps, warmup):
    """Per-call times of `steps` back-to-back calls (rotating over fns) on
    the launch stream, after at least `warmup` untimed calls and at least
    MIN_WARM_S seconds of them.  HIP events are recorded between
    SUB_BLOCKS equal sub-blocks of the timed calls (one event per sub-block,
    so the stream stays full): `mean_ms` is first to last event over all
    calls, `median_ms` and `min_ms` are over the sub-blocks' means."""
    n = len(fns)
    done = 0
    t_warm = time.perf_counter()
    while True:
        for _ in range(max(warmup, 1)):
            fns[done % n]()
            done += 1
        torch.cuda.synchronize()
        if done >= warmup and time.perf_counter() - t_warm >= MIN_WARM_S:
            break
    warmup = done
    nb = max(1, min(SUB_BLOCKS, steps))
    per = [steps // nb + (1 if b < steps % nb else 0) for b in range(nb)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    i = 0
    for b in range(nb):
        for _ in range(per[b]):
            fns[(warmup + i) % n]()
            i += 1
        evs[b + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    blocks = sorted(evs[b].elapsed_time(evs[b + 1]) / per[b] for b in range(nb))
    return {"mean_ms": evs[0].elapsed_time(evs[nb]) / steps,
            "median_ms": blocks[nb // 2] if nb % 2 else
            0.5 * (blocks[nb // 2 - 1] + blocks[nb // 2]),
            "min_ms": blocks[0], "wall_ms": wall, "sub_blocks": nb}


def time_raw(torch, fns, steps, warmup):
    """(mean ms per call, host wall ms per call) of time_stats."""
    st = time_stats(torch, fns, steps, warmup)
    return st["mean_ms"], st["wall_ms"]


def us3(st):
    """mean / median / min of a time_stats result, in us."""
    return {"us_mean": round(st["mean_ms"] * 1e3, 3),
            "us_median": round(st["median_ms"] * 1e3, 3),
            "us_min": round(st["min_ms"] * 1e3, 3)}


REL, ABS = 2e-3, 1e-5   # |y - y64| <= REL * sum|x w| + ABS per output


def sig3(v):
    """Three significant digits (the parity ratios are far below 1)."""
    return float(f"{v:.3g}")


def parity(torch, synth, x, y, W_host, N, K, threads):
    """Largest err/bound of every output of y against the oracle (fp64 over
    the dequantized planar bytes W_host), outside the timed region."""
    import numpy as np
    import oracle
    torch.cuda.synchronize()
    _, y64, a64, _ = oracle.gemm(synth.bf16_bits(x), W_host, N, K,
                                 threads=threads)
    got = y.cpu().numpy().astype(np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - y64) / (REL * a64 + ABS)))


ENTRY_LAYOUT = {"q4_gemm_verify": "planar", "q4_gemm_verify_tiled": "tiled",
                "q4_gemm_verify_tiled_ws": "tiled",
                "q4_gemm_verify_tiled_dot": "tiled"}


def plan_brief(q4, entry, M, N, K):
    if entry == "q4_gemm_verify":
        p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_PLANAR)
    elif entry in ("q4_gemm_verify_tiled", "q4_gemm_verify_tiled_dot"):
        p = q4.q4_gemm_verify_plan(M, N, K, q4.LAYOUT_TILED16)
    else:
        p = q4.q4_gemm_verify_tiled_ws_plan(M, N, K)
    return {"kernel": KERNEL_NAMES[p["kernel"]], "grid": p["grid"],
            "waves": p["block"] // 64, "k_parts": p["k_parts"],
            "k_seq_parts": p["k_seq_parts"], "workspace_bytes":
            p["workspace_bytes"]}


def measure_sweep(torch, synth, q4, name, Ms, entries, steps, warmup,
                  rotate_gb, dev, threads):
    """One projection shape at every M of `Ms` through each entry point of
    `entries`, over rotated weight copies (planar copies for
    q4_gemm_verify, their repacks for the tiled entry points).  Per (entry,
    M): mean / median / min us per call, effective GB/s, fraction of the
    HBM peak, and the parity verdict: after the timed block the prepared
    call on copy 0 runs once more and every output is compared with the
    oracle on that copy's planar bytes (max err/bound, pass if <= 1)."""
    N, K = WORKLOADS[name]
    wbytes = 9 * N * K // 16
    copies = max(2, math.ceil(rotate_gb * 1e9 / wbytes))
    Ws = [synth.q4_weights(N, K, seed=0, stream=7000 + i, device=dev)
          for i in range(copies)]
    Wts = []
    for W in Ws:
        Wt = torch.empty_like(W)
        q4.q4_repack(W, Wt, N, K)
        Wts.append(Wt)
    torch.cuda.synchronize()
    W0 = Ws[0].cpu().numpy()
    xs = synth.activations(max(Ms), K, seed=0, stream=7100, device=dev)
    out = {"N": N, "K": K, "weight_bytes": wbytes, "copies": copies,
           "parity_rule": f"|y - y64| <= {REL} sum|x w| + {ABS}"}
    n = max(20, min(steps, int(20e3 / (wbytes / 5e6))))
    for entry in entries:
        rec = out.setdefault(entry, {})
        for M in Ms:
            x = xs[:M].contiguous()
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            ws = (q4.workspace_for(M, N, K, dev)
                  if entry == "q4_gemm_verify_tiled_ws" else None)
            fns = raw_calls(torch, q4, entry, x,
                            Ws if ENTRY_LAYOUT[entry] == "planar" else Wts,
                            y, M, N, K, ws)
            st = time_stats(torch, fns, n, warmup)
            fns[0]()
            ratio = parity(torch, synth, x, y, W0, N, K, threads)
            b = alg_bytes(M, N, K)
            gbps = b / (st["mean_ms"] * 1e-3) / 1e9
            r = dict(us3(st), gbps=round(gbps, 1),
                     frac_of_peak=round(gbps / HBM_PEAK_GBPS, 4),
                     parity_max_err_over_bound=sig3(ratio),
                     parity="pass" if ratio <= 1.0 else "FAIL",
                     plan=plan_brief(q4, entry, M, N, K))
            rec[str(M)] = r
            log(f"sweep {name} {entry} M={M}: {r}")
        m1 = rec[str(min(Ms))]["us_mean"]
        rec["ratio_m16_m1"] = (round(rec["16"]["us_mean"] / m1, 4)
                               if "16" in rec else None)
    del Ws, Wts
    torch.cuda.empty_cache()
    return out


def measure_tiny(torch, synth, q4, steps, warmup, dev, threads):
    """The small shape (N = 256, K = 512, M in {1, 4}): its 73,728 weight
    bytes stay in the caches, so this is the per-call latency of a launch
    (no rotation), through the planar and the tiled entry points, with the
    parity verdict of the timed outputs."""
    N, K = 256, 512
    W = synth.q4_weights(N, K, seed=0, device=dev)
    Wt = torch.empty_like(W)
    q4.q4_repack(W, Wt, N, K)
    W0 = W.cpu().numpy()
    out = {"N": N, "K": K, "weight_bytes": 9 * N * K // 16}
    for M in (1, 4):
        x = synth.activations(M, K, seed=0, stream=1, device=dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        for entry, Wx in (("q4_gemm_verify", W), ("q4_gemm_verify_tiled", Wt)):
            fns = raw_calls(torch, q4, entry, x, [Wx], y, M, N, K)
            st = time_stats(torch, fns, steps, warmup)
            ratio = parity(torch, synth, x, y, W0, N, K, threads)
            out.setdefault(entry, {})[str(M)] = dict(
                us3(st), parity_max_err_over_bound=sig3(ratio),
                parity="pass" if ratio <= 1.0 else "FAIL")
    log(f"tiny: {out}")
    return out


def measure_stream_probe(torch, synth, q4, sizes, rotate_gb, dev):
    """q4_stream_read over rotated buffers of each size (bytes), the
    streaming read rate the GEMM is set against: best GB/s per size."""
    out = {}
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    lib = q4.load()
    import functools
    stream = torch.cuda.current_stream().cuda_stream
    for nbytes in sizes:
        copies = max(2, math.ceil(rotate_gb * 1e9 / nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev)
                for _ in range(copies)]
        for b in bufs:
            b.fill_(1)
        fns = [functools.partial(lib.q4_stream_read, b.data_ptr(), nbytes,
                                 sink.data_ptr(), stream) for b in bufs]
        st = time_stats(torch, fns, max(20, min(200, int(4e9 / nbytes))), 10)
        out[str(nbytes)] = {"us_mean": round(st["mean_ms"] * 1e3, 3),
                            "us_min": round(st["min_ms"] * 1e3, 3),
                            "gbps": round(nbytes / (st["mean_ms"] * 1e-3)
                                          / 1e9, 1)}
        del bufs
    torch.cuda.empty_cache()
    log(f"stream read probe: {out}")
    return out


def cpu_configs(torch, synth, dev, budget_s):
    """The CPU oracle (test infrastructure, as it stands) on the host cores:
    each of the small, gate+up, down and LM-head shapes at M = 1 and 16
    (whole matrices), and every other projection of the 64-layer pass at
    M = 16, repeated until about budget_s seconds in all; the pass figure
    is per shape x its count per pass."""
    import oracle
    threads = min(16, len(os.sched_getaffinity(0)))
    shapes = [("tiny", (256, 512))] + [(n, WORKLOADS[n]) for n in
                                       ("gate_up", "down", "lm_head",
                                        "attn_in", "gdn_in", "o_proj")]
    res = {}
    used_max = 0
    per_call = {}
    t_all = time.perf_counter()
    for name, (N, K) in shapes:
        W = synth.q4_weights(N, K, seed=0, stream=1, device=dev).cpu().numpy()
        Ms = (1, 16) if name in ("tiny", "gate_up", "down", "lm_head") else (16,)
        for M in Ms:
            x = synth.activations(M, K, seed=0, stream=2, device=dev)
            xb = synth.bf16_bits(x)
            runs, t0 = 0, time.perf_counter()
            while True:
                _, _, _, used = oracle.gemm(xb, W, N, K, threads=threads)
                runs += 1
                if time.perf_counter() - t0 >= budget_s / 12 or runs >= 50:
                    break
            dt = (time.perf_counter() - t0) / runs
            used_max = max(used_max, used)
            per_call[(name, M)] = dt
            res[f"{name}_M{M}"] = {
                "N": N, "K": K, "M": M, "s_per_call": round(dt, 5),
                "gbps": round(alg_bytes(M, N, K) / dt / 1e9, 4), "runs": runs}
        del W
    counts = {}
    for name, _ in pass_calls():
        counts[name] = counts.get(name, 0) + 1
    pass_s = sum(c * per_call[(n, 16)] for n, c in counts.items())
    pass_b = sum(c * alg_bytes(16, *WORKLOADS[n]) for n, c in counts.items())
    res["full_pass_M16"] = {"calls": sum(counts.values()), "counts": counts,
                            "s_per_pass": round(pass_s, 3),
                            "gbps": round(pass_b / pass_s / 1e9, 4),
                            "how": "sum over shapes of count x s_per_call"}
    res["threads"] = used_max
    res["seconds"] = round(time.perf_counter() - t_all, 1)
    log(f"cpu oracle per config: {res}")
    return res


def measure_shapes(torch, synth, q4, names, steps, warmup, rotate_gb, dev):
    """Every projection shape of the 27B pass at M = 16 and M = 1 (order
    16, 1, 16), each over its own rotated copies, through the workspace
    entry point called directly (prepared ctypes calls, back to back)."""
    res = {}
    threads = min(16, len(os.sched_getaffinity(0)))
    for i, name in enumerate(names):
        N, K = WORKLOADS[name]
        Wts, W0 = rotated_tiled(torch, synth, q4, N, K, rotate_gb,
                                1000 * (i + 1), dev, keep_first=True)
        x16 = synth.activations(16, K, seed=0, stream=100 + i, device=dev)
        x1 = x16[:1].contiguous()
        y16 = torch.empty((16, N), dtype=torch.float32, device=dev)
        y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
        ws = q4.workspace_for(16, N, K, dev)
        f16 = raw_calls(torch, q4, "q4_gemm_verify_tiled_ws", x16, Wts, y16,
                        16, N, K, ws)
        f1 = raw_calls(torch, q4, "q4_gemm_verify_tiled_ws", x1, Wts, y1,
                       1, N, K, ws)
        n = max(20, min(steps, int(20e3 / (9 * N * K / 16 / 5e6))))
        sa = time_stats(torch, f16, n, warmup)
        f16[0]()
        par16 = parity(torch, synth, x16, y16, W0, N, K, threads)
        sb = time_stats(torch, f1, n, warmup)
        f1[0]()
        par1 = parity(torch, synth, x1, y1, W0, N, K, threads)
        sc = time_stats(torch, f16, n, warmup)
        a, b, c = sa["mean_ms"], sb["mean_ms"], sc["mean_ms"]
        # 32 rows (two MFMA row tiles; K split into parts as needed)
        x32 = synth.activations(32, K, seed=0, stream=400 + i, device=dev)
        y32 = torch.empty((32, N), dtype=torch.float32, device=dev)
        ws32 = q4.workspace_for(32, N, K, dev)
        f32 = raw_calls(torch, q4, "q4_gemm_verify_tiled_ws", x32, Wts, y32,
                        32, N, K, ws32)
        sd = time_stats(torch, f32, n, warmup)
        d = sd["mean_ms"]
        f32[0]()
        par32 = parity(torch, synth, x32, y32, W0, N, K, threads)
        p32 = q4.q4_gemm_verify_tiled_ws_plan(32, N, K)
        m16 = 0.5 * (a + c)
        plan = q4.q4_gemm_verify_tiled_ws_plan(16, N, K)
        rec = {"N": N, "K": K, "weight_bytes": 9 * N * K // 16,
               "copies": len(Wts), "steps": n,
               "kernel": KERNEL_NAMES[plan["kernel"]],
               "k_parts": plan["k_parts"],
               "us_m1": round(b * 1e3, 3), "us_m16": round(m16 * 1e3, 3),
               "gbps_m1": round(alg_bytes(1, N, K) / (b * 1e-3) / 1e9, 1),
               "gbps_m16": round(alg_bytes(16, N, K) / (m16 * 1e-3) / 1e9, 1),
               "ratio_m16_m1": round(m16 / b, 4)}
        rec["frac_m1"] = round(rec["gbps_m1"] / HBM_PEAK_GBPS, 4)
        rec["frac_m16"] = round(rec["gbps_m16"] / HBM_PEAK_GBPS, 4)
        rec["us_m32"] = round(d * 1e3, 3)
        rec["gbps_m32"] = round(alg_bytes(32, N, K) / (d * 1e-3) / 1e9, 1)
        rec["ratio_m32_m1"] = round(d / b, 4)
        rec["k_parts_m32"] = p32["k_parts"]
        rec["blocks_us"] = {"m16": us3(sa), "m1": us3(sb), "m16_again": us3(sc),
                            "m32": us3(sd)}
        worst = max(par16, par1, par32)
        rec["parity_max_err_over_bound"] = {"m16": sig3(par16),
                                            "m1": sig3(par1),
                                            "m32": sig3(par32)}
        rec["parity"] = "pass" if worst <= 1.0 else "FAIL"
        log(f"shape {name}: {rec}")
        res[name] = rec
        del Wts, x16, x1, y16, y1, ws, x32, y32, ws32
        torch.cuda.empty_cache()
    return res


# The 27B model's projection list: 16 attention and 48 gated-DeltaNet layers,
# each with its input and output projection and the MLP (gate+up, down), and
# the LM head called twice (draft readout, then verify) on the same weights.
def measure_verify_sample(torch, synth, q4, dev, steps, warmup):
    """The sampling epilogue on the LM head's logits (16 rows x 248320,
    top_k 20, top_p 0.95, temperature 1, 16 draft candidates per row), alone
    and after the LM head GEMM (one verify step's tail), as prepared C-ABI
    calls back to back."""
    import ctypes
    import functools
    from speculative_verify_gemm_q4_amd._lib import _SampleParams
    M, (V, K) = 16, WORKLOADS["lm_head"]
    lib = q4.load()
    gen = torch.Generator(device=dev).manual_seed(0)
    logits = torch.randn((M, V), generator=gen, device=dev) * 3.0
    inp = synth.sample_inputs(M, V, 16, seed=0, device=dev)
    out = q4.verify_sample(logits, 1.0, 0.95, 20, inp["draft_tok"],
                           inp["draft_idx"], inp["draft_q"], inp["u"],
                           inp["v"])
    ws = torch.empty(q4.q4_verify_sample_workspace(M, V), dtype=torch.uint8,
                     device=dev)
    prm = _SampleParams(1.0, 0.95, 20, 16)
    stream = torch.cuda.current_stream().cuda_stream
    args = [logits.data_ptr(), M, V, ctypes.byref(prm)] + [
        t.data_ptr() for t in (inp["draft_tok"], inp["draft_idx"],
                               inp["draft_q"], inp["u"], inp["v"],
                               out["top_idx"], out["top_val"],
                               out["top_prob"], out["greedy"], out["accept"],
                               out["token"])] + [ws.data_ptr(), ws.numel(),
                                                 stream]
    f = functools.partial(lib.q4_verify_sample, *args)
    if f() != 0:
        raise RuntimeError("q4_verify_sample failed")
    ms, _ = time_raw(torch, [f], steps, warmup)
    rec = {"M": M, "V": V, "top_k": 20, "draft_k": 16,
           "us": round(ms * 1e3, 3), "logits_bytes": M * V * 4,
           "gbps": round(M * V * 4 / (ms * 1e-3) / 1e9, 1)}
    # the LM head GEMM writing those logits, then the epilogue
    Wts = rotated_tiled(torch, synth, q4, V, K, 1.2, 9000, dev)
    x = synth.activations(M, K, seed=0, stream=300, device=dev)
    g = raw_calls(torch, q4, "q4_gemm_verify_tiled", x, Wts, logits, M, V, K)
    steps2 = max(10, steps // 8)
    ms_g, _ = time_raw(torch, g, steps2, max(2, warmup // 8))
    both = [lambda gi=gi: (gi(), f()) for gi in g]
    ms_b, _ = time_raw(torch, both, steps2, max(2, warmup // 8))
    rec["lm_head_us"] = round(ms_g * 1e3, 3)
    rec["lm_head_plus_sample_us"] = round(ms_b * 1e3, 3)
    # the same step with the epilogue fused into the LM head (the logits
    # never written): q4_gemm_verify_sample on the same weights and rows
    fws = torch.empty(q4.q4_gemm_verify_sample_workspace(M, V, K),
                      dtype=torch.uint8, device=dev)
    fargs = lambda Wt: [x.data_ptr(), Wt.data_ptr(), M, V, K,
                        ctypes.byref(prm)] + [
        t.data_ptr() for t in (inp["draft_tok"], inp["draft_idx"],
                               inp["draft_q"], inp["u"], inp["v"],
                               out["top_idx"], out["top_val"],
                               out["top_prob"], out["greedy"], out["accept"],
                               out["token"])] + [fws.data_ptr(), fws.numel(),
                                                 stream]
    fused = [functools.partial(lib.q4_gemm_verify_sample, *fargs(Wt))
             for Wt in Wts]
    if any(fn() != 0 for fn in fused):
        raise RuntimeError("q4_gemm_verify_sample failed")
    ms_f, _ = time_raw(torch, fused, steps2, max(2, warmup // 8))
    rec["fused_us"] = round(ms_f * 1e3, 3)
    rec["fused_over_lm_head"] = round(ms_f / ms_g, 4)
    rec["candidates_bytes"] = fws.numel()
    log(f"verify sample: {rec}")
    del Wts
    torch.cuda.empty_cache()
    return rec


GDN_SHAPE = {"layers": 48, "heads": 48, "key_heads": 16, "dv": 128,
             "dk": 128, "tree_nodes": 16}


def gdn_alg_bytes(L, H, Hk, dv, dk, n):
    """Unique bytes of one commit: the state read and written, the accepted
    nodes' keys, values, gates and strengths, the path and the count."""
    return (2 * L * H * dv * dk * 4 + L * n * (Hk * dk + H * dv + 2 * H) * 4
            + (n + 1) * 4)


def measure_gdn_commit(torch, synth, q4, dev, steps, warmup):
    """The Gated DeltaNet state commit of one step: 48 layers x 48 value
    heads x 128 x 128 fp32 (147 MiB read and written), a 16-node tree, for
    accepted paths of 1, 7 and 16 nodes.  Three state copies (453 MB, more
    than the 256 MB last-level cache) are rotated so that each call streams
    its state from HBM.  Prepared C-ABI calls back to back, HIP events on the
    launch stream."""
    import functools
    g = GDN_SHAPE
    L, H, Hk, dv, dk, M = (g["layers"], g["heads"], g["key_heads"], g["dv"],
                           g["dk"], g["tree_nodes"])
    lib = q4.load()
    inp = synth.gdn_inputs(L, H, Hk, M, dv=dv, dk=dk, seed=0, device=dev)
    states = [inp["S"]] + [inp["S"].clone() for _ in range(2)]
    stream = torch.cuda.current_stream().cuda_stream
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {"shape": dict(g), "copies": len(states), "paths": []}
    for n in (1, 7, 16):
        path = torch.tensor(list(range(n)) + [0] * (M - n), dtype=torch.int32,
                            device=dev)
        cnt = torch.tensor([n], dtype=torch.int32, device=dev)
        fns = [functools.partial(
            lib.q4_gdn_commit, S.data_ptr(), L, H, Hk, dv, dk, M,
            inp["k"].data_ptr(), inp["v"].data_ptr(),
            inp["alpha"].data_ptr(), inp["beta"].data_ptr(), path.data_ptr(),
            cnt.data_ptr(), status.data_ptr(), stream) for S in states]
        if any(f() != 0 for f in fns):
            raise RuntimeError("q4_gdn_commit failed")
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError("q4_gdn_commit rejected its path")
        ms, _ = time_raw(torch, fns, steps, warmup)
        nb = gdn_alg_bytes(L, H, Hk, dv, dk, n)
        gbps = nb / (ms * 1e-3) / 1e9
        out["paths"].append({"accepted": n, "us": round(ms * 1e3, 3),
                             "alg_bytes": nb, "gbps": round(gbps, 1),
                             "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)})
    # every tree node's output of one layer, from that layer's state (one
    # of the 3 x 48 layer states in turn, so that each call reads from HBM)
    par = torch.tensor(inp["parent"], dtype=torch.int32, device=dev)
    outs = torch.empty((M, H, dv), dtype=torch.float32, device=dev)
    lstates = [S[l] for S in states for l in range(L)]
    fns = [functools.partial(
        lib.q4_gdn_tree_out, Sl.data_ptr(), H, Hk, dv, dk, M,
        inp["q"][0].data_ptr(), inp["k"][0].data_ptr(), inp["v"][0].data_ptr(),
        inp["alpha"][0].data_ptr(), inp["beta"][0].data_ptr(), par.data_ptr(),
        outs.data_ptr(), status.data_ptr(), stream) for Sl in lstates]
    if any(f() != 0 for f in fns[:1]):
        raise RuntimeError("q4_gdn_tree_out failed")
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("q4_gdn_tree_out rejected its tree")
    ms, _ = time_raw(torch, fns, steps, warmup)
    # the layer's state, the nodes' queries, keys, values, gates and parents,
    # and the outputs
    nb = (H * dv * dk * 4 + 2 * M * Hk * dk * 4 + M * H * dv * 4
          + 2 * M * H * 4 + M * 4 + M * H * dv * 4)
    gbps = nb / (ms * 1e-3) / 1e9
    out["tree_out"] = {"layer_states": len(lstates), "tree_nodes": M,
                       "us": round(ms * 1e3, 3), "alg_bytes": nb,
                       "gbps": round(gbps, 1),
                       "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    log(f"gdn commit: {out}")
    del states, inp, lstates, fns
    torch.cuda.empty_cache()
    return out


ATTN_SHAPE = {"query_heads": 24, "kv_heads": 4, "head_dim": 256,
              "tree_nodes": 16, "page_tokens": 32}


def attn_alg_bytes(M, Hq, Hkv, D, ctx):
    """Unique bytes of one tree-attention layer: the int8 keys and values of
    every page touched with their fp32 scales, the bf16 queries, the page
    table and ancestor sets, and the fp32 output."""
    pages = (ctx + M + 31) // 32
    return (pages * Hkv * (2 * 32 * D + 2 * 32 * 4) + M * Hq * D * 2
            + pages * 4 + M * 4 + M * Hq * D * 4)


def measure_tree_attn(torch, synth, q4, dev, steps, warmup):
    """Tree-verify attention of one layer (24 query heads over 4 KV heads of
    256, 16 tree nodes) at 4K and 32K tokens of context, the default split,
    as prepared C-ABI calls back to back (the KV pages of one layer are
    read per call; at 32K they are 68 MB, more than a quarter of the
    last-level cache, and two caches are rotated)."""
    import functools
    g = ATTN_SHAPE
    M, Hq, Hkv, D = g["tree_nodes"], g["query_heads"], g["kv_heads"], g["head_dim"]
    lib = q4.load()
    stream = torch.cuda.current_stream().cuda_stream
    out = {"shape": dict(g), "contexts": []}
    for ctx in (4096, 32768):
        caches = [synth.attn_inputs(M, Hq, Hkv, ctx, seed=0, stream=i,
                                    device=dev) for i in range(2)]
        s, nws = q4.q4_tree_attn_plan(M, Hq, Hkv, ctx)
        o = torch.empty((M, Hq, D), dtype=torch.float32, device=dev)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        fns = [functools.partial(
            lib.q4_tree_attn, c["q"].data_ptr(), M, Hq, Hkv, D,
            c["k_pages"].data_ptr(), c["v_pages"].data_ptr(),
            c["k_scale"].data_ptr(), c["v_scale"].data_ptr(),
            c["page_table"].data_ptr(), int(c["k_pages"].shape[0]), ctx,
            c["anc"].data_ptr(), 1.0 / 16.0, o.data_ptr(), 0, ws.data_ptr(),
            ws.numel(), None, stream) for c in caches]
        if any(f() != 0 for f in fns):
            raise RuntimeError("q4_tree_attn failed")
        ms, _ = time_raw(torch, fns, steps, warmup)
        nb = attn_alg_bytes(M, Hq, Hkv, D, ctx)
        gbps = nb / (ms * 1e-3) / 1e9
        out["contexts"].append({"ctx": ctx, "splits": s, "us": round(ms * 1e3, 3),
                                "alg_bytes": nb, "workspace_bytes": nws,
                                "gbps": round(gbps, 1),
                                "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        del caches
    log(f"tree attention: {out}")
    torch.cuda.empty_cache()
    return out


def pass_calls():
    calls = []
    for layer in range(64):
        attn = layer % 4 == 3            # 16 of 64 layers are attention
        calls.append(("attn_in" if attn else "gdn_in", layer))
        calls.append(("o_proj", layer))
        calls.append(("gate_up", layer))
        calls.append(("down", layer))
    calls.append(("lm_head", 0))
    calls.append(("lm_head", 0))
    return calls


def measure_full_pass(torch, synth, q4, reps, dev):
    """One 64-layer pass of every projection (distinct weights per layer),
    captured once per M as a HIP graph and replayed; activations are not
    chained between calls (only the projections are on the path)."""
    calls = pass_calls()
    weights = {}
    for name, layer in calls:
        if (name, layer) in weights:
            continue
        N, K = WORKLOADS[name]
        W = synth.q4_weights(N, K, seed=0, stream=50000 + 16 * layer +
                             sorted(WORKLOADS).index(name), device=dev)
        Wt = torch.empty_like(W)
        q4.q4_repack(W, Wt, N, K)
        weights[(name, layer)] = Wt
        del W
    torch.cuda.synchronize()
    wbytes = sum(9 * WORKLOADS[n][0] * WORKLOADS[n][1] // 16 for n, _ in calls)
    xs = {K: synth.activations(32, K, seed=0, stream=200 + K, device=dev)
          for K in {k for _, k in WORKLOADS.values()}}
    ys = {n: torch.empty((32, N), dtype=torch.float32, device=dev)
          for n, (N, _) in WORKLOADS.items()}
    # calls run in order on one stream, so one workspace serves them all
    need = max(q4.q4_gemm_verify_tiled_ws_plan(32, N, K)["workspace_bytes"]
               for N, K in WORKLOADS.values())
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    out = {"calls": len(calls), "weight_bytes": wbytes,
           "entry_point": "q4_gemm_verify_tiled_ws (K > 5120 split across "
                          "workgroups)",
           "graph": "one HIP graph per M, replayed back to back"}
    graphs = {}
    for M in (16, 1, 32):
        x_m = {K: v[:M].contiguous() for K, v in xs.items()}

        def run_pass(M=M, x_m=x_m):
            for name, layer in calls:
                N, K = WORKLOADS[name]
                q4.q4_gemm_verify_tiled_ws(x_m[K], weights[(name, layer)],
                                           ys[name][:M], M, N, K, ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_pass()                  # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_pass()
        torch.cuda.synchronize()
        graphs[M] = (g, run_pass)

    def timed(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for M in (16, 1, 16, 32):
        g, run_pass = graphs[M]
        ms = timed(g.replay, reps)
        key = f"M={M}"
        b = sum(alg_bytes(M, *WORKLOADS[n]) for n, _ in calls)
        rec = out.setdefault(key, {"alg_bytes": b, "ms": []})
        rec["ms"].append(ms)
    import functools
    lib = q4.load()
    stream = torch.cuda.current_stream().cuda_stream
    for M in (16, 1, 32):
        rec = out[f"M={M}"]
        ms = sum(rec["ms"]) / len(rec["ms"])
        rec["ms"] = round(ms, 4)
        rec["gbps"] = round(rec["alg_bytes"] / (ms * 1e-3) / 1e9, 1)
        rec["frac_of_peak"] = round(rec["gbps"] / HBM_PEAK_GBPS, 4)
        x_m = {K: v[:M].contiguous() for K, v in xs.items()}
        fns = [functools.partial(
            lib.q4_gemm_verify_tiled_ws, x_m[WORKLOADS[n][1]].data_ptr(),
            weights[(n, layer)].data_ptr(), ys[n].data_ptr(), M,
            WORKLOADS[n][0], WORKLOADS[n][1], ws.data_ptr(), ws.numel(),
            stream) for n, layer in calls]

        bad = [st for st in (f() for f in fns) if st != 0]
        if bad:
            raise RuntimeError(f"q4_gemm_verify_tiled_ws returned {bad[0]}")

        def eager(fns=fns):
            for f in fns:
                f()
        rec["eager_ms"] = round(timed(eager, max(2, reps // 2)), 4)
        rec["eager"] = ("the same 258 calls launched directly "
                        "(prepared C-ABI calls)")
    out["ratio_m16_m1"] = round(out["M=16"]["ms"] / out["M=1"]["ms"], 4)
    out["ratio_m32_m1"] = round(out["M=32"]["ms"] / out["M=1"]["ms"], 4)
    log(f"full pass: {out}")
    del weights, graphs
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ profiling aids
#
# rocprofv3 runs a program after `--`; these modes give it one kernel to look
# at (`--repeat`), and turn its CSV output into the short text summaries kept
# with the sources (`--summarize-trace`, `--summarize-pmc`).

SIMDS = 1024            # 256 CUs x 4 SIMDs
CLOCK_GHZ = 2.4         # peak engine clock, for busy fractions


def repeat_mode(spec, copy_mb):
    """ENTRY:SHAPE:M:REPS -- REPS prepared calls of one entry point on one
    projection shape over rotated weight copies (>= 1.2 GB), for a counter
    or trace pass, after three q4_stream_copy calls over copy_mb MiB (the
    known traffic the byte counters are scaled by) when copy_mb > 0; the
    last call's outputs are checked against the oracle when the run is
    short enough (M * N * K <= 2^34)."""
    import torch
    import synth
    import speculative_verify_gemm_q4_amd as q4
    entry, shape, M, reps = spec.split(":")
    M, reps = int(M), int(reps)
    if entry in ("attn", "fused", "sample"):
        return repeat_other(entry, shape, M, reps)
    entry = {"planar": "q4_gemm_verify", "tiled": "q4_gemm_verify_tiled",
             "ws": "q4_gemm_verify_tiled_ws",
             "dot": "q4_gemm_verify_tiled_dot"}.get(entry, entry)
    N, K = WORKLOADS[shape]
    dev = torch.device("cuda:0")
    q4.load()
    if copy_mb:
        nb = copy_mb * 2 ** 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(3):
            q4.q4_stream_copy(src, dst, nb)
        torch.cuda.synchronize()
        del src, dst
    copies = max(2, math.ceil(1.2e9 / (9 * N * K // 16)))
    Ws = [synth.q4_weights(N, K, seed=0, stream=i, device=dev)
          for i in range(copies)]
    if ENTRY_LAYOUT[entry] == "tiled":
        Wts = []
        for W in Ws:
            Wt = torch.empty_like(W)
            q4.q4_repack(W, Wt, N, K)
            Wts.append(Wt)
    else:
        Wts = Ws
    x = synth.activations(M, K, seed=0, stream=1, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = (q4.workspace_for(M, N, K, dev)
          if entry == "q4_gemm_verify_tiled_ws" else None)
    fns = raw_calls(torch, q4, entry, x, Wts, y, M, N, K, ws)
    # 0.1 s of calls first, so that the clocks have settled
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.1:
        for _ in range(20):
            fns[i % len(fns)]()
            i += 1
        torch.cuda.synchronize()
    for i in range(reps):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    fns[0]()
    if M * N * K <= 2 ** 34:
        r = parity(torch, synth, x, y, Ws[0].cpu().numpy(), N, K,
                   min(16, len(os.sched_getaffinity(0))))
        print(f"parity max err/bound {r:.3g}", flush=True)
    print(f"done {entry} {shape} M={M} reps={reps}", flush=True)


def repeat_other(entry, shape, M, reps):
    """Profiling aid for the steps beside the GEMM: `attn:CTX:M:REPS` runs
    the tree-verify attention layer of measure_tree_attn at CTX tokens of
    context (two caches rotated), `fused:lm_head:16:REPS` the LM head with
    the sampling epilogue fused in (rotated weights), `sample:lm_head:16:REPS`
    the standalone epilogue on the LM head's logits (two logit arrays
    rotated), REPS prepared calls each after 0.1 s of warm-up."""
    import ctypes
    import functools
    import torch
    import synth
    import speculative_verify_gemm_q4_amd as q4
    dev = torch.device("cuda:0")
    lib = q4.load()
    stream = torch.cuda.current_stream().cuda_stream
    if entry == "attn":
        g = ATTN_SHAPE
        Hq, Hkv, D = g["query_heads"], g["kv_heads"], g["head_dim"]
        ctx = int(shape)
        caches = [synth.attn_inputs(M, Hq, Hkv, ctx, seed=0, stream=i,
                                    device=dev) for i in range(2)]
        _, nws = q4.q4_tree_attn_plan(M, Hq, Hkv, ctx)
        o = torch.empty((M, Hq, D), dtype=torch.float32, device=dev)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
        fns = [functools.partial(
            lib.q4_tree_attn, c["q"].data_ptr(), M, Hq, Hkv, D,
            c["k_pages"].data_ptr(), c["v_pages"].data_ptr(),
            c["k_scale"].data_ptr(), c["v_scale"].data_ptr(),
            c["page_table"].data_ptr(), int(c["k_pages"].shape[0]), ctx,
            c["anc"].data_ptr(), 1.0 / 16.0, o.data_ptr(), 0, ws.data_ptr(),
            ws.numel(), None, stream) for c in caches]
    elif entry == "sample":
        from speculative_verify_gemm_q4_amd._lib import _SampleParams
        V, _ = WORKLOADS[shape]
        gen = torch.Generator(device=dev).manual_seed(0)
        logits = [torch.randn((M, V), generator=gen, device=dev) * 3.0
                  for _ in range(2)]
        inp = synth.sample_inputs(M, V, 16, seed=0, device=dev)
        out = {k: torch.empty(s, dtype=t, device=dev) for k, s, t in (
            ("top_idx", (M, 20), torch.int32), ("top_val", (M, 20), torch.float32),
            ("top_prob", (M, 20), torch.float32), ("greedy", (M,), torch.int32),
            ("accept", (M,), torch.int32), ("token", (M,), torch.int32))}
        prm = _SampleParams(1.0, 0.95, 20, 16)
        sws = torch.empty(q4.q4_verify_sample_workspace(M, V), dtype=torch.uint8,
                          device=dev)
        fns = [functools.partial(
            lib.q4_verify_sample, lg.data_ptr(), M, V, ctypes.byref(prm),
            *[inp[k].data_ptr() for k in (
                "draft_tok", "draft_idx", "draft_q", "u", "v")],
            *[out[k].data_ptr() for k in (
                "top_idx", "top_val", "top_prob", "greedy", "accept", "token")],
            sws.data_ptr(), sws.numel(), stream) for lg in logits]
    else:
        from speculative_verify_gemm_q4_amd._lib import _SampleParams
        V, K = WORKLOADS[shape]
        Wts = rotated_tiled(torch, synth, q4, V, K, 1.2, 9000, dev)
        x = synth.activations(M, K, seed=0, stream=300, device=dev)
        inp = synth.sample_inputs(M, V, 16, seed=0, device=dev)
        out = {k: torch.empty(s, dtype=t, device=dev) for k, s, t in (
            ("top_idx", (M, 20), torch.int32), ("top_val", (M, 20), torch.float32),
            ("top_prob", (M, 20), torch.float32), ("greedy", (M,), torch.int32),
            ("accept", (M,), torch.int32), ("token", (M,), torch.int32))}
        prm = _SampleParams(1.0, 0.95, 20, 16)
        fws = torch.empty(q4.q4_gemm_verify_sample_workspace(M, V, K),
                          dtype=torch.uint8, device=dev)
        fns = [functools.partial(
            lib.q4_gemm_verify_sample, x.data_ptr(), Wt.data_ptr(), M, V, K,
            ctypes.byref(prm), *[inp[k].data_ptr() for k in (
                "draft_tok", "draft_idx", "draft_q", "u", "v")],
            *[out[k].data_ptr() for k in (
                "top_idx", "top_val", "top_prob", "greedy", "accept", "token")],
            fws.data_ptr(), fws.numel(), stream) for Wt in Wts]
    if any(f() != 0 for f in fns):
        raise RuntimeError(f"{entry} failed")
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.1:
        for _ in range(10):
            fns[i % len(fns)]()
            i += 1
        torch.cuda.synchronize()
    for i in range(reps):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    print(f"done {entry} {shape} M={M} reps={reps}", flush=True)


def _short_name(name):
    """Kernel name without return type, namespaces and argument list."""
    name = name.replace("void ", "", 1).replace("(anonymous namespace)::", "")
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    base = name.split("<", 1)
    head = base[0].split("::")[-1]
    return head + ("<" + base[1] if len(base) > 1 else "")


def trace_means(d, kernel):
    """Median duration (us) per kernel name holding `kernel`, from the
    kernel-trace CSV output under d."""
    import csv
    import glob
    durs = {}
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"),
                       recursive=True):
        for row in csv.DictReader(open(f)):
            n = _short_name(row["Kernel_Name"])
            if kernel in n:
                durs.setdefault(n, []).append(
                    (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    return {n: sorted(v)[len(v) // 2] for n, v in durs.items()}


def summarize_trace(dirs, title, cmd):
    import csv
    import glob
    import statistics
    durs = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"),
                           recursive=True):
            for row in csv.DictReader(open(f)):
                n = _short_name(row["Kernel_Name"])
                durs.setdefault(n, []).append(
                    int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    total = sum(sum(v) for v in durs.values()) or 1
    print(f"# rocprofv3 kernel-trace summary: {title}")
    print(f"# command: {cmd}")
    print("# columns: kernel, calls, average ns, median ns, min ns, max ns, "
          "share of GPU time %")
    for n, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        # the library's kernels only (not torch's generators and copies)
        if "at::" in n or n.startswith("__amd"):
            continue
        print(f"{n:60s} {len(v):6d} {sum(v) / len(v):11.1f} "
              f"{statistics.median(v):11.1f} {min(v):9d} {max(v):9d} "
              f"{100 * sum(v) / total:6.2f}")


def summarize_pmc(dirs, kernel, title, cmds, duration_us, spec, copy_mb):
    """Per-dispatch means of every counter for the kernels whose name holds
    `kernel` (grouped by full template name), over the runs in `dirs`
    (one counter pass each), with derived figures:
      mfma_busy  = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDS x cycles)
      valu_busy  = 4 SQ_INSTS_VALU / (SIMDS x cycles)   (wave64: 4 cycles)
      l2_hit     = TCC_HIT / (TCC_HIT + TCC_MISS)
      l2_latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ (cycles)
      lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
    with cycles = duration_us x CLOCK_GHZ x 1e3 (the kernel's duration from
    the kernel-trace run, not the counter runs, which serialise dispatches),
    and HBM bytes = FETCH_SIZE x fetch_scale + WRITE_SIZE x write_scale, the
    scales being what the counters read for q4_stream_copy of copy_mb MiB
    (read once and written once) in the same runs.  `spec` is the
    ENTRY:SHAPE:M:REPS of the runs (for the algorithmic bytes); the JSON
    line also records the kernel source's hash, so that a later change of
    the kernels marks the byte count stale."""
    import csv
    import glob
    vals = {}
    copy = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                           recursive=True):
            for row in csv.DictReader(open(f)):
                n = _short_name(row["Kernel_Name"])
                c, v = row["Counter_Name"], float(row["Counter_Value"])
                if "stream_copy_kernel" in n:
                    copy.setdefault(c, []).append(
                        (v, int(row["Grid_Size"])))
                if kernel in n:
                    vals.setdefault(n, {}).setdefault(c, []).append(v)
    print(f"# rocprofv3 counters: {title}")
    for c in cmds:
        print(f"# command: {c}")
    print(f"# derived figures use {SIMDS} SIMDs, {CLOCK_GHZ} GHz and the "
          "kernel-trace median duration per dispatch")
    entry, shape, M, _ = spec.split(":")
    M = int(M)
    if entry == "attn":
        g = ATTN_SHAPE
        ab = attn_alg_bytes(M, g["query_heads"], g["kv_heads"], g["head_dim"],
                            int(shape))
        N = K = None
    else:
        N, K = WORKLOADS[shape]
        ab = alg_bytes(M, N, K)
    out = {"entry": entry, "shape": shape, "N": N, "K": K, "M": M,
           "kernel_filter": kernel, "duration_us": duration_us,
           "alg_bytes_per_dispatch": ab,
           "kernel_source_sha256": kernel_source_hash(
               os.path.join(os.path.dirname(KERNEL_SOURCE), "q4verify_attn.hip")
               if entry == "attn" else None), "kernels": {}}
    fscale = wscale = None
    if copy_mb and copy.get("FETCH_SIZE") and copy.get("WRITE_SIZE"):
        kib = copy_mb * 1024.0
        f = sum(v for v, _ in copy["FETCH_SIZE"]) / len(copy["FETCH_SIZE"])
        w = sum(v for v, _ in copy["WRITE_SIZE"]) / len(copy["WRITE_SIZE"])
        fscale, wscale = kib / f, kib / w
        out["copy_calibration"] = {"bytes": copy_mb * 2 ** 20,
                                   "fetch_kib_raw": round(f, 1),
                                   "write_kib_raw": round(w, 1),
                                   "fetch_scale": round(fscale, 4),
                                   "write_scale": round(wscale, 4)}
    for n, cs in vals.items():
        dur = duration_us
        if isinstance(duration_us, dict):
            dur = duration_us.get(n, 0.0)
        cyc = max(dur, 1e-9) * CLOCK_GHZ * 1e3
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        d = {"dispatches": max(len(v) for v in cs.values()),
             "duration_us": round(dur, 3),
             "counters": {c: round(v, 1) for c, v in sorted(m.items())}}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            d["mfma_busy"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc), 4)
        if "SQ_INSTS_VALU" in m:
            d["valu_busy"] = round(4 * m["SQ_INSTS_VALU"] / (SIMDS * cyc), 4)
        if "SQ_INSTS_VALU" in m and "SQ_WAVES" in m:
            d["valu_insts_per_wave"] = round(m["SQ_INSTS_VALU"] / m["SQ_WAVES"], 1)
        if "SQ_INSTS_MFMA" in m and "SQ_WAVES" in m:
            d["mfma_insts_per_wave"] = round(m["SQ_INSTS_MFMA"] / m["SQ_WAVES"], 1)
        if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m:
            h, mi = m["TCC_HIT_sum"], m["TCC_MISS_sum"]
            d["l2_hit"] = round(h / max(h + mi, 1), 4)
        if "TCP_TCC_READ_REQ_LATENCY_sum" in m and "TCP_TCC_READ_REQ_sum" in m:
            d["l2_read_latency_cycles"] = round(
                m["TCP_TCC_READ_REQ_LATENCY_sum"] /
                max(m["TCP_TCC_READ_REQ_sum"], 1), 1)
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_LDS_IDX_ACTIVE" in m:
            d["lds_bank_conflict_over_active"] = round(
                m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_LDS_IDX_ACTIVE"], 1), 4)
        if "FETCH_SIZE" in m:
            d["fetch_kib_raw"] = round(m["FETCH_SIZE"], 1)
        if "WRITE_SIZE" in m:
            d["write_kib_raw"] = round(m["WRITE_SIZE"], 1)
        if fscale and "FETCH_SIZE" in m and "WRITE_SIZE" in m:
            hb = 1024 * (m["FETCH_SIZE"] * fscale + m["WRITE_SIZE"] * wscale)
            d["hbm_bytes_per_dispatch"] = int(hb)
            d["traffic_over_alg"] = round(hb / out["alg_bytes_per_dispatch"], 4)
        out["kernels"][n] = d
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="gate_up", choices=sorted(WORKLOADS))
    ap.add_argument("--rotate-gb", type=float, default=1.2)
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the M in {1,2,4,8,16} sweep of gate+up and "
                         "down and the small shape's latency")
    ap.add_argument("--no-shapes", action="store_true",
                    help="skip the per-shape table of every projection")
    ap.add_argument("--no-full-pass", action="store_true",
                    help="skip the 64-layer pass (15.1 GB of weights)")
    ap.add_argument("--pass-reps", type=int, default=10)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run q4_stream_copy over this many MB three times "
                         "(the known-traffic kernel the byte counters are "
                         "scaled against)")
    ap.add_argument("--repeat", metavar="ENTRY:SHAPE:M:REPS",
                    help="profiling aid: only REPS calls of one entry point "
                         "(planar, tiled or ws) on one shape")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DIR",
                    help="print the kernel-trace summary of rocprofv3 CSV "
                         "output under DIR (no GPU)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print the counter summary of rocprofv3 --pmc CSV "
                         "output under each DIR (no GPU)")
    ap.add_argument("--kernel", default="gemm_kslice_kernel")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", action="append", default=[],
                    help="the command(s) that made the CSV files")
    ap.add_argument("--duration-us", type=float, default=0.0)
    ap.add_argument("--trace-dir", default="",
                    help="kernel-trace output of the same program, for the "
                         "kernels' mean durations")
    ap.add_argument("--spec", default="tiled:gate_up:16:30",
                    help="the --repeat spec of the counter runs summarized")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.title,
                        " ; ".join(args.cmd))
        return
    if args.summarize_pmc:
        dur = args.duration_us
        if args.trace_dir:
            dur = trace_means(args.trace_dir, args.kernel)
        summarize_pmc(args.summarize_pmc, args.kernel, args.title, args.cmd,
                      dur, args.spec, args.copy_calibration_mb)
        return
    if args.repeat:
        repeat_mode(args.repeat, args.copy_calibration_mb)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (the verify GEMM shards by output rows with no exchange; "
              "see the design notes).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import speculative_verify_gemm_q4_amd as q4
    q4.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    st = stamp(torch)
    N, K = WORKLOADS[args.workload]
    Mv = 16
    b16, b1 = alg_bytes(Mv, N, K), alg_bytes(1, N, K)
    log(f"stamp: {json.dumps(st)}")
    log(f"bytes/call: M=16 {b16:,}  M=1 {b1:,}; floor at {HBM_PEAK_GBPS:.0f} "
        f"GB/s: {b16 / HBM_PEAK_GBPS / 1e3:.2f} us / {b1 / HBM_PEAK_GBPS / 1e3:.2f}"
        " us (prediction)")

    wbytes = 9 * N * K // 16
    copies = max(2, math.ceil(args.rotate_gb * 1e9 / wbytes))
    Ws = [synth.q4_weights(N, K, seed=0, stream=i, device=dev)
          for i in range(copies)]
    x16 = synth.activations(Mv, K, seed=0, stream=100, device=dev)
    x1 = x16[:1].contiguous()
    y16 = torch.empty((Mv, N), dtype=torch.float32, device=dev)
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)

    if args.copy_calibration_mb:
        nb = args.copy_calibration_mb * 2 ** 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(3):
            q4.q4_stream_copy(src, dst, nb)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 3 x {nb} bytes read and written")

    # one-time repack into the tiled layout, timed on its own
    Wts = [torch.empty_like(W) for W in Ws]
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for W, Wt in zip(Ws, Wts):
        q4.q4_repack(W, Wt, N, K)
    e1.record()
    torch.cuda.synchronize()
    repack_ms = e0.elapsed_time(e1) / copies
    repack = {"ms_per_matrix": round(repack_ms, 4),
              "gbps_read_plus_write": round(2 * wbytes / (repack_ms * 1e-3)
                                            / 1e9, 1)}
    log(f"repack: {repack}")

    threads = min(16, len(os.sched_getaffinity(0)))
    W0 = Ws[0].cpu().numpy()
    # timed steps: tiled M = 16 (the step), then M = 1, then M = 16 again
    # (A-B-A order for the ratio); then the planar entry point at M = 16
    # and 1.  After each block the call on copy 0 is checked against the
    # oracle (outside the timed region).
    t16 = raw_calls(torch, q4, "q4_gemm_verify_tiled", x16, Wts, y16, Mv,
                    N, K)
    t1 = raw_calls(torch, q4, "q4_gemm_verify_tiled", x1, Wts, y1, 1, N, K)
    sa = time_stats(torch, t16, args.steps, args.warmup)
    t16[0]()
    par16 = parity(torch, synth, x16, y16, W0, N, K, threads)
    s1 = time_stats(torch, t1, args.steps, args.warmup)
    t1[0]()
    par1 = parity(torch, synth, x1, y1, W0, N, K, threads)
    sb = time_stats(torch, t16, args.steps, args.warmup)
    ms16a, wall16, ms1, ms16b = (sa["mean_ms"], sa["wall_ms"], s1["mean_ms"],
                                 sb["mean_ms"])
    p16 = raw_calls(torch, q4, "q4_gemm_verify", x16, Ws, y16, Mv, N, K)
    p1 = raw_calls(torch, q4, "q4_gemm_verify", x1, Ws, y1, 1, N, K)
    ps16 = time_stats(torch, p16, args.steps, args.warmup)
    p16[0]()
    ppar16 = parity(torch, synth, x16, y16, W0, N, K, threads)
    ps1 = time_stats(torch, p1, args.steps, args.warmup)
    p1[0]()
    ppar1 = parity(torch, synth, x1, y1, W0, N, K, threads)
    pms16, pms1 = ps16["mean_ms"], ps1["mean_ms"]
    ms_per_step = ms16a
    k16 = 0.5 * (ms16a + ms16b)
    gbps16 = b16 / (ms_per_step * 1e-3) / 1e9
    gbps1 = b1 / (ms1 * 1e-3) / 1e9
    ach16 = b16 / (k16 * 1e-3) / 1e9
    plan = q4.q4_gemm_verify_plan(Mv, N, K, q4.LAYOUT_TILED16)
    traffic = load_traffic("tiled", args.workload, Mv)
    log(f"tiled M=16: {ms16a * 1e3:.2f} / {ms16b * 1e3:.2f} us per call "
        f"({gbps16:.0f} GB/s); M=1: {ms1 * 1e3:.2f} us ({gbps1:.0f} GB/s)")
    log(f"planar M=16: {pms16 * 1e3:.2f} us ({b16 / (pms16 * 1e-3) / 1e9:.0f}"
        f" GB/s); M=1: {pms1 * 1e3:.2f} us "
        f"({b1 / (pms1 * 1e-3) / 1e9:.0f} GB/s)")

    # free the headline shape's copies before the wider measurements
    del Ws, Wts
    torch.cuda.empty_cache()

    probe = probe_sizes = None
    if not args.no_probe:
        probe_sizes = measure_stream_probe(
            torch, synth, q4, [wbytes, 9 * 248320 * 5120 // 16],
            args.rotate_gb, dev)
        probe = probe_sizes[str(wbytes)]["gbps"]
    sweep = tiny = None
    if not args.no_sweep:
        sweep = {
            "gate_up": measure_sweep(
                torch, synth, q4, "gate_up", (1, 2, 4, 8, 16),
                ("q4_gemm_verify_tiled", "q4_gemm_verify"), args.steps,
                args.warmup, args.rotate_gb, dev, threads),
            # the VALU dot-product form against MFMA where it applies
            "gate_up_dot": measure_sweep(
                torch, synth, q4, "gate_up", (1, 2, 4),
                ("q4_gemm_verify_tiled_dot",), args.steps, args.warmup,
                args.rotate_gb, dev, threads),
            "o_proj": measure_sweep(
                torch, synth, q4, "o_proj", (1, 2, 4),
                ("q4_gemm_verify_tiled", "q4_gemm_verify_tiled_dot"),
                args.steps, args.warmup, args.rotate_gb, dev, threads),
            "down": measure_sweep(
                torch, synth, q4, "down", (1, 2, 4, 8, 16),
                ("q4_gemm_verify_tiled", "q4_gemm_verify",
                 "q4_gemm_verify_tiled_ws"), args.steps, args.warmup,
                args.rotate_gb, dev, threads)}
        tiny = measure_tiny(torch, synth, q4, args.steps, args.warmup, dev,
                            threads)
    shapes = None
    if not args.no_shapes:
        shapes = measure_shapes(torch, synth, q4, [n for n in WORKLOADS],
                                args.steps, args.warmup, args.rotate_gb, dev)
    vsample = None
    if not args.no_shapes:
        vsample = measure_verify_sample(torch, synth, q4, dev, args.steps,
                                        args.warmup)
    gdn = attn = None
    if not args.no_shapes:
        gdn = measure_gdn_commit(torch, synth, q4, dev, args.steps,
                                 args.warmup)
        attn = measure_tree_attn(torch, synth, q4, dev, args.steps,
                                 args.warmup)
    full = None
    if not args.no_full_pass:
        full = measure_full_pass(torch, synth, q4, args.pass_reps, dev)

    cpu = None
    if not args.no_cpu_baseline:
        per = cpu_configs(torch, synth, dev, args.cpu_budget_s)
        head = per[f"{args.workload}_M16"] if f"{args.workload}_M16" in per \
            else None
        if head is None:
            c = cpu_baseline(torch, synth.q4_weights(N, K, seed=0, stream=0,
                                                     device=dev),
                             x16, N, K, args.cpu_budget_s)
            head = {"gbps": c["value"], "s_per_call": c["s_per_call"]}
        cpu = {"value": head["gbps"], "unit": "GB/s", "cores": per["threads"],
               "kind": "oracle",
               "sample": f"whole {N}x{K} matrix at M=16, fp64 accumulation, "
                         f"{per['threads']} threads (the box's host share); "
                         "per_config: configs 0-3 at M=1/16 and the 64-layer "
                         "pass as shape x count",
               "s_per_call": head["s_per_call"], "per_config": per}
        log(f"cpu oracle: {cpu['value']} GB/s")

    rec = {
        "metric": METRIC,
        "value": round(gbps16, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Q4 codes/scales/biases, bf16 N(0,1) x)",
        "config": {"workload": f"{args.workload}_{N}x{K}", "N": N, "K": K,
                   "M": Mv, "weight_copies": copies,
                   "layout": "tiled16 (one-time q4_repack, timed apart)",
                   "parallelism": "single GPU", "plan": plan},
        "frac_of_peak": round(gbps16 / HBM_PEAK_GBPS, 4),
        "m1": {"ms_per_step": round(ms1, 6), "gbps": round(gbps1, 1),
               "frac_of_peak": round(gbps1 / HBM_PEAK_GBPS, 4)},
        "ratio_m16_m1": round(k16 / ms1, 4),
        "repack": repack,
        "blocks_us": {"m16_first": us3(sa), "m1": us3(s1),
                      "m16_second": us3(sb)},
        "parity": {"rule": f"|y - y64| <= {REL} sum|x w| + {ABS}, every "
                           "output of the call on weight copy 0 after the "
                           "timed block",
                   "m16_max_err_over_bound": sig3(par16),
                   "m1_max_err_over_bound": sig3(par1),
                   "planar_m16_max_err_over_bound": sig3(ppar16),
                   "planar_m1_max_err_over_bound": sig3(ppar1),
                   "verdict": "pass" if max(par16, par1, ppar16, ppar1) <= 1
                   else "FAIL"},
        "planar": {"entry_point": "q4_gemm_verify",
                   "ms_per_step_m16": round(pms16, 6),
                   "gbps_m16": round(b16 / (pms16 * 1e-3) / 1e9, 1),
                   "frac_m16": round(b16 / (pms16 * 1e-3) / 1e9
                                     / HBM_PEAK_GBPS, 4),
                   "ms_per_step_m1": round(pms1, 6),
                   "gbps_m1": round(b1 / (pms1 * 1e-3) / 1e9, 1),
                   "frac_m1": round(b1 / (pms1 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                    4),
                   "ratio_m16_m1": round(pms16 / pms1, 4),
                   "blocks_us": {"m16": us3(ps16), "m1": us3(ps1)}},
        "wall_ms_per_step": round(wall16, 6),
        "stream_read_gbps": None if probe is None else round(probe, 1),
        "stream_read_by_size": probe_sizes,
        "frac_of_stream_read": None if probe is None else
        round(gbps16 / probe, 4),
        "m_sweep": sweep,
        "tiny": tiny,
        "roofline": {
            "bound": "hbm",
            "achieved": round(ach16, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(ach16 / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": KERNEL_NAMES[plan["kernel"]],
            "kernel_us": round(k16 * 1e3, 3),
            "timing": "HIP events around back-to-back launches (prepared "
                      "C-ABI calls) on the launch stream, mean of the two "
                      "M=16 blocks",
            "alg_bytes_per_launch": b16,
        },
        "cpu_baseline": cpu,
        "shapes": shapes,
        "verify_sample": vsample,
        "gdn_commit": gdn,
        "tree_attention": attn,
        "full_pass": full,
        "stamp": st,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
