"""Benchmark of the fused attention forward on one MI355X.

One step is one attn_fwd_split call over one batch of seeded synthetic input
already resident in HBM: the whole fused path (Q tile load, K/V streaming,
both MFMA products, online softmax, masking, epilogue).  Where the query
blocks fill the GPU (the 8K and 16K GQA workloads) that is a single attention
kernel launch, the same as attn_fwd; for short sequences the library's
automatic key split adds the merge kernel, and the step is both launches.
Prints ONE JSON line:

  value         causal-adjusted TFLOP/s: (4*Sq*Sk*d*Hq*B, halved when causal)
                divided by the mean wall time per step over the timed steps
  roofline      the kernel against the MI355X dense fp16/bf16 MFMA peak, with the
                kernel's own duration from HIP events on its launch stream
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded sample
                of rows of the same workload (a baseline, not a target)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--kv-split N] [--backward] [--head-size D] [--dtype T]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (causal-adjusted) and % of MI355X bf16 MFMA peak"
# MI355X published dense fp16/bf16 matrix peak (256 CUs at 2.4 GHz), TFLOP/s
PEAK_MFMA_TFLOPS = 2516.6
# MI355X published HBM3E bandwidth, GB/s
PEAK_HBM_GBS = 8000.0
# the largest single-GPU workload of the long causal GQA pair the target is
# set on (the 8K one runs with --workload gqa4_causal_bf16_b1_hq32_hkv8_s8192_d128)
DEFAULT_WORKLOAD = "gqa8_causal_outlier_bf16_b1_hq32_hkv4_s16384_d128"
# untimed warmup: at least --warmup steps and at least this many seconds of
# back-to-back steps (--min-warmup-s), so that the board's power management
# has settled the clock before the timed steps (the first tens of milliseconds
# of a burst run at a dipped clock)
MIN_WARMUP_S = 1.0


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for p in ("exact_attention_19_amd/csrc/attn_fwd.hip",
              "exact_attention_19_amd/csrc/attn_common.h", "include/attn.h"):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, budget_s: float = 22.0):
    """Time the fp64 oracle on a bounded, seeded sample of query rows of the
    workload (rows drawn uniformly over batch, heads and positions) and scale
    to TFLOP/s with the exact FLOPs of the sampled rows (4*d per visible
    key).  The sample is sized from a calibration run of at least a second
    for budget_s; the larger timed sample keeps the threads busier than the
    calibration did, so the run takes less (measured: about 0.55 x budget_s,
    i.e. 10-15 s on 16 host threads)."""
    import numpy as np
    from oracle import attn_fwd_oracle

    cores = min(16, len(os.sched_getaffinity(0)))
    rng = np.random.default_rng(0)
    # widen to fp64 once, outside the timed region (exact for fp16/bf16)
    q, k, v = (t.double().numpy() for t in (q, k, v))
    total_rows = w.B * w.Hq * w.Sq

    def visible(rows):
        i = rows % w.Sq
        if not w.causal:
            return np.full(rows.shape, w.Sk, dtype=np.int64)
        return np.clip(i + (w.Sk - w.Sq) + 1, 0, w.Sk)

    # calibrate: grow the sample until it takes a second, then size the timed
    # sample to the budget by visible keys (the oracle's cost per row)
    n_cal = 4 * cores
    while True:
        calib = rng.integers(0, total_rows, n_cal)
        t0 = time.perf_counter()
        attn_fwd_oracle(q, k, v, w.scale, w.causal, rows=calib, nthreads=cores)
        t_cal = time.perf_counter() - t0
        if t_cal >= 1.0 or n_cal >= total_rows:
            break
        n_cal = min(total_rows, n_cal * max(2, int(1.5 / max(t_cal, 1e-3))))
    per_key = t_cal / max(1, int(visible(calib).sum()))
    mean_keys = float(visible(rng.integers(0, total_rows, 4096)).mean())
    n = int(max(cores, min(total_rows, budget_s / (per_key * max(mean_keys, 1.0)))))
    rows = rng.integers(0, total_rows, n)
    t0 = time.perf_counter()
    attn_fwd_oracle(q, k, v, w.scale, w.causal, rows=rows, nthreads=cores)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * float(visible(rows).sum())
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
           "kind": "oracle",
           "sample": f"{n} random query rows of {w.name} ({n / total_rows:.2%} of "
                     f"all rows), fp64, {dt:.1f} s",
           "seconds": round(dt, 2)}
    return res, rows


def sample_parity(w, rows, o_gpu, lse_gpu, q, k, v):
    """max |dO| and |dLSE| of the timed launch's output on the baseline's
    sampled rows against the oracle (the rows' oracle values are recomputed
    here, untimed)."""
    import numpy as np
    from oracle import attn_fwd_oracle
    rows = np.unique(rows)
    o_ref, lse_ref = attn_fwd_oracle(q, k, v, w.scale, w.causal, rows=rows)
    i = rows % w.Sq
    h = (rows // w.Sq) % w.Hq
    b = rows // (w.Sq * w.Hq)
    og = o_gpu.double().numpy()[b, i, h]
    lg = lse_gpu.double().numpy()[b, h, i]
    fin = np.isfinite(lse_ref)
    return {"rows": int(rows.size), "max_abs_dO": float(np.abs(og - o_ref).max()),
            "max_abs_dLSE": float(np.abs(lg[fin] - lse_ref[fin]).max()) if fin.any() else 0.0,
            "tol_O": 2e-3 if w.dtype == "f16" else 1e-2, "tol_LSE": 1e-3}


def bwd_bytes(w) -> int:
    """Algorithmic bytes of the backward pass: Q, O, dO, dQ (query side) and
    K, V, dK, dV (key side) once each at 2 bytes per element, plus the LSE."""
    q = w.B * w.Sq * w.Hq * w.d * 2
    kv = w.B * w.Sk * w.Hkv * w.d * 2
    return 4 * q + 4 * kv + w.B * w.Hq * w.Sq * 4


def copy_probe(mib: int, steps: int):
    """Device-to-device copy of a known size, for scaling the HBM byte counters
    (FETCH_SIZE, WRITE_SIZE) of a profiler run to bytes."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    # read n and write n bytes per launch
    print(json.dumps({"copy_probe_bytes": n, "launches": steps + 1, "ms_per_copy": round(ms, 4),
                      "read_plus_write_GBps": round(2 * n / ms / 1e6, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first ~30 back-to-back launches run while the board's power
    # management settles the clock; the default warmup covers them so the
    # timed steps measure the sustained rate
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--kv-split", type=int, default=0,
                    help="key split of attn_fwd_split: 0 = the library's choice, "
                         "1 = none, N = at most N pieces per query block")
    ap.add_argument("--backward", action="store_true",
                    help="time attn_bwd (dQ, dK, dV from O, LSE and a seeded dO) instead of "
                         "the forward; FLOPs are 2.5x the forward's (five products of the "
                         "forward's two-product size)")
    ap.add_argument("--cold", type=int, default=1, metavar="N",
                    help="rotate N copies of the inputs and outputs across steps, so that a "
                         "step's data is not left in the 256 MB MALL by the step before "
                         "(forward only; default 1 = warm)")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="decode workloads: time attn_decode_paged with K and V in a "
                         "shuffled pool of BLOCK-token blocks (every sequence Sk long)")
    ap.add_argument("--min-warmup-s", type=float, default=MIN_WARMUP_S, metavar="S",
                    help="untimed warmup lasts at least S seconds as well as --warmup steps "
                         "(default 1.0; 0 under counter collection, where every warmup "
                         "dispatch is recorded and the clock does not matter)")
    ap.add_argument("--head-size", type=int, default=0, metavar="D",
                    help="run the named workload with head size D (scale 1/sqrt(D)); "
                         "the workload's name then ends in _dD")
    ap.add_argument("--dtype", choices=("f16", "bf16"), default="",
                    help="run the named workload in this dtype; the workload's name "
                         "then has it in place of its own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, metavar="MIB", default=0,
                    help="only run a device copy of MIB MiB --steps times "
                         "(calibration of the profiler's byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the attention forward is built and "
              "timed on a single GPU only (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe > 0:
        copy_probe(args.copy_probe, args.steps)
        return

    import torch
    from exact_attention_19_amd import (attn_bwd, attn_bwd_workspace, attn_fwd, attn_fwd_plan,
                                        attn_fwd_split, attn_fwd_split_plan,
                                        attn_fwd_split_workspace, load_library)
    from exact_attention_19_amd.binding import ATTN_DTYPE_BF16, ATTN_DTYPE_F16
    from exact_attention_19_amd.workloads import WORKLOADS, input_digest, make_inputs

    load_library()
    w = WORKLOADS[args.workload]
    if args.head_size:
        hd = args.head_size
        w = w.with_(name=re.sub(r"_d\d+$", f"_d{hd}", w.name), d=hd, scale=1.0 / math.sqrt(hd))
    if args.dtype and args.dtype != w.dtype:
        w = w.with_(name=re.sub(r"_(f16|bf16)_", f"_{args.dtype}_", w.name), dtype=args.dtype)
    dev = torch.device("cuda:0")
    q_cpu, k_cpu, v_cpu = make_inputs(w, seed=0)
    digest = input_digest(q_cpu, k_cpu, v_cpu)
    q, k, v = q_cpu.to(dev), k_cpu.to(dev), v_cpu.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dt_code = ATTN_DTYPE_BF16 if w.dtype == "bf16" else ATTN_DTYPE_F16
    shape = (w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.d, int(w.causal), dt_code)
    split = attn_fwd_split_plan(*shape, kv_split=args.kv_split)
    ws_bytes = attn_fwd_split_workspace(*shape, kv_split=args.kv_split)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    sets = [(q, k, v, o, lse)]
    for _ in range(max(args.cold, 1) - 1):
        sets.append((q.clone(), k.clone(), v.clone(), torch.empty_like(o), torch.empty_like(lse)))
    turn = [0]

    def step():
        qs, ks, vs, os_, ls = sets[turn[0] % len(sets)]
        turn[0] += 1
        attn_fwd_split(qs, ks, vs, scale=w.scale, causal=w.causal, kv_split=args.kv_split,
                       out=os_, lse=ls, workspace=ws, stream=stream)

    if args.paged:
        from exact_attention_19_amd import attn_decode_paged, attn_decode_paged_workspace
        from exact_attention_19_amd.workloads import make_paged_cache
        kp, vp, table, seqlens = (t.to(dev) for t in make_paged_cache(
            k_cpu, v_cpu, [w.Sk] * w.B, args.paged, seed=1))
        pws = torch.empty(max(attn_decode_paged_workspace(w.B, w.Sq, w.Hq, w.Hkv, w.d, w.Sk,
                                                          args.kv_split), 1),
                          dtype=torch.uint8, device=dev)

        def step():  # noqa: F811 (the paged step replaces the dense one)
            attn_decode_paged(q, kp, vp, table, seqlens, scale=w.scale, causal=w.causal,
                              max_seqlen=w.Sk, kv_split=args.kv_split, out=o, lse=lse,
                              workspace=pws, stream=stream)

    if args.backward:
        attn_fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, stream=stream)
        gen = torch.Generator().manual_seed(1)
        dout = torch.randn(q.shape, generator=gen).to(q.dtype).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(attn_bwd_workspace(w.B, w.Sq, w.Hq), dtype=torch.uint8, device=dev)

        def step():  # noqa: F811 (the backward step replaces the forward one)
            attn_bwd(q, k, v, o, lse, dout, scale=w.scale, causal=w.causal, dq=dq, dk=dk,
                     dv=dv, workspace=bws, stream=stream)

    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.min_warmup_s:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()  # the clock runs on the device's time
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_w

    # timed region: K launches on one stream, a HIP event pair around each
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_avg_s = sum(kern_ms) / len(kern_ms) / 1e3
    kern_min_s = min(kern_ms) / 1e3
    kern_med_s = sorted(kern_ms)[len(kern_ms) // 2] / 1e3
    ms_per_step = wall / args.steps * 1e3

    flops = w.metric_flops() * (2.5 if args.backward else 1.0)
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / kern_avg_s / 1e12
    plan = attn_fwd_plan(*shape)
    # the bound: arithmetic intensity (exact FLOPs per algorithmic byte)
    # against the ridge point of the two MI355X peaks
    ridge = PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if args.backward or w.exact_flops() / w.algorithmic_bytes() >= ridge:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_TFLOPS, 4)}
    else:
        gbs = w.algorithmic_bytes() / kern_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                "tflops_at_kernel_time": round(achieved, 2)}
    props = torch.cuda.get_device_properties(dev)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        # untimed steps actually run: --warmup, extended to MIN_WARMUP_S
        "warmup_steps_run": n_warm,
        "warmup_s": round(warm_s, 3),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) / outlier recipe, resident in HBM)",
        "config": {"workload": w.name, "pass": "backward" if args.backward else "forward",
                   "kv_cache": f"paged, {args.paged}-token blocks" if args.paged else "dense",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Sq": w.Sq, "Sk": w.Sk, "d": w.d, "causal": w.causal,
                   "scale": w.scale, "input_sha256": digest[:16]},
        "pct_of_peak": round(100.0 * value / PEAK_MFMA_TFLOPS, 2),
        "roofline": dict(roof, **{
            "traffic": measured_traffic(w.name),
            # with a key split the step is two launches (attention, merge):
            # the event pair then times both
            "launches_per_step": 3 if args.backward else (2 if split["keys_per_piece"] > 0 else 1),
            "kernel_avg_us": round(kern_avg_s * 1e6, 2),
            # the algorithmic bytes over the kernel time, whatever the bound
            "algorithmic_gbs": round(((bwd_bytes(w) if args.backward else w.algorithmic_bytes())
                                      / kern_avg_s / 1e9), 1),
            "kernel_min_us": round(kern_min_s * 1e6, 2),
            "kernel_median_us": round(kern_med_s * 1e6, 2),
            "flops_per_launch": flops,
            "exact_visible_flops_per_launch": w.exact_flops() * (2.5 if args.backward else 1.0),
            # backward: Q, K, V, O, dO and the LSE read, dQ, dK, dV written
            "algorithmic_bytes_per_launch": (bwd_bytes(w) if args.backward
                                             else w.algorithmic_bytes()),
        }),
        "launch": plan,
        "split": dict(split, kv_split_arg=args.kv_split, workspace_bytes=ws_bytes),
        "input_sets_rotated": len(sets),
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_source_digest": kernel_source_digest(),
    }
    if not args.no_cpu_baseline and not args.backward:
        base, rows = cpu_baseline(w, q_cpu, k_cpu, v_cpu)
        result["cpu_baseline"] = base
        # the timed launches' output (input set 0; the paged step writes it too)
        # on the sampled rows
        result["sample_parity"] = sample_parity(w, rows, sets[0][3].cpu(), sets[0][4].cpu(),
                                                q_cpu, k_cpu, v_cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
