#!/usr/bin/env python3
"""Benchmark of the BDLM masked-attention hot path on one MI355X.

One step = forward + backward of BDLM attention over [x0 ; xt] on one batch of
synthetic inputs already resident in HBM.  Default workload: batch 1,
L = 32768 (2L = 64K tokens), B = 64, 32 q / 8 kv heads, head_dim 128, bf16.

value = useful TFLOP/s = 14 * d * P * batch * Hq / time, P = L(L+B) visible
(query, key) pairs per (batch, q-head) (masked pairs excluded; the backward
counts 2.5x the forward, i.e. its S recompute).  One JSON line is printed.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


# HBM bytes per launch of the dominant kernel, from rocprofv3 --pmc FETCH_SIZE
# and WRITE_SIZE (KiB per dispatch) on one step of the default workload, each
# scaled by what the same counter reads for a 1 GiB device copy (FETCH_SIZE
# reads 0.5 GiB there: x2.0; WRITE_SIZE 1 GiB: x1.0).  Valid only for the
# kernel sources with this SHA-256; after any change the field is null until
# the counters are taken again.
MEASURED_TRAFFIC = {
    "kernel": "bdlm_dkdv",
    "sources_sha256": "ea79f824dd86b8d9fe827c90191824bc96a04d7153110bfa557ea13f16eea090",
    "fetch_kib": 1.46e7, "fetch_scale": 2.0,
    "write_kib": 2.622e5, "write_scale": 1.0,
}
KERNEL_SOURCES = ["bdlm_kernels.hip", "bdlm_kernels.h", "bdlm_device.h", "bdlm_common.h"]


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "masked_attention_bdlm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    m = MEASURED_TRAFFIC
    if kernel != m["kernel"] or kernel_sources_sha256() != m["sources_sha256"]:
        return None
    return 1024.0 * (m["fetch_kib"] * m["fetch_scale"] + m["write_kib"] * m["write_scale"])


def visible_pairs(L, B):
    n = L // B
    return B * B * n * (n + 1)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(w, x, seconds_budget=15.0, max_units=1024):
    """Time the fp64 oracle on sampled units of the same workload (bounded)."""
    import torch
    from threadpoolctl import threadpool_info
    from oracle import bdlm_oracle as O
    from synth import draw_units, to_f64

    units = draw_units(w.nblocks, w.hq, w.batch, max_units, w.seed)
    L, B = w.seqlen, w.block
    done, useful, t_used = 0, 0.0, 0.0
    kv = {}
    for (b, st, blk, h) in units.tolist():
        g = h // (w.hq // w.hkv)
        if (b, g) not in kv:
            kv.clear()
            kv[(b, g)] = (to_f64(torch.cat([x["kc"][b, :, g], x["kx"][b, :, g]])),
                          to_f64(torch.cat([x["vc"][b, :, g], x["vx"][b, :, g]])))
        k_all, v_all = kv[(b, g)]
        tok = slice(blk * B, (blk + 1) * B)
        q_rows = to_f64(x["qc" if st == 0 else "qx"][b, tok, h])
        do_rows = to_f64(x["doc" if st == 0 else "dox"][b, tok, h])
        rows = st * L + np.arange(blk * B, (blk + 1) * B)
        t0 = time.perf_counter()
        O.unit_rows_fwd_bwd(q_rows, k_all, v_all, O.bdlm_mask_rows(L, B, rows), do_rows, w.scale)
        t_used += time.perf_counter() - t0
        done += 1
        useful += 14.0 * w.head_dim * B * (blk + 1) * B
        if t_used >= seconds_budget:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": useful / t_used / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "seconds": round(t_used, 3),
        "sample": (f"{done} sampled (batch, stream, block, q-head) units of {w.name}: each {B} query rows "
                   f"against all 2L={2 * L} keys of its kv head, fp64 numpy with the explicit mask rows; "
                   f"rate over the units' visible pairs (the oracle also spends work on masked pairs)"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_64k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import masked_attention_bdlm_amd as M
    from masked_attention_bdlm_amd.api import bdlm_attn_bwd, bdlm_attn_fwd, desc_for, workspace
    from synth import WORKLOADS, make_full_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    M.load()
    if args.copy_bytes > 0:
        # One device-to-device copy of a known size: what the HBM byte counters
        # read for it calibrates their reading for the attention kernels.
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes}), flush=True)
        return
    w = WORKLOADS[args.workload]
    if w.share_blocks:
        print("share-mode workloads are measured by bench_share in the tests; use a full-mode workload",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    log(f"workload {w.name}: batch {w.batch} L {w.seqlen} B {w.block} hq {w.hq} hkv {w.hkv} d {w.head_dim}")
    x = make_full_inputs(w, device=dev)
    torch.cuda.synchronize()
    desc = desc_for(x["qc"], x["kc"], w.block, w.scale)
    b, L, hq, d = x["qc"].shape
    oc, ox = torch.empty_like(x["qc"]), torch.empty_like(x["qx"])
    lse_c = torch.empty((b, hq, L), dtype=torch.float32, device=dev)
    lse_x = torch.empty_like(lse_c)
    dqc, dqx = torch.empty_like(x["qc"]), torch.empty_like(x["qx"])
    dkc, dvc, dkx, dvx = (torch.empty_like(x["kc"]) for _ in range(4))
    ws = workspace(desc, True, dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        bdlm_attn_fwd(desc, x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], oc, ox, lse_c, lse_x,
                      None, stream)
        bdlm_attn_bwd(desc, x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], oc, ox, lse_c, lse_x,
                      x["doc"], x["dox"], dqc, dkc, dvc, dqx, dkx, dvx, ws, stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    torch.cuda.synchronize()
    with M.KernelTimer(max_launches=16 * args.steps + 16) as kt:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step")

    P = visible_pairs(w.seqlen, w.block)
    heads = w.batch * w.hq
    useful = 14.0 * d * P * heads
    strict = 12.0 * d * P * heads
    value = useful / (ms * 1e-3) / 1e12

    kernels = {k: {"launches": n, "avg_ms": t / max(n, 1), "total_ms": t} for k, (n, t) in kt.times.items()}
    # MFMA flops each kernel executes per launch (all 2*d per visible pair per
    # product): forward S, PV; dK/dV kernel S, dP, dV, dK; dQ kernel S, dP, dQ.
    # bdlm_bwd_pre (D = rowsum(dO * O)) is HBM-bound and small.
    kernel_flop = {"bdlm_fwd": 4.0 * d * P * heads, "bdlm_dkdv": 8.0 * d * P * heads,
                   "bdlm_dq": 6.0 * d * P * heads}
    per_kernel = {}
    for name, fl in kernel_flop.items():
        kk = kernels.get(name)
        if kk:
            a = fl / (kk["avg_ms"] * 1e-3) / 1e12
            per_kernel[name] = {"achieved": round(a, 2), "frac": round(a / PEAK_BF16_TFLOPS, 4),
                                "avg_launch_ms": round(kk["avg_ms"], 4), "flop_per_launch": fl}
    roof = None
    timed = [n for n in kernel_flop if n in kernels]
    if timed:
        dom = max(timed, key=lambda n: kernels[n]["total_ms"])
        pk = per_kernel[dom]
        traffic = measured_traffic(dom)
        roof = {"kernel": dom, "bound": "mfma", "achieved": pk["achieved"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": pk["frac"],
                "traffic": None if traffic is None else round(traffic),
                "traffic_unit": "bytes per launch (HBM, counter-calibrated)",
                "flop_per_launch": pk["flop_per_launch"], "avg_launch_ms": pk["avg_launch_ms"]}
    extra = {"kernel_roofline": per_kernel}

    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on sampled units (CPU baseline)")
        cpu = cpu_baseline(w, x, seconds_budget=args.cpu_seconds)

    out = {
        "metric": "BDLM attn fwd+bwd useful TFLOP/s and % bf16 MFMA peak at 2L=64K, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len_clean": w.seqlen,
                   "seq_len_total": 2 * w.seqlen, "block": w.block, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "strict_12_tflops": round(strict / (ms * 1e-3) / 1e12, 3),
        "useful_flop_per_step": useful,
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in kernels.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
