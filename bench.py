#!/usr/bin/env python3
"""Benchmark of the BDLM masked-attention hot path on one MI355X.

One step = forward + backward of BDLM attention over [x0 ; xt] on one batch of
synthetic inputs already resident in HBM.  Default workload: batch 1,
L = 32768 (2L = 64K tokens), B = 64, 32 q / 8 kv heads, head_dim 128, bf16.

value = useful TFLOP/s = 14 * d * P * batch * Hq / time, P = L(L+B) visible
(query, key) pairs per (batch, q-head) (masked pairs excluded; the backward
counts 2.5x the forward, i.e. its S recompute).  One JSON line is printed.

--workload csbp_share_256k times one rank's CSBP share instead: 16 corrupted
blocks of 1024 against a 262144-token clean sequence streamed in 8192-token
chunks with the running merge, forward and backward (P = sum of B^2 (b_i + 1)
over the local blocks), plus the merge kernel alone on every partial of a step.

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
    "sources_sha256": "cb7e5bd3f12daf65cedb3ab19b262fb99c458cfaff2486653a27e861ef03f6ba",
    "fetch_kib": 9.709e6, "fetch_scale": 2.0,
    "write_kib": 2.621e5, "write_scale": 1.0,
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


def time_steps(step, steps, warmup, launches_per_step):
    """Warm up, then time `steps` steps: wall clock bracketed by device
    synchronisation (the reported rate), per-step HIP events on the stream
    (median / min), and per-kernel launch times recorded by the library."""
    import torch
    import masked_attention_bdlm_amd as M
    for i in range(warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{warmup} done")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    with M.KernelTimer(max_launches=launches_per_step * steps + 16) as kt:
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record()
            step()
            ev[i][1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    per_step = sorted(a.elapsed_time(b_) for a, b_ in ev)
    log(f"timed {steps} steps: {ms:.3f} ms/step (median {per_step[len(per_step) // 2]:.3f}, min {per_step[0]:.3f})")
    return ms, per_step, kt


def step_stats(per_step):
    return {"median_ms": round(per_step[len(per_step) // 2], 4), "min_ms": round(per_step[0], 4)}


def bench_share(args, w, dev, stream):
    """One rank's CSBP share at its real shape: own-block partial, clean chunks
    streamed with the running merge fused into the forward's epilogue, then the
    chunked backward.  Also
    times one all-at-once merge of every partial a step produces (the merge
    kernel alone, HBM-bound)."""
    import torch
    from masked_attention_bdlm_amd.api import bdlm_attn_merge_partials
    from masked_attention_bdlm_amd.csbp import (ShareBuffers, _chunks, _clean_chunks, clean_share_backward,
                                                clean_share_forward, share_backward, share_forward)
    from synth import make_share_inputs

    x = make_share_inputs(w, device=dev)
    ids = [int(i) for i in x["block_ids"]]
    B, L, d, hq = w.block, w.seqlen, w.head_dim, w.hq
    T = len(ids) * B
    log(f"workload {w.name}: {len(ids)} local blocks of {B} at ids {ids}, clean L {L}, chunk {w.share_chunk}")
    bufs = ShareBuffers(x["qx"], x["kc"], x["kx"])
    cids = [int(i) for i in x["clean_ids"]] if w.clean_share else []
    if cids:
        log(f"clean query shard (rank 0 of {w.share_ranks}, zigzag): blocks {cids}")
        cbufs = ShareBuffers(x["qs"], x["kc"])
    torch.cuda.synchronize()

    def step():
        o, lse = share_forward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk,
                               w.scale, bufs, stream)
        share_backward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse,
                       x["dox"], w.scale, bufs, stream)
        if cids:
            oc, lc = clean_share_forward(x["qs"], x["kc"], x["vc"], cids, B, w.share_chunk, w.scale, cbufs,
                                         stream)
            clean_share_backward(x["qs"], x["kc"], x["vc"], cids, B, w.share_chunk, oc, lc, x["dos"], w.scale,
                                 cbufs, stream)

    nchunks = len(_chunks(L, w.share_chunk, ids, B))
    ncchunks = len(_clean_chunks(L, w.share_chunk, cids, B)) if cids else 0
    ms, per_step, kt = time_steps(step, args.steps, args.warmup,
                                  launches_per_step=8 * (nchunks + ncchunks) + 24)
    # visible pairs: corrupted block b_i sees its clean prefix b_i*B plus its own
    # block; clean block c_j sees the clean blocks up to and including itself
    pairs = sum(B * B * (bid + 1) for bid in ids) + sum(B * B * (c + 1) for c in cids)
    useful = 14.0 * d * pairs * hq
    kernels = {k: {"launches": n, "avg_ms": tt / max(n, 1), "total_ms": tt} for k, (n, tt) in kt.times.items()}

    # merge kernel alone: all nchunks + 1 partials of a step merged at once into bf16
    nparts = nchunks + 1
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    po = [torch.randn((1, T, hq, d), device=dev, generator=g) for _ in range(nparts)]
    pl = [torch.randn((1, hq, T), device=dev, generator=g) for _ in range(nparts)]
    mo = torch.empty((1, T, hq, d), dtype=x["qx"].dtype, device=dev)
    ml = torch.empty((1, hq, T), dtype=torch.float32, device=dev)
    bdlm_attn_merge_partials(po, pl, mo, ml, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        bdlm_attn_merge_partials(po, pl, mo, ml, stream)
    e1.record()
    torch.cuda.synchronize()
    mms = e0.elapsed_time(e1) / reps
    mbytes = T * hq * (nparts * (4 * d + 4) + (mo.element_size() * d + 4))
    out = {
        "metric": ("BDLM attn CSBP rank share (corrupted blocks and the clean query shard vs the streamed "
                   "clean prefix) fwd+bwd useful TFLOP/s, 1 GPU" if cids else
                   "BDLM attn CSBP share (one rank's corrupted blocks vs the streamed clean prefix) "
                   "fwd+bwd useful TFLOP/s, 1 GPU"),
        "value": round(useful / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), **step_stats(per_step),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "clean_len": L, "block": B, "local_blocks": len(ids),
                   "block_ids": ids, "chunk": w.share_chunk, "chunks": nchunks,
                   **({"clean_block_ids": cids, "clean_chunks": ncchunks, "ranks": w.share_ranks} if cids else {}),
                   "q_heads": hq,
                   "kv_heads": w.hkv, "head_dim": d, "parallelism": "single GPU (one rank's share)"},
        "pct_of_peak": round(100.0 * useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "useful_flop_per_step": useful,
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in kernels.items()},
        "kernel_launches_per_step": {k: v["launches"] // args.steps for k, v in kernels.items()},
        "merge_alone": {"parts": nparts, "rows": T, "heads": hq, "bytes": mbytes, "ms": round(mms, 4),
                        "achieved_GBps": round(mbytes / (mms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(mbytes / (mms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_balance(args, w, dev, stream):
    """Every rank's whole attention share (its corrupted blocks and its clean
    query shard against the streamed clean K/V) timed one after another on this
    GPU, for the contiguous and the zigzag block layout: the slowest rank sets
    the step time of a data-parallel-free CSBP layer, so max/mean per layout
    and max(contiguous)/max(zigzag) measure what the layout is worth."""
    import torch
    from masked_attention_bdlm_amd.csbp import (ShareBuffers, clean_share_backward, clean_share_forward,
                                                rank_blocks, rank_cost, share_backward, share_forward)
    from synth import make_share_inputs

    R, B, nb = w.share_ranks, w.block, w.seqlen // w.block
    x = make_share_inputs(w, device=dev, nlocal=nb // R)     # input values do not affect the timing
    bufs = ShareBuffers(x["qx"], x["kc"], x["kx"])
    cbufs = ShareBuffers(x["qs"], x["kc"])
    res = {}
    for layout in ("contiguous", "zigzag"):
        per = []
        for r in range(R):
            ids = rank_blocks(nb, R, r, layout)

            def step(ids=ids):
                o, lse = share_forward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk,
                                       w.scale, bufs, stream)
                share_backward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse,
                               x["dox"], w.scale, bufs, stream)
                oc, lc = clean_share_forward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, w.scale, cbufs,
                                             stream)
                clean_share_backward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, oc, lc, x["dos"], w.scale,
                                     cbufs, stream)

            ms, _, _ = time_steps(step, args.steps, args.warmup, launches_per_step=8 * 2 * (nb * B // w.share_chunk + 1) + 32)
            per.append({"rank": r, "blocks": ids, "ms": round(ms, 3), "block_pairs": 2 * rank_cost(ids)})
            log(f"{layout} rank {r}: {ms:.2f} ms")
        t = [p["ms"] for p in per]
        res[layout] = {"max_ms": max(t), "mean_ms": round(sum(t) / R, 3), "min_ms": min(t),
                       "max_over_mean": round(max(t) / (sum(t) / R), 4),
                       "cost_max_over_mean": round(max(p["block_pairs"] for p in per) /
                                                   (sum(p["block_pairs"] for p in per) / R), 4),
                       "ranks": per}
    speed = res["contiguous"]["max_ms"] / res["zigzag"]["max_ms"]
    out = {
        "metric": f"CSBP layer attention step time over {R} simulated ranks at 256K: slowest rank, "
                  "contiguous vs zigzag block layout (speedup)",
        "value": round(speed, 4), "unit": "x", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "clean_len": w.seqlen, "block": B, "ranks": R,
                   "blocks_per_rank": nb // R, "chunk": w.share_chunk, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": w.head_dim, "parallelism": "single GPU (ranks timed one after another)"},
        "layouts": res,
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_64k")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--balance", action="store_true",
                    help="with a rank-share workload: time all ranks under the contiguous and zigzag layouts")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if w.share_blocks and args.balance:
        if not w.clean_share:
            print("--balance needs a workload with the clean query shard (csbp_rank_256k)", file=sys.stderr)
            sys.exit(2)
        bench_balance(args, w, dev, stream)
        return
    if w.share_blocks:
        bench_share(args, w, dev, stream)
        return
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

    def step():
        bdlm_attn_fwd(desc, x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], oc, ox, lse_c, lse_x,
                      None, stream)
        bdlm_attn_bwd(desc, x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], oc, ox, lse_c, lse_x,
                      x["doc"], x["dox"], dqc, dkc, dvc, dqx, dkx, dvx, ws, stream)

    ms, per_step, kt = time_steps(step, args.steps, args.warmup, launches_per_step=16)

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
        **step_stats(per_step),
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
