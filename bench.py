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
--workload csbp_memory compares one rank's peak device bytes under pure block
parallelism and under CSBP (clean chunks staged through a bounded buffer).

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
    "sources_sha256": "0694fba203434932e6abb01f08862d443f66d931e0fed9405e2733ad219e7ab3",
    "fetch_kib": 1.1945241e7, "fetch_scale": 2.0,
    "write_kib": 2.62144e5, "write_scale": 1.0,
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


def cpu_full_oracle(w, x):
    """The fp64 oracle on the whole problem (the tiny fp32 case): its wall
    seconds for one forward + backward, and the useful rate."""
    from threadpoolctl import threadpool_info
    from oracle import bdlm_oracle as O
    from synth import to_f64
    xh = {k: to_f64(v) for k, v in x.items()}
    t0 = time.perf_counter()
    O.bdlm_fwd_bwd(xh["qc"], xh["kc"], xh["vc"], xh["qx"], xh["kx"], xh["vx"], xh["doc"], xh["dox"],
                   w.block, w.scale)
    sec = time.perf_counter() - t0
    useful = 14.0 * w.head_dim * visible_pairs(w.seqlen, w.block) * w.batch * w.hq
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": useful / sec / 1e12, "unit": "TFLOP/s", "seconds": round(sec, 4), "cores": int(threads),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"the whole {w.name} problem: explicit {2 * w.seqlen}x{2 * w.seqlen} mask, fp64 numpy "
                      f"forward + backward of every (batch, head)"}


def cpu_baseline_share(w, x, ids, clean_ids, seconds_budget=15.0):
    """The fp64 oracle on sampled share units (local block, q-head): each one
    the block's B query rows against its visible keys (clean prefix and own
    block; a clean query block: its inclusive clean prefix), forward + backward."""
    from threadpoolctl import threadpool_info
    from oracle import bdlm_oracle as O
    from synth import to_f64
    B, d = w.block, w.head_dim
    rep = w.hq // w.hkv
    rng = np.random.default_rng(w.seed + 300)
    units = [("x", i) for i in range(len(ids))] + [("c", i) for i in range(len(clean_ids))]
    order = rng.permutation(len(units) * w.hq)
    done, useful, t_used = 0, 0.0, 0.0
    for u in order.tolist():
        kind, i = units[u // w.hq]
        h = u % w.hq
        g = h // rep
        r = slice(i * B, (i + 1) * B)
        if kind == "x":
            end = ids[i] * B
            keys = np.concatenate([to_f64(x["kc"][0, :end, g]), to_f64(x["kx"][0, r, g])])
            vals = np.concatenate([to_f64(x["vc"][0, :end, g]), to_f64(x["vx"][0, r, g])])
            q, do = to_f64(x["qx"][0, r, h]), to_f64(x["dox"][0, r, h])
        else:
            end = (clean_ids[i] + 1) * B
            keys, vals = to_f64(x["kc"][0, :end, g]), to_f64(x["vc"][0, :end, g])
            q, do = to_f64(x["qs"][0, r, h]), to_f64(x["dos"][0, r, h])
        t0 = time.perf_counter()
        o, lse, p = O.attention_fwd(q, keys, vals, np.ones((B, len(keys)), dtype=bool), w.scale)
        O.attention_bwd(q, keys, vals, p, o, do, w.scale)
        t_used += time.perf_counter() - t0
        done += 1
        useful += 14.0 * d * B * len(keys)
        if t_used >= seconds_budget:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": useful / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle", "seconds": round(t_used, 3),
            "sample": f"{done} sampled (local block, q-head) units of {w.name}: each block's {B} query rows "
                      f"against its visible keys, fp64 numpy forward + backward; rate over those pairs"}


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


def share_kernel_roofline(kernels, flop, steps, peak):
    """Per-kernel figures of a share step: each kernel's algorithmic flops per
    step over its summed launch time per step (the kernels are launched once
    per chunk, with windows of different sizes)."""
    out = {}
    for name, fl in flop.items():
        kk = kernels.get(name)
        if not kk:
            continue
        per_step_ms = kk["total_ms"] / steps
        a = fl / (per_step_ms * 1e-3) / 1e12
        out[name] = {"achieved": round(a, 2), "frac": round(a / peak, 4), "ms_per_step": round(per_step_ms, 4),
                     "launches_per_step": kk["launches"] // steps, "flop_per_step": fl}
    return out


def bench_share(args, w, dev, stream):
    """One rank's CSBP share at its real shape: own-block partial, clean chunks
    streamed with the running merge fused into the forward's epilogue, then the
    chunked backward.  The merge kernel is also timed alone on every partial
    that the unfused form of the same step produces (one per chunk plus the
    own-block partial), merged at once."""
    import torch
    from masked_attention_bdlm_amd.api import bdlm_attn_merge_partials, share_fwd
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

    chunks = _chunks(L, w.share_chunk, ids, B)
    nchunks = len(chunks)
    ncchunks = len(_clean_chunks(L, w.share_chunk, cids, B)) if cids else 0
    ms, per_step, kt = time_steps(step, args.steps, args.warmup,
                                  launches_per_step=8 * (nchunks + ncchunks) + 24)
    # visible pairs: corrupted block b_i sees its clean prefix b_i*B plus its own
    # block; clean block c_j sees the clean blocks up to and including itself
    pairs = sum(B * B * (bid + 1) for bid in ids) + sum(B * B * (c + 1) for c in cids)
    useful = 14.0 * d * pairs * hq
    kernels = {k: {"launches": n, "avg_ms": tt / max(n, 1), "total_ms": tt} for k, (n, tt) in kt.times.items()}
    flop = {"bdlm_fwd": 4.0 * d * pairs * hq, "bdlm_dkdv": 8.0 * d * pairs * hq, "bdlm_dq": 2.0 * d * pairs * hq}
    per_kernel = share_kernel_roofline(kernels, flop, args.steps, PEAK_BF16_TFLOPS)
    if "bdlm_dq" in per_kernel:      # the dQ kernel also recomputes S and dP^T: 6 d P executed
        ex = 3.0 * per_kernel["bdlm_dq"]["achieved"]
        per_kernel["bdlm_dq"]["executed_6dP_achieved"] = round(ex, 2)
        per_kernel["bdlm_dq"]["executed_6dP_frac"] = round(ex / PEAK_BF16_TFLOPS, 4)
    dom = max(per_kernel, key=lambda n: per_kernel[n]["ms_per_step"])
    pk = per_kernel[dom]
    roof = {"kernel": dom, "bound": "mfma", "achieved": pk["achieved"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": pk["frac"], "traffic": None,
            "note": "algorithmic flops per step over the kernel's summed launch time per step (one launch per "
                    "chunk)"}

    # merge kernel alone on the partials of this step in its unfused form:
    # the own-block partial and one partial per clean chunk, all merged at once
    nparts = nchunks + 1
    po = [torch.empty((1, T, hq, d), dtype=torch.float32, device=dev) for _ in range(nparts)]
    pl = [torch.empty((1, hq, T), dtype=torch.float32, device=dev) for _ in range(nparts)]
    share_fwd(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, 0, 0, 1, w.scale, out=(po[0], pl[0]),
              stream=stream)
    for n, (j0, j1) in enumerate(chunks):
        share_fwd(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, j0, j1, 0, w.scale,
                  out=(po[n + 1], pl[n + 1]), stream=stream)
    mo = torch.empty((1, T, hq, d), dtype=x["qx"].dtype, device=dev)
    ml = torch.empty((1, hq, T), dtype=torch.float32, device=dev)
    bdlm_attn_merge_partials(po, pl, mo, ml, stream)
    torch.cuda.synchronize()
    # algorithmic bytes: every live part's O row (4d) and LSE (4) read, the
    # output row (2d bf16) and LSE written; parts with LSE = -inf (chunks above
    # a block's prefix) are not read
    live = [torch.isfinite(l).sum().item() for l in pl]          # (row, head) pairs with a live part
    mbytes = sum(live) * (4 * d + 4) + T * hq * (mo.element_size() * d + 4)
    reps = 10
    from masked_attention_bdlm_amd.api import KernelTimer
    with KernelTimer(reps + 4) as mk:
        for _ in range(reps):
            bdlm_attn_merge_partials(po, pl, mo, ml, stream)
        torch.cuda.synchronize()
    mn, mt = mk.times["bdlm_merge"]
    mms = mt / mn
    merge = {"parts": nparts, "rows": T, "heads": hq, "algorithmic_bytes": mbytes, "avg_launch_ms": round(mms, 4),
             "achieved_GBps": round(mbytes / (mms * 1e-3) / 1e9, 1),
             "frac_of_hbm_peak": round(mbytes / (mms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del po, pl

    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on sampled share units (CPU baseline)")
        cpu = cpu_baseline_share(w, x, ids, cids, seconds_budget=args.cpu_seconds)
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
        "kernels_ms_per_step": {k: round(v["total_ms"] / args.steps, 4) for k, v in kernels.items()},
        "fwd_ms": round(sum(kernels.get(n, {}).get("total_ms", 0.0) for n in ("bdlm_fwd", "bdlm_merge")) / args.steps, 4),
        "bwd_ms": round(sum(kernels.get(n, {}).get("total_ms", 0.0)
                            for n in ("bdlm_bwd_pre", "bdlm_dkdv", "bdlm_dq")) / args.steps, 4),
        "kernel_launches_per_step": {k: v["launches"] // args.steps for k, v in kernels.items()},
        "roofline": roof,
        "kernel_roofline": per_kernel,
        "merge_roofline": {"kernel": "bdlm_merge", "bound": "hbm", "achieved": merge["achieved_GBps"],
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": merge["frac_of_hbm_peak"],
                           "traffic": None, **merge},
        "cpu_baseline": cpu,
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


def bench_memory(args, dev, stream):
    """Peak device bytes of one rank's corrupted-block attention share under
    pure block parallelism (the clean prefix its blocks need held whole on the
    rank, with its gradient) and under CSBP (the rank's own clean shard, plus
    chunks of the other ranks' clean K/V received into two staging slots and
    their gradients handed off from two more), at 256K and 512K clean tokens,
    16 ranks, zigzag rank 0, blocks of 1024, 8192-token chunks, 32/8 heads,
    d = 128, bf16.  On one GPU, pinned host memory stands in for the other
    ranks: a chunk is received by a host-to-device copy and its gradient sent
    by a device-to-host copy.  Each scheme runs one forward + backward; the
    peak is torch's allocator peak over that step (every tensor of the
    scheme, inputs included, is allocated inside the measured region)."""
    import torch
    import masked_attention_bdlm_amd as M
    from masked_attention_bdlm_amd.csbp import (StagedBuffers, rank_blocks, share_backward_staged,
                                                share_forward_staged)
    R, B, C, hq, hkv, d = 16, 1024, 8192, 32, 8, 128
    dt = torch.bfloat16
    res = {}
    for L in (262144, 524288):
        nb = L // B
        ids = rank_blocks(nb, R, 0, "zigzag")
        T = len(ids) * B
        top = max(ids) * B                        # clean prefix the rank's blocks need
        scale = d ** -0.5
        # the other ranks' clean K/V and the gradients sent back: pinned host memory
        g = torch.Generator(device=dev).manual_seed(4)
        kc_h = torch.empty((1, L, hkv, d), dtype=dt, pin_memory=True)
        vc_h = torch.empty_like(kc_h, pin_memory=True)
        for j in range(0, L, C):
            kc_h[:, j:j + C].copy_(torch.randn((1, C, hkv, d), generator=g, device=dev).mul_(scale).to(dt))
            vc_h[:, j:j + C].copy_(torch.randn((1, C, hkv, d), generator=g, device=dev).mul_(scale).to(dt))
        dk_h = torch.empty_like(kc_h, pin_memory=True)
        dv_h = torch.empty_like(kc_h, pin_memory=True)

        def local():
            gl = torch.Generator(device=dev).manual_seed(5)
            q = (torch.randn((1, T, hq, d), generator=gl, device=dev) * scale).to(dt)
            k = (torch.randn((1, T, hkv, d), generator=gl, device=dev) * scale).to(dt)
            v = (torch.randn((1, T, hkv, d), generator=gl, device=dev) * scale).to(dt)
            do = torch.randn((1, T, hq, d), generator=gl, device=dev).to(dt)
            return q, k, v, do

        def measure(run):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base = torch.cuda.memory_allocated(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            t0 = time.perf_counter()
            run()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3
            peak = torch.cuda.max_memory_allocated(dev) - base
            torch.cuda.empty_cache()
            return peak, ms

        def pure_bp():
            q, k, v, do = local()
            kc = kc_h[:, :top].to(dev)             # the whole clean prefix, resident
            vc = vc_h[:, :top].to(dev)
            dkc, dvc = torch.empty_like(kc), torch.empty_like(vc)
            # the prefix buffer holds clean rows [0, top): one staged window over all of it
            o_acc, lse = M.share_fwd(q, k, v, kc, vc, ids, B, 0, top, 1, scale, stream=stream, seqlen=L,
                                     kv_staged=1)
            o, lse_f = M.merge_partials([o_acc], [lse], dt, stream=stream)
            dq = torch.zeros((1, T, hq, d), dtype=torch.float32, device=dev)
            dkx, dvx = torch.empty_like(k), torch.empty_like(v)
            M.share_bwd(q, k, v, kc, vc, ids, B, 0, top, 1, o, lse_f, do, dq, dkc, dvc, dkx, dvx, scale,
                        stream=stream, seqlen=L, kv_staged=1)
            dk_h[:, :top].copy_(dkc)
            dv_h[:, :top].copy_(dvc)

        def csbp():
            q, k, v, do = local()
            shard = torch.cat([torch.arange(b * B, (b + 1) * B) for b in ids])
            k_own = kc_h[:, shard].to(dev)          # the rank's own clean shard (resident on its owner)
            v_own = vc_h[:, shard].to(dev)
            dk_own, dv_own = torch.zeros_like(k_own), torch.zeros_like(v_own)   # its reduce-scatter result
            sb = StagedBuffers(q, k, hkv, C)

            def fetch(j0, j1, k_dst, v_dst):
                k_dst.copy_(kc_h[:, j0:j1], non_blocking=True)
                v_dst.copy_(vc_h[:, j0:j1], non_blocking=True)

            def deliver(j0, j1, dk, dv):
                dk_h[:, j0:j1].copy_(dk, non_blocking=True)
                dv_h[:, j0:j1].copy_(dv, non_blocking=True)
            o, lse = share_forward_staged(q, k, v, L, ids, B, C, fetch, scale, sb, stream)
            share_backward_staged(q, k, v, L, ids, B, C, o, lse, do, fetch, deliver, scale, sb, stream)
            torch.cuda.synchronize()
            del dk_own, dv_own, k_own, v_own

        log(f"memory L={L}: rank 0 blocks {len(ids)} (max id {max(ids)}), clean prefix {top} rows")
        bp_peak, bp_ms = measure(pure_bp)
        cs_peak, cs_ms = measure(csbp)
        row = 2 * hkv * d * 2                     # K and V bytes per clean token
        res[str(L)] = {
            "local_blocks": len(ids), "clean_prefix_rows": top,
            "pure_bp_peak_bytes": int(bp_peak), "csbp_peak_bytes": int(cs_peak),
            "ratio": round(bp_peak / cs_peak, 3),
            "pure_bp_clean_kv_and_grad_bytes": 2 * top * row,
            "csbp_clean_shard_and_staging_bytes": 2 * T * row + 4 * C * row,
            "pure_bp_step_ms": round(bp_ms, 2), "csbp_step_ms_incl_host_copies": round(cs_ms, 2),
        }
        log(f"  pure BP {bp_peak / 2**30:.3f} GiB, CSBP {cs_peak / 2**30:.3f} GiB")
        del kc_h, vc_h, dk_h, dv_h
    out = {
        "metric": "one rank's peak device bytes for its corrupted-block attention share: pure BP over CSBP "
                  "(16 ranks, zigzag rank 0), 1 GPU",
        "value": res["262144"]["ratio"], "unit": "x", "n_gpus": 1, "steps": 1, "warmup": 0,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "csbp_memory", "ranks": R, "block": B, "chunk": C, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "contexts": [262144, 524288], "parallelism": "single GPU (one rank)"},
        "by_context": res,
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_mfma_ceiling(dev, stream, iters: int = 1600000):
    """Sustained bf16 MFMA rate for four operand / instruction mixes
    (bdlm_calib_mfma, one launch of every SIMD's matrix core kept busy for
    about 0.2 s each): how far below the published 2516.6 TFLOP/s the chip's
    power limit holds the clock, and so the rate a fully busy matrix core
    reaches, with constant operands, random ones, and random ones beside the
    attention kernels' LDS operand traffic (1 KB per MFMA) or VALU work."""
    import torch
    from masked_attention_bdlm_amd.api import bdlm_calib_mfma
    wg = torch.cuda.get_device_properties(dev).multi_processor_count
    cycles = torch.zeros(wg * 16, dtype=torch.int64, device=dev)
    sink = torch.zeros(wg * 512, dtype=torch.float32, device=dev)
    names = ("constant_operands", "random_operands", "random_operands_lds_1KB_per_mfma",
             "random_operands_4_fma_per_mfma")
    modes = {}
    for mode, name in enumerate(names):
        bdlm_calib_mfma(mode, wg, iters // 10 // 2 * 2, cycles, sink, stream)   # warm the clock
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bdlm_calib_mfma(mode, wg, iters, cycles, sink, stream)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        c = cycles.view(-1, 2).double().cpu()
        clock = float(c[:, 0].sum() / c[:, 1].sum()) * 0.1          # GHz (ticks at 100 MHz)
        flop = wg * 8.0 * iters * 4 * 32768.0
        tf = flop / (ms * 1e-3) / 1e12
        modes[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "clock_GHz": round(clock, 3), "ms": round(ms, 2)}
        log(f"mfma ceiling {name}: {tf:.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:.1f} % of peak) "
            f"at {clock:.2f} GHz, {ms:.1f} ms")
    line = {
        "metric": "sustained bf16 MFMA TFLOP/s, every SIMD's matrix core busy (v_mfma_f32_32x32x16_bf16, "
                  "8 waves per CU), random operands",
        "value": modes["random_operands"]["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "higher_is_better": True, "peak": PEAK_BF16_TFLOPS, "workgroups": wg, "iters_per_wave": iters,
        "flop_per_launch": wg * 8.0 * iters * 4 * 32768.0, "modes": modes,
    }
    print(json.dumps(line), flush=True)


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
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the bf16 MFMA rate the chip sustains (calibration of the peak)")
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
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.mfma_ceiling:
        bench_mfma_ceiling(dev, stream)
        return
    if args.workload == "csbp_memory":
        bench_memory(args, dev, stream)
        return
    w = WORKLOADS[args.workload]
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
    # the contraction's own dtype sets the peak: bf16 MFMA, or fp32 MFMA for the fp32 path
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    per_kernel = {}
    for name, fl in kernel_flop.items():
        kk = kernels.get(name)
        if kk:
            a = fl / (kk["avg_ms"] * 1e-3) / 1e12
            per_kernel[name] = {"achieved": round(a, 2), "frac": round(a / peak, 4),
                                "avg_launch_ms": round(kk["avg_ms"], 4), "flop_per_launch": fl}
    if "bdlm_dq" in per_kernel:
        # the dQ product alone is 2 d P; the kernel also recomputes S and dP^T
        alg = per_kernel["bdlm_dq"]["achieved"] / 3.0
        per_kernel["bdlm_dq"]["executed_flop_per_launch"] = kernel_flop["bdlm_dq"]
        per_kernel["bdlm_dq"]["algorithmic_2dP_achieved"] = round(alg, 2)
        per_kernel["bdlm_dq"]["algorithmic_2dP_frac"] = round(alg / peak, 4)
    roof = None
    timed = [n for n in kernel_flop if n in kernels]
    if timed:
        dom = max(timed, key=lambda n: kernels[n]["total_ms"])
        pk = per_kernel[dom]
        traffic = measured_traffic(dom) if w.name == "gqa_64k" else None
        roof = {"kernel": dom, "bound": "mfma", "achieved": pk["achieved"], "peak": peak,
                "unit": "TFLOP/s", "frac": pk["frac"],
                "traffic": None if traffic is None else round(traffic),
                "traffic_unit": "bytes per launch (HBM, counter-calibrated)",
                "flop_per_launch": pk["flop_per_launch"], "avg_launch_ms": pk["avg_launch_ms"]}
    extra = {"kernel_roofline": per_kernel}

    cpu = None
    if not args.no_cpu:
        if w.name == "tiny_f32":
            log("timing the fp64 oracle on the whole problem (CPU baseline)")
            cpu = cpu_full_oracle(w, x)
        else:
            log("timing the fp64 oracle on sampled units (CPU baseline)")
            cpu = cpu_baseline(w, x, seconds_budget=args.cpu_seconds)

    if w.name == "gqa_64k":
        metric = "BDLM attn fwd+bwd useful TFLOP/s and % bf16 MFMA peak at 2L=64K, 1 GPU"
    else:
        metric = (f"BDLM attn fwd+bwd useful TFLOP/s and % {'bf16' if w.dtype == 'bf16' else 'fp32'} MFMA peak "
                  f"at 2L={2 * w.seqlen}, 1 GPU")
    out = {
        "metric": metric,
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
        "pct_of_peak": round(100.0 * value / peak, 2),
        "strict_12_tflops": round(strict / (ms * 1e-3) / 1e12, 3),
        "useful_flop_per_step": useful,
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in kernels.items()},
        # forward and backward separately (per step, from the kernels' HIP events)
        "fwd_ms": round(kernels.get("bdlm_fwd", {}).get("total_ms", 0.0) / args.steps, 4),
        "bwd_ms": round(sum(kernels.get(n, {}).get("total_ms", 0.0)
                            for n in ("bdlm_bwd_pre", "bdlm_dkdv", "bdlm_dq")) / args.steps, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
