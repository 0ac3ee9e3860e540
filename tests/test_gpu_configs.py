"""GPU parity at the full workload sizes, in the launch configuration bench.py
times.

The oracle runs on seeded sampled units (batch, stream, block, q-head): 64
units per configuration, always including the first and last block of each
stream.  Inside a unit the oracle takes a seeded subset of the block's rows
(first and last row always; every row when the block has at most that many):
O, LSE and dQ are row-local, so they are exact on those rows.  dK/dV are
checked with a second backward whose dO is zero outside the sampled rows: the
GPU's dK/dV must then equal the oracle's contributions of those rows, and be
exactly zero on keys no sampled row sees.  The 8K MHA configuration runs the
full oracle on every (batch, head).  Every configuration also has a "sharp"
variant (Q and K drawn unscaled, logits ~ N(0, 1)), because the pre-scaled
inputs make the softmax nearly uniform.  The oracle's units run on a thread
pool; each one is the oracle's own per-unit function."""
import numpy as np
import pytest
import torch

import masked_attention_bdlm_amd as M
from masked_attention_bdlm_amd import csbp
from oracle import bdlm_oracle as O
from synth import WORKLOADS, draw_units, make_full_inputs, make_share_inputs, to_f64
from tests.gpu_util import (TOL_REL, announce, check_outputs, gpu_full, mask_dout, rel_fro, require_gpu,
                            row_sample, run_parallel)

pytestmark = pytest.mark.gpu

UNITS = 64            # sampled units per configuration (the configurations' statement)
ROWS = 64             # rows per unit (all rows when B <= 64)


def _rows(offs, blk, B, dev):
    return torch.as_tensor(blk * B + np.asarray(offs), device=dev)


def _kv_all(x, b, g):
    """fp64 host copy of kv head g's 2L keys and values, [clean ; corrupted]."""
    k = to_f64(torch.cat([x["kc"][b, :, g], x["kx"][b, :, g]]))
    v = to_f64(torch.cat([x["vc"][b, :, g], x["vx"][b, :, g]]))
    return k, v


def _sampled_check(w, x, got, n_units, rows_per_unit, label):
    """Compare GPU outputs `got` with the oracle on sampled units, then run the
    dO-masked backward and compare dK/dV."""
    B, L = w.block, w.seqlen
    rep = w.hq // w.hkv
    dev = x["qc"].device
    units = draw_units(w.nblocks, w.hq, w.batch, n_units, w.seed)
    offs = row_sample(B, rows_per_unit, w.seed + 7)
    announce(f"{label}: {len(units)} units x {len(offs)} rows of B={B}")
    kv = {}
    for (b, st, blk, h) in units.tolist():
        if (b, h // rep) not in kv:
            kv[(b, h // rep)] = _kv_all(x, b, h // rep)
    jobs = []
    for n, (b, st, blk, h) in enumerate(units.tolist()):
        rows = _rows(offs, blk, B, dev)
        s = "c" if st == 0 else "x"
        jobs.append(dict(n=n, b=b, st=st, blk=blk, h=h, g=h // rep,
                         q=to_f64(x["q" + s][b, rows, h]), do=to_f64(x["do" + s][b, rows, h]),
                         got_o=to_f64(got["o" + s][b, rows, h]), got_lse=to_f64(got["lse_" + s][b, h, rows]),
                         got_dq=to_f64(got["dq" + s][b, rows, h])))
    dk_s = np.zeros((w.batch, 2 * L, w.hkv, w.head_dim))
    dv_s = np.zeros_like(dk_s)
    per = {}

    def fn(j):
        k_all, v_all = kv[(j["b"], j["g"])]
        mask = O.bdlm_mask_rows(L, B, j["st"] * L + j["blk"] * B + offs)
        return O.unit_rows_fwd_bwd(j["q"], k_all, v_all, mask, j["do"], w.scale)

    def consume(j, r):
        o, lse, dq, dk, dv = r
        per[j["n"]] = (o, lse, dq)
        dk_s[j["b"], :, j["g"]] += dk
        dv_s[j["b"], :, j["g"]] += dv

    run_parallel(jobs, fn, consume)
    gg = {"oc": np.concatenate([j["got_o"] for j in jobs]), "lse_c": np.concatenate([j["got_lse"] for j in jobs]),
          "dqc": np.concatenate([j["got_dq"] for j in jobs])}
    rr = {"oc": np.concatenate([per[j["n"]][0] for j in jobs]),
          "lse_c": np.concatenate([per[j["n"]][1] for j in jobs]),
          "dqc": np.concatenate([per[j["n"]][2] for j in jobs])}
    rep_ = check_outputs(gg, rr, w.dtype, where=label)
    announce(f"{label} sampled rows: {rep_}")

    doc2, dox2 = mask_dout(x, units, offs, B)
    _, dkc, dvc, _, dkx, dvx = M.attention_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"],
                                               got["oc"], got["ox"], got["lse_c"], got["lse_x"],
                                               doc2, dox2, B, w.scale)
    torch.cuda.synchronize()
    dk = np.concatenate([to_f64(dkc), to_f64(dkx)], axis=1)
    dv = np.concatenate([to_f64(dvc), to_f64(dvx)], axis=1)
    seen = np.any(dv_s != 0, axis=-1)            # [batch, 2L, Hkv]
    assert not np.any(dk[~seen]) and not np.any(dv[~seen]), f"{label}: non-zero dK/dV on unseen keys"
    ek, ev = rel_fro(dk, dk_s), rel_fro(dv, dv_s)
    announce(f"{label} dO-masked dK rel {ek:.3e} dV rel {ev:.3e}")
    assert ek <= TOL_REL and ev <= TOL_REL


@pytest.mark.parametrize("sharp", [False, True], ids=["prescaled", "sharp"])
def test_mha_8k_full_oracle_on_every_head(sharp):
    """batch 2, L=4096, B=32, 16/16 heads: the full oracle (explicit 8192 x 8192
    mask) on every (batch, head), all outputs of both streams."""
    require_gpu()
    w = WORKLOADS["mha_8k"]
    label = w.name + (" sharp" if sharp else "")
    announce(label)
    x = make_full_inputs(w, device="cuda", sharp=sharp)
    got = gpu_full(x, w.block, w.scale)
    L, B = w.seqlen, w.block
    mask = O.bdlm_mask(L, B)
    cat = lambda a, c: np.concatenate([to_f64(a), to_f64(c)])
    jobs = []
    for b in range(w.batch):
        for h in range(w.hq):
            jobs.append(dict(b=b, h=h, q=cat(x["qc"][b, :, h], x["qx"][b, :, h]),
                             k=cat(x["kc"][b, :, h], x["kx"][b, :, h]), v=cat(x["vc"][b, :, h], x["vx"][b, :, h]),
                             do=cat(x["doc"][b, :, h], x["dox"][b, :, h])))
    worst = {}

    def fn(j):
        o, lse, p = O.attention_fwd(j["q"], j["k"], j["v"], mask, w.scale)
        dq, dk, dv = O.attention_bwd(j["q"], j["k"], j["v"], p, o, j["do"], w.scale)
        return o, lse, dq, dk, dv

    def consume(j, r):
        o, lse, dq, dk, dv = r
        b, h = j["b"], j["h"]
        gg = dict(oc=cat(got["oc"][b, :, h], got["ox"][b, :, h]), lse_c=cat(got["lse_c"][b, h], got["lse_x"][b, h]),
                  dqc=cat(got["dqc"][b, :, h], got["dqx"][b, :, h]), dkc=cat(got["dkc"][b, :, h], got["dkx"][b, :, h]),
                  dvc=cat(got["dvc"][b, :, h], got["dvx"][b, :, h]))
        rep = check_outputs(gg, dict(oc=o, lse_c=lse, dqc=dq, dkc=dk, dvc=dv), w.dtype, where=f"{label} b{b}h{h}")
        for k_, v_ in rep.items():
            worst[k_] = max(worst.get(k_, v_), v_)

    run_parallel(jobs, fn, consume, workers=8)
    announce(f"{label}: {len(jobs)} (batch, head) pairs, worst {worst}")


@pytest.mark.parametrize("sharp", [False, True], ids=["prescaled", "sharp"])
def test_gqa_64k_sampled(sharp):
    """Headline shape: batch 1, L=32768, B=64, 32/8 heads, 1 % outlier keys
    (sharp: unscaled Q/K, logits ~ N(0,1), outlier logits ~ N(0, 64))."""
    require_gpu()
    w = WORKLOADS["gqa_64k"]
    x = make_full_inputs(w, device="cuda", sharp=sharp)
    got = gpu_full(x, w.block, w.scale)
    _sampled_check(w, x, got, UNITS, ROWS, w.name + ("_sharp" if sharp else ""))


def test_gqa_64k_zero_query_closed_form_and_invariants():
    """Q = 0 at full size: LSE = log((b+1)B) on every row of both streams, O =
    mean of the visible V rows.  With the real inputs: sum_k dV = sum_q dO per
    kv head, sum_k dK = 0."""
    require_gpu()
    w = WORKLOADS["gqa_64k"]
    announce(w.name + " Q=0")
    x = make_full_inputs(w, device="cuda")
    L, B = w.seqlen, w.block
    z = torch.zeros_like(x["qc"])
    oc, ox, lc, lx = M.attention_fwd(z, x["kc"], x["vc"], z, x["kx"], x["vx"], B, w.scale)
    torch.cuda.synchronize()
    blk = np.arange(L) // B
    want = np.log((blk + 1) * B)
    for lse in (lc, lx):
        e = np.max(np.abs(to_f64(lse[0]) - want[None, :]))
        assert e <= 1e-5 * want.max(), e
    vc, vx = to_f64(x["vc"][0]), to_f64(x["vx"][0])            # [L, Hkv, d]
    csum = np.cumsum(vc, axis=0)
    ends = (blk + 1) * B - 1
    clean_mean = csum[ends] / ((blk + 1) * B)[:, None, None]
    prefix = np.where(blk[:, None, None] > 0, csum[np.maximum(blk * B - 1, 0)], 0.0)
    own = vx.reshape(L // B, B, *vx.shape[1:]).sum(axis=1)[blk]
    noisy_mean = (prefix + own) / ((blk + 1) * B)[:, None, None]
    rep = w.hq // w.hkv
    ocm = to_f64(oc[0]).reshape(L, w.hkv, rep, -1)
    oxm = to_f64(ox[0]).reshape(L, w.hkv, rep, -1)
    assert rel_fro(ocm, np.repeat(clean_mean[:, :, None], rep, axis=2)) <= 5e-3
    assert rel_fro(oxm, np.repeat(noisy_mean[:, :, None], rep, axis=2)) <= 5e-3

    got = gpu_full(x, B, w.scale)
    dv_sum = to_f64(got["dvc"][0]).sum(0) + to_f64(got["dvx"][0]).sum(0)           # [Hkv, d]
    do_sum = (to_f64(x["doc"][0]).sum(0) + to_f64(x["dox"][0]).sum(0)).reshape(w.hkv, rep, -1).sum(1)
    assert rel_fro(dv_sum, do_sum) <= 1e-2
    dk = np.concatenate([to_f64(got["dkc"][0]), to_f64(got["dkx"][0])])
    assert np.linalg.norm(dk.sum(0)) <= 1e-2 * np.abs(dk).sum(0).mean() * np.sqrt(dk.shape[-1] * w.hkv)


@pytest.mark.parametrize("sharp", [False, True], ids=["prescaled", "sharp"])
@pytest.mark.parametrize("B", [128, 256, 512, 1024])
def test_sweep_256k_sampled(B, sharp):
    """batch 1, L=131072 (2L = 256K), 32/8 heads, one B of the sweep: 64
    sampled query blocks, 64 rows each."""
    require_gpu()
    w = WORKLOADS[f"sweep_256k_B{B}"]
    x = make_full_inputs(w, device="cuda", sharp=sharp)
    got = gpu_full(x, w.block, w.scale)
    _sampled_check(w, x, got, UNITS, ROWS, w.name + ("_sharp" if sharp else ""))
    del x, got
    torch.cuda.empty_cache()


def _share_units(nblocks, hq, count, seed):
    """(local block, q-head) units: the first and last local block always, the
    rest drawn without repetition, sorted by kv-head order of the heads."""
    rng = np.random.default_rng(seed)
    units = [(i, int(rng.integers(hq))) for i in (0, nblocks - 1)]
    while len(units) < min(count, nblocks * hq):
        u = (int(rng.integers(nblocks)), int(rng.integers(hq)))
        if u not in units:
            units.append(u)
    return units


def _share_check(w, x, q_name, do_name, ids, units, offs, key_end, own, o, lse, dq, dmasked, label):
    """Sampled rows of a share's (O, LSE, dQ) against the oracle's attention of
    each local block over its keys ([0, key_end(id)) of the clean sequence,
    plus its own corrupted block when `own`), then the dO-masked backward's
    clean (and own-block) dK/dV against those rows' contributions.  dmasked
    runs the share's backward with a given dO and returns (dkc, dvc, dkx, dvx)."""
    B, L = w.block, w.seqlen
    rep = w.hq // w.hkv
    dev = x[q_name].device
    kc_h = {g: to_f64(x["kc"][0, :, g]) for g in range(w.hkv)}
    vc_h = {g: to_f64(x["vc"][0, :, g]) for g in range(w.hkv)}
    T = len(ids) * B
    dkc_s = np.zeros((L, w.hkv, w.head_dim))
    dvc_s = np.zeros_like(dkc_s)
    dkx_s = np.zeros((T, w.hkv, w.head_dim))
    dvx_s = np.zeros_like(dkx_s)
    jobs = []
    for n, (i, h) in enumerate(units):
        rows = _rows(offs, i, B, dev)
        g = h // rep
        jobs.append(dict(n=n, i=i, h=h, g=g, q=to_f64(x[q_name][0, rows, h]), do=to_f64(x[do_name][0, rows, h]),
                         own_k=to_f64(x["kx"][0, i * B:(i + 1) * B, g]) if own else None,
                         own_v=to_f64(x["vx"][0, i * B:(i + 1) * B, g]) if own else None,
                         got=(to_f64(o[0, rows, h]), to_f64(lse[0, h, rows]), to_f64(dq[0, rows, h]))))
    per = {}

    def fn(j):
        e = key_end(ids[j["i"]])
        keys, vals = kc_h[j["g"]][:e], vc_h[j["g"]][:e]
        if own:
            keys = np.concatenate([keys, j["own_k"]])
            vals = np.concatenate([vals, j["own_v"]])
        ro, rl, p = O.attention_fwd(j["q"], keys, vals, np.ones((len(offs), len(keys)), dtype=bool), w.scale)
        rdq, rdk, rdv = O.attention_bwd(j["q"], keys, vals, p, ro, j["do"], w.scale)
        return ro, rl, rdq, rdk, rdv, e

    def consume(j, r):
        ro, rl, rdq, rdk, rdv, e = r
        per[j["n"]] = (ro, rl, rdq)
        i, g = j["i"], j["g"]
        dkc_s[:e, g] += rdk[:e]
        dvc_s[:e, g] += rdv[:e]
        if own:
            dkx_s[i * B:(i + 1) * B, g] += rdk[e:]
            dvx_s[i * B:(i + 1) * B, g] += rdv[e:]

    run_parallel(jobs, fn, consume)
    gg = {"ox": np.concatenate([j["got"][0] for j in jobs]), "lse_x": np.concatenate([j["got"][1] for j in jobs]),
          "dqx": np.concatenate([j["got"][2] for j in jobs])}
    rr = {"ox": np.concatenate([per[j["n"]][0] for j in jobs]),
          "lse_x": np.concatenate([per[j["n"]][1] for j in jobs]),
          "dqx": np.concatenate([per[j["n"]][2] for j in jobs])}
    rep_ = check_outputs(gg, rr, w.dtype, where=label)
    announce(f"{label} sampled rows ({len(units)} units x {len(offs)} rows): {rep_}")
    do2 = torch.zeros_like(x[do_name])
    for (i, h) in units:
        rows = _rows(offs, i, B, dev)
        do2[0, rows, h] = x[do_name][0, rows, h]
    g_dkc, g_dvc, g_dkx, g_dvx = dmasked(do2)
    torch.cuda.synchronize()
    checks = [("dkc", g_dkc, dkc_s), ("dvc", g_dvc, dvc_s)]
    if own:
        checks += [("dkx", g_dkx, dkx_s), ("dvx", g_dvx, dvx_s)]
    for name, gt, ref in checks:
        a = to_f64(gt[0])
        seen = np.any(ref != 0, axis=-1)
        assert not np.any(a[~seen]), f"{label} {name}: non-zero gradient on unseen keys"
        e = rel_fro(a, ref)
        announce(f"{label} dO-masked {name} rel {e:.3e}")
        assert e <= TOL_REL, (name, e)


@pytest.mark.parametrize("sharp", [False, True], ids=["prescaled", "sharp"])
def test_csbp_share_256k_sampled(sharp):
    """One rank's CSBP share at 256K: 16 blocks of 1024 at seeded positions,
    clean prefix streamed in 8192-token chunks with the online merge; 64
    sampled (block, head) units of 64 rows."""
    require_gpu()
    w = WORKLOADS["csbp_share_256k"]
    label = w.name + ("_sharp" if sharp else "")
    announce(label)
    x = make_share_inputs(w, device="cuda", sharp=sharp)
    ids = [int(i) for i in x["block_ids"]]
    B = w.block
    bufs = csbp.ShareBuffers(x["qx"], x["kc"], x["kx"])
    o, lse = csbp.share_forward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, w.scale, bufs)
    o, lse = o.clone(), lse.clone()
    dqx = csbp.share_backward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse,
                              x["dox"], w.scale, bufs)[0].clone()
    torch.cuda.synchronize()

    def dmasked(do2):
        return csbp.share_backward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse,
                                   do2, w.scale, bufs)[1:]

    units = _share_units(len(ids), w.hq, UNITS, w.seed + 100)
    _share_check(w, x, "qx", "dox", ids, units, row_sample(B, ROWS, w.seed + 7), lambda bid: bid * B, True,
                 o, lse, dqx, dmasked, label)


@pytest.mark.parametrize("sharp", [False, True], ids=["prescaled", "sharp"])
def test_csbp_rank_256k_clean_shard_sampled(sharp):
    """The clean-query half of one rank's share at 256K: the rank's zigzag shard
    of 16 clean blocks of 1024 against the streamed clean K/V (each block sees
    its own and every earlier clean block); 64 sampled (block, head) units of
    64 rows against the oracle's attention over the block's inclusive prefix,
    and the dO-masked rerun's dK/dV against those rows' contributions."""
    require_gpu()
    w = WORKLOADS["csbp_rank_256k"]
    label = w.name + " clean shard" + (" sharp" if sharp else "")
    announce(label)
    x = make_share_inputs(w, device="cuda", sharp=sharp)
    ids = [int(i) for i in x["clean_ids"]]
    B = w.block
    bufs = csbp.ShareBuffers(x["qs"], x["kc"])
    o, lse = csbp.clean_share_forward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, w.scale, bufs)
    o, lse = o.clone(), lse.clone()
    dq = csbp.clean_share_backward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse, x["dos"], w.scale,
                                   bufs)[0].clone()
    torch.cuda.synchronize()

    def dmasked(do2):
        _, dkc, dvc = csbp.clean_share_backward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse, do2,
                                                w.scale, bufs)
        return dkc, dvc, None, None

    units = _share_units(len(ids), w.hq, UNITS, w.seed + 200)
    _share_check(w, x, "qs", "dos", ids, units, row_sample(B, ROWS, w.seed + 9), lambda cid: (cid + 1) * B, False,
                 o, lse, dq, dmasked, label)


def test_csbp_share_256k_staged_equals_resident():
    """At full size (16 blocks of 1024, 256K clean tokens, 8192-token chunks)
    the staged share step (clean K/V received chunk by chunk into two staging
    slots, clean dK/dV handed off per chunk) is bit-identical to the step that
    reads the resident clean K/V."""
    require_gpu()
    w = WORKLOADS["csbp_share_256k"]
    announce(w.name + " staged")
    x = make_share_inputs(w, device="cuda")
    ids = [int(i) for i in x["block_ids"]]
    B, L, C = w.block, w.seqlen, w.share_chunk
    bufs = csbp.ShareBuffers(x["qx"], x["kc"], x["kx"])
    o, lse = (t.clone() for t in csbp.share_forward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, C,
                                                    w.scale, bufs))
    ref = [t.clone() for t in csbp.share_backward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, C, o, lse,
                                                  x["dox"], w.scale, bufs)]
    del bufs
    sb = csbp.StagedBuffers(x["qx"], x["kx"], w.hkv, C)
    dkc, dvc = torch.zeros_like(x["kc"]), torch.zeros_like(x["vc"])

    def fetch(j0, j1, k_dst, v_dst):
        k_dst.copy_(x["kc"][:, j0:j1])
        v_dst.copy_(x["vc"][:, j0:j1])

    def deliver(j0, j1, dk, dv):
        dkc[:, j0:j1].copy_(dk)
        dvc[:, j0:j1].copy_(dv)

    so, slse = csbp.share_forward_staged(x["qx"], x["kx"], x["vx"], L, ids, B, C, fetch, w.scale, sb)
    assert torch.equal(so, o) and torch.equal(slse, lse)
    sdq, sdkx, sdvx = csbp.share_backward_staged(x["qx"], x["kx"], x["vx"], L, ids, B, C, so, slse, x["dox"],
                                                 fetch, deliver, w.scale, sb)
    torch.cuda.synchronize()
    for name, a, b in (("dqx", sdq, ref[0]), ("dkc", dkc, ref[1]), ("dvc", dvc, ref[2]), ("dkx", sdkx, ref[3]),
                       ("dvx", sdvx, ref[4])):
        assert torch.equal(a, b), name
