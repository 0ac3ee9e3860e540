"""GPU parity at the full workload sizes, in the launch configuration bench.py
times.  The oracle runs on seeded sampled units (batch, stream, block, q-head),
optionally on a seeded subset of rows inside each block; O, LSE and dQ are
row-local, so they are exact on those rows.  dK/dV are checked with a second
backward whose dO is zero outside the sampled rows: the GPU's dK/dV must then
equal the oracle's contributions of those rows, and be exactly zero on keys no
sampled row sees."""
import numpy as np
import pytest
import torch

import masked_attention_bdlm_amd as M
from masked_attention_bdlm_amd import csbp
from oracle import bdlm_oracle as O
from synth import WORKLOADS, draw_units, make_full_inputs, make_share_inputs, to_f64
from tests.gpu_util import (HostView, announce, check_outputs, gpu_full, mask_dout, rel_fro,
                            require_gpu, row_sample, TOL_REL)

pytestmark = pytest.mark.gpu


def _rows(offs, blk, B, dev):
    return torch.as_tensor(blk * B + np.asarray(offs), device=dev)


def _sampled_check(w, x, got, n_units, rows_per_unit, label):
    """Compare GPU outputs `got` with the oracle on sampled units, then run the
    dO-masked backward and compare dK/dV."""
    B = w.block
    dev = x["qc"].device
    units = draw_units(w.nblocks, w.hq, w.batch, n_units, w.seed)
    offs = row_sample(B, rows_per_unit, w.seed + 7)
    hv = {k: HostView(v) for k, v in x.items()}
    res, dk_s, dv_s = O.sampled_fwd_bwd(hv["qc"], hv["kc"], hv["vc"], hv["qx"], hv["kx"], hv["vx"],
                                        hv["doc"], hv["dox"], B, w.scale, units, row_offsets=offs)
    g, r = {"o": [], "lse": [], "dq": []}, {"o": [], "lse": [], "dq": []}
    for u in res:
        b, st, blk, h = u["unit"]
        s = "c" if st == 0 else "x"
        rows = _rows(offs, blk, B, dev)
        g["o"].append(to_f64(got["o" + s][b, rows, h]))
        g["lse"].append(to_f64(got["lse_" + s][b, h, rows]))
        g["dq"].append(to_f64(got["dq" + s][b, rows, h]))
        r["o"].append(u["o"])
        r["lse"].append(u["lse"])
        r["dq"].append(u["dq"])
    gg = {"oc": np.concatenate(g["o"]), "lse_c": np.concatenate(g["lse"]), "dqc": np.concatenate(g["dq"])}
    rr = {"oc": np.concatenate(r["o"]), "lse_c": np.concatenate(r["lse"]), "dqc": np.concatenate(r["dq"])}
    rep = check_outputs(gg, rr, w.dtype, where=label)
    announce(f"{label} sampled rows: {rep}")

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


def test_mha_8k_full_oracle_on_heads():
    """batch 2, L=4096, B=32, 16/16 heads: the full oracle on three whole heads."""
    require_gpu()
    w = WORKLOADS["mha_8k"]
    announce(w.name)
    x = make_full_inputs(w, device="cuda")
    got = gpu_full(x, w.block, w.scale)
    L, B = w.seqlen, w.block
    mask = O.bdlm_mask(L, B)
    for (b, h) in [(0, 0), (1, 7), (0, 15)]:
        q = np.concatenate([to_f64(x["qc"][b, :, h]), to_f64(x["qx"][b, :, h])])
        k = np.concatenate([to_f64(x["kc"][b, :, h]), to_f64(x["kx"][b, :, h])])
        v = np.concatenate([to_f64(x["vc"][b, :, h]), to_f64(x["vx"][b, :, h])])
        do = np.concatenate([to_f64(x["doc"][b, :, h]), to_f64(x["dox"][b, :, h])])
        o, lse, p = O.attention_fwd(q, k, v, mask, w.scale)
        dq, dk, dv = O.attention_bwd(q, k, v, p, o, do, w.scale)
        del p
        cat = lambda a, c: np.concatenate([to_f64(a), to_f64(c)])
        gg = dict(oc=cat(got["oc"][b, :, h], got["ox"][b, :, h]),
                  lse_c=cat(got["lse_c"][b, h], got["lse_x"][b, h]),
                  dqc=cat(got["dqc"][b, :, h], got["dqx"][b, :, h]),
                  dkc=cat(got["dkc"][b, :, h], got["dkx"][b, :, h]),
                  dvc=cat(got["dvc"][b, :, h], got["dvx"][b, :, h]))
        rep = check_outputs(gg, dict(oc=o, lse_c=lse, dqc=dq, dkc=dk, dvc=dv), w.dtype, where=f"{w.name} b{b}h{h}")
        announce(f"{w.name} (b={b}, h={h}): {rep}")


def test_gqa_64k_sampled():
    """Headline shape: batch 1, L=32768, B=64, 32/8 heads, 1 % outlier keys."""
    require_gpu()
    w = WORKLOADS["gqa_64k"]
    announce(w.name)
    x = make_full_inputs(w, device="cuda")
    got = gpu_full(x, w.block, w.scale)
    _sampled_check(w, x, got, 64, 64, w.name)


def test_gqa_64k_sharp_sampled():
    """Same shape with unscaled Q/K (logits ~ N(0,1), outlier logits ~ N(0, 64))."""
    require_gpu()
    w = WORKLOADS["gqa_64k"]
    announce(w.name + " sharp")
    x = make_full_inputs(w, device="cuda", sharp=True)
    got = gpu_full(x, w.block, w.scale)
    _sampled_check(w, x, got, 32, 64, w.name + "_sharp")


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


@pytest.mark.parametrize("B", [128, 256, 512, 1024])
def test_sweep_256k_sampled(B):
    """batch 1, L=131072 (2L = 256K), 32/8 heads, one B of the sweep."""
    require_gpu()
    w = WORKLOADS[f"sweep_256k_B{B}"]
    announce(w.name)
    x = make_full_inputs(w, device="cuda")
    got = gpu_full(x, w.block, w.scale)
    _sampled_check(w, x, got, 24, 32, w.name)


def test_csbp_share_256k_sampled():
    """One rank's CSBP share at 256K: 16 blocks of 1024 at seeded positions,
    clean prefix streamed in 8192-token chunks with the online merge."""
    require_gpu()
    w = WORKLOADS["csbp_share_256k"]
    announce(w.name)
    x = make_share_inputs(w, device="cuda")
    ids = [int(i) for i in x["block_ids"]]
    B, L = w.block, w.seqlen
    bufs = csbp.ShareBuffers(x["qx"], x["kc"], x["kx"])
    o, lse = csbp.share_forward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, w.scale, bufs)
    o, lse = o.clone(), lse.clone()
    dqx, dkc, dvc, dkx, dvx = (t.clone() for t in csbp.share_backward(
        x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse, x["dox"], w.scale, bufs))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 100)
    units = [(i, int(rng.integers(w.hq))) for i in (0, len(ids) - 1)]
    while len(units) < 24:
        u = (int(rng.integers(len(ids))), int(rng.integers(w.hq)))
        if u not in units:
            units.append(u)
    offs = row_sample(B, 32, w.seed + 7)
    kc_h, vc_h = HostView(x["kc"]), HostView(x["vc"])
    gs, rs = {"o": [], "lse": [], "dq": []}, {"o": [], "lse": [], "dq": []}
    dkc_s = np.zeros((L, w.hkv, w.head_dim))
    dvc_s = np.zeros_like(dkc_s)
    T = len(ids) * B
    dkx_s = np.zeros((T, w.hkv, w.head_dim))
    dvx_s = np.zeros_like(dkx_s)
    dox2 = torch.zeros_like(x["dox"])
    for (i, h) in units:
        g = h // (w.hq // w.hkv)
        bid = ids[i]
        rows = _rows(offs, i, B, x["qx"].device)
        keys = np.concatenate([kc_h[0, :bid * B, g], to_f64(x["kx"][0, i * B:(i + 1) * B, g])])
        vals = np.concatenate([vc_h[0, :bid * B, g], to_f64(x["vx"][0, i * B:(i + 1) * B, g])])
        q = to_f64(x["qx"][0, rows, h])
        do = to_f64(x["dox"][0, rows, h])
        ro, rl, p = O.attention_fwd(q, keys, vals, np.ones((len(offs), len(keys)), dtype=bool), w.scale)
        rdq, rdk, rdv = O.attention_bwd(q, keys, vals, p, ro, do, w.scale)
        del p
        gs["o"].append(to_f64(o[0, rows, h])); rs["o"].append(ro)
        gs["lse"].append(to_f64(lse[0, h, rows])); rs["lse"].append(rl)
        gs["dq"].append(to_f64(dqx[0, rows, h])); rs["dq"].append(rdq)
        dkc_s[:bid * B, g] += rdk[:bid * B]
        dvc_s[:bid * B, g] += rdv[:bid * B]
        dkx_s[i * B:(i + 1) * B, g] += rdk[bid * B:]
        dvx_s[i * B:(i + 1) * B, g] += rdv[bid * B:]
        dox2[0, rows, h] = x["dox"][0, rows, h]
    gg = {k + ("x" if k != "lse" else "_x"): np.concatenate(v) for k, v in gs.items()}
    rr = {k + ("x" if k != "lse" else "_x"): np.concatenate(v) for k, v in rs.items()}
    rep = check_outputs(gg, rr, w.dtype, where=w.name)
    announce(f"{w.name} sampled rows: {rep}")
    _, g_dkc, g_dvc, g_dkx, g_dvx = csbp.share_backward(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B,
                                                         w.share_chunk, o, lse, dox2, w.scale, bufs)
    torch.cuda.synchronize()
    for name, gt, ref in (("dkc", g_dkc, dkc_s), ("dvc", g_dvc, dvc_s), ("dkx", g_dkx, dkx_s),
                          ("dvx", g_dvx, dvx_s)):
        a = to_f64(gt[0])
        seen = np.any(ref != 0, axis=-1)
        assert not np.any(a[~seen]), f"{name}: non-zero gradient on unseen keys"
        e = rel_fro(a, ref)
        announce(f"{w.name} dO-masked {name} rel {e:.3e}")
        assert e <= TOL_REL, (name, e)


def test_csbp_rank_256k_clean_shard_sampled():
    """The clean-query half of one rank's share at 256K: the rank's zigzag shard
    of 16 clean blocks of 1024 against the streamed clean K/V (each block sees
    its own and every earlier clean block).  Sampled rows of O, LSE and dQ
    against the oracle's attention over the block's inclusive prefix, and the
    dO-masked rerun's dK/dV against those rows' contributions."""
    require_gpu()
    w = WORKLOADS["csbp_rank_256k"]
    announce(w.name + " clean shard")
    x = make_share_inputs(w, device="cuda")
    ids = [int(i) for i in x["clean_ids"]]
    B, L = w.block, w.seqlen
    bufs = csbp.ShareBuffers(x["qs"], x["kc"])
    o, lse = csbp.clean_share_forward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, w.scale, bufs)
    o, lse = o.clone(), lse.clone()
    dq, _, _ = (t.clone() for t in csbp.clean_share_backward(
        x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse, x["dos"], w.scale, bufs))
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 200)
    units = [(i, int(rng.integers(w.hq))) for i in (0, len(ids) - 1)]
    while len(units) < 16:
        u = (int(rng.integers(len(ids))), int(rng.integers(w.hq)))
        if u not in units:
            units.append(u)
    offs = row_sample(B, 32, w.seed + 9)
    kc_h, vc_h = HostView(x["kc"]), HostView(x["vc"])
    gs, rs = {"o": [], "lse": [], "dq": []}, {"o": [], "lse": [], "dq": []}
    dkc_s = np.zeros((L, w.hkv, w.head_dim))
    dvc_s = np.zeros_like(dkc_s)
    dos2 = torch.zeros_like(x["dos"])
    for (i, h) in units:
        g = h // (w.hq // w.hkv)
        cid = ids[i]
        rows = _rows(offs, i, B, x["qs"].device)
        keys, vals = kc_h[0, :(cid + 1) * B, g], vc_h[0, :(cid + 1) * B, g]
        q = to_f64(x["qs"][0, rows, h])
        do = to_f64(x["dos"][0, rows, h])
        ro, rl, p = O.attention_fwd(q, keys, vals, np.ones((len(offs), len(keys)), dtype=bool), w.scale)
        rdq, rdk, rdv = O.attention_bwd(q, keys, vals, p, ro, do, w.scale)
        del p
        gs["o"].append(to_f64(o[0, rows, h])); rs["o"].append(ro)
        gs["lse"].append(to_f64(lse[0, h, rows])); rs["lse"].append(rl)
        gs["dq"].append(to_f64(dq[0, rows, h])); rs["dq"].append(rdq)
        dkc_s[:(cid + 1) * B, g] += rdk
        dvc_s[:(cid + 1) * B, g] += rdv
        dos2[0, rows, h] = x["dos"][0, rows, h]
    gg = {k + ("x" if k != "lse" else "_x"): np.concatenate(v) for k, v in gs.items()}
    rr = {k + ("x" if k != "lse" else "_x"): np.concatenate(v) for k, v in rs.items()}
    rep = check_outputs(gg, rr, w.dtype, where=w.name)
    announce(f"{w.name} clean shard sampled rows: {rep}")
    _, g_dkc, g_dvc = csbp.clean_share_backward(x["qs"], x["kc"], x["vc"], ids, B, w.share_chunk, o, lse, dos2,
                                                w.scale, bufs)
    torch.cuda.synchronize()
    for name, gt, ref in (("dkc", g_dkc, dkc_s), ("dvc", g_dvc, dvc_s)):
        a = to_f64(gt[0])
        seen = np.any(ref != 0, axis=-1)
        assert not np.any(a[~seen]), f"{name}: non-zero gradient on unseen keys"
        e = rel_fro(a, ref)
        announce(f"{w.name} clean shard dO-masked {name} rel {e:.3e}")
        assert e <= TOL_REL, (name, e)
