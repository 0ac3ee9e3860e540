"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
hand-written mask fixtures, closed forms, library routines (torch SDPA and its
autograd, scipy logsumexp), finite differences, and the exactness identities of
block parallelism (BP) and chunked-prefix merging that the paper proves
(review Strengths, Prop. 1 / App. A)."""
import itertools
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import bdlm_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _inputs(rng, bsz, L, hq, hkv, d, q_std=1.0):
    qc, qx = _rand(rng, bsz, L, hq, d) * q_std, _rand(rng, bsz, L, hq, d) * q_std
    kc, kx = _rand(rng, bsz, L, hkv, d) * q_std, _rand(rng, bsz, L, hkv, d) * q_std
    vc, vx = _rand(rng, bsz, L, hkv, d), _rand(rng, bsz, L, hkv, d)
    doc, dox = _rand(rng, bsz, L, hq, d), _rand(rng, bsz, L, hq, d)
    return dict(qc=qc, kc=kc, vc=vc, qx=qx, kx=kx, vx=vx, doc=doc, dox=dox)


def _load_mask(name):
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, name)) if ln.strip() and not ln.startswith("#")]
    return np.array([[int(x) for x in r] for r in rows], dtype=bool)


# ------------------------------------------------------------------------ the mask
@pytest.mark.parametrize("name,L,B", [("mask_L4_B2.txt", 4, 2), ("mask_L6_B2.txt", 6, 2)])
def test_mask_matches_hand_written_fixture(name, L, B):
    np.testing.assert_array_equal(O.bdlm_mask(L, B), _load_mask(name))


@pytest.mark.parametrize("L,B", [(8, 1), (8, 2), (8, 8), (48, 16), (64, 16), (30, 5)])
def test_visible_pair_count_closed_form(L, B):
    m = O.bdlm_mask(L, B)
    assert m.sum() == L * (L + B)
    # every query block of either stream sees (b+1)B keys
    per_row = m.sum(axis=1)
    blk = (np.arange(2 * L) % L) // B
    np.testing.assert_array_equal(per_row, (blk + 1) * B)
    # clean rows never see corrupted keys
    assert not m[:L, L:].any()


def test_mask_rows_subset():
    L, B = 24, 4
    rows = np.array([0, 5, 23, 24, 30, 47])
    np.testing.assert_array_equal(O.bdlm_mask_rows(L, B, rows), O.bdlm_mask(L, B)[rows])


# ----------------------------------------------------- library special cases (SDPA)
def _sdpa(q, k, v, mask, scale):
    """torch SDPA in fp64 on the CPU; q [Tq, d], k/v [Tk, d], boolean mask."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64)[None, None] for x in (q, k, v))
    m = torch.tensor(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                            scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("L,B,hq,hkv,d", [(16, 4, 2, 1, 8), (24, 8, 4, 2, 16), (12, 3, 3, 3, 5)])
def test_forward_equals_sdpa_with_explicit_mask(L, B, hq, hkv, d):
    rng = np.random.default_rng(11)
    x = _inputs(rng, 2, L, hq, hkv, d)
    scale = 0.37
    r = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], None, None, B, scale)
    mask = O.bdlm_mask(L, B)
    for b in range(2):
        for h in range(hq):
            g = h * hkv // hq      # contiguous groups, written independently of the oracle
            q = np.concatenate([x["qc"][b, :, h], x["qx"][b, :, h]])
            k = np.concatenate([x["kc"][b, :, g], x["kx"][b, :, g]])
            v = np.concatenate([x["vc"][b, :, g], x["vx"][b, :, g]])
            ref = _sdpa(q, k, v, mask, scale)
            np.testing.assert_allclose(np.concatenate([r["oc"][b, :, h], r["ox"][b, :, h]]), ref,
                                       rtol=0, atol=1e-13)
            # LSE against scipy's logsumexp of the visible scores
            s = scale * q @ k.T
            lse_ref = np.array([logsumexp(s[i][mask[i]]) for i in range(2 * L)])
            np.testing.assert_allclose(np.concatenate([r["lse_c"][b, h], r["lse_x"][b, h]]),
                                       lse_ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("L,B,hq,hkv,d", [(16, 4, 4, 2, 8), (20, 5, 2, 2, 6)])
def test_backward_equals_sdpa_autograd(L, B, hq, hkv, d):
    rng = np.random.default_rng(12)
    x = _inputs(rng, 1, L, hq, hkv, d)
    scale = 0.5
    r = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], x["doc"], x["dox"],
                       B, scale)
    q = torch.tensor(np.concatenate([x["qc"], x["qx"]], 1)[0].transpose(1, 0, 2), requires_grad=True)
    k = torch.tensor(np.concatenate([x["kc"], x["kx"]], 1)[0].transpose(1, 0, 2), requires_grad=True)
    v = torch.tensor(np.concatenate([x["vc"], x["vx"]], 1)[0].transpose(1, 0, 2), requires_grad=True)
    do = torch.tensor(np.concatenate([x["doc"], x["dox"]], 1)[0].transpose(1, 0, 2))
    rep = hq // hkv
    ke = k.repeat_interleave(rep, dim=0)
    ve = v.repeat_interleave(rep, dim=0)
    m = torch.tensor(O.bdlm_mask(L, B))
    o = torch.nn.functional.scaled_dot_product_attention(q[None], ke[None], ve[None],
                                                         attn_mask=m, scale=scale)[0]
    (o * do).sum().backward()
    dq = q.grad.numpy().transpose(1, 0, 2)
    dk = k.grad.numpy().transpose(1, 0, 2)
    dv = v.grad.numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(np.concatenate([r["dqc"][0], r["dqx"][0]]), dq, atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.concatenate([r["dkc"][0], r["dkx"][0]]), dk, atol=1e-12, rtol=0)
    np.testing.assert_allclose(np.concatenate([r["dvc"][0], r["dvx"][0]]), dv, atol=1e-12, rtol=0)


def test_block_equals_L_is_bidirectional_attention():
    """B = L: clean queries see every clean key, corrupted queries every
    corrupted key and no clean key -- two plain bidirectional attentions."""
    rng = np.random.default_rng(13)
    L, hq, hkv, d = 12, 2, 1, 8
    x = _inputs(rng, 1, L, hq, hkv, d)
    r = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], None, None, L, 0.3)
    full = np.ones((L, L), dtype=bool)
    for h in range(hq):
        np.testing.assert_allclose(r["oc"][0, :, h], _sdpa(x["qc"][0, :, h], x["kc"][0, :, 0],
                                                           x["vc"][0, :, 0], full, 0.3), atol=1e-13)
        np.testing.assert_allclose(r["ox"][0, :, h], _sdpa(x["qx"][0, :, h], x["kx"][0, :, 0],
                                                           x["vx"][0, :, 0], full, 0.3), atol=1e-13)


def test_block_one_clean_stream_is_causal_attention():
    rng = np.random.default_rng(14)
    L, hq, hkv, d = 10, 1, 1, 4
    x = _inputs(rng, 1, L, hq, hkv, d)
    r = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], None, None, 1, 0.7)
    qt, kt, vt = (torch.tensor(x[n][0, :, 0])[None, None] for n in ("qc", "kc", "vc"))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=0.7)
    np.testing.assert_allclose(r["oc"][0, :, 0], ref[0, 0].numpy(), atol=1e-13)


# ----------------------------------------------------------------- closed forms
def test_zero_query_closed_form():
    """Q = 0 makes P uniform on the visible set: LSE = log((b+1)B) for both
    streams of block b, O = mean of the visible V rows (prefix sums)."""
    rng = np.random.default_rng(15)
    L, B, hq, hkv, d = 24, 4, 2, 1, 6
    x = _inputs(rng, 1, L, hq, hkv, d)
    z = np.zeros_like(x["qc"])
    r = O.bdlm_fwd_bwd(z, x["kc"], x["vc"], z, x["kx"], x["vx"], None, None, B, 1.0)
    blk = np.arange(L) // B
    np.testing.assert_allclose(r["lse_c"][0, 0], np.log((blk + 1) * B), atol=1e-14)
    np.testing.assert_allclose(r["lse_x"][0, 1], np.log((blk + 1) * B), atol=1e-14)
    vc, vx = x["vc"][0, :, 0], x["vx"][0, :, 0]
    csum = np.cumsum(vc, axis=0)
    for t in range(L):
        b = t // B
        clean_mean = csum[(b + 1) * B - 1] / ((b + 1) * B)
        np.testing.assert_allclose(r["oc"][0, t, 0], clean_mean, atol=1e-13)
        prefix = csum[b * B - 1] if b else np.zeros(d)
        own = vx[b * B:(b + 1) * B].sum(axis=0)
        np.testing.assert_allclose(r["ox"][0, t, 1], (prefix + own) / ((b + 1) * B), atol=1e-13)


def test_gradient_invariants_and_constant_v():
    rng = np.random.default_rng(16)
    L, B, hq, hkv, d = 16, 4, 4, 2, 5
    x = _inputs(rng, 2, L, hq, hkv, d)
    r = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], x["doc"], x["dox"], B, 0.4)
    rep = hq // hkv
    for b in range(2):
        for g in range(hkv):
            dv_sum = r["dvc"][b, :, g].sum(0) + r["dvx"][b, :, g].sum(0)
            do_sum = sum(x["doc"][b, :, h].sum(0) + x["dox"][b, :, h].sum(0)
                         for h in range(g * rep, (g + 1) * rep))
            np.testing.assert_allclose(dv_sum, do_sum, atol=1e-12)
            dk_sum = r["dkc"][b, :, g].sum(0) + r["dkx"][b, :, g].sum(0)
            np.testing.assert_allclose(dk_sum, 0.0, atol=1e-12)
    cv = np.full_like(x["vc"], 2.5)
    r2 = O.bdlm_fwd_bwd(x["qc"], x["kc"], cv, x["qx"], x["kx"], cv, None, None, B, 0.4)
    np.testing.assert_allclose(r2["oc"], 2.5, atol=1e-13)
    np.testing.assert_allclose(r2["ox"], 2.5, atol=1e-13)


# ------------------------------------------------------------ finite differences
def test_backward_matches_central_finite_differences():
    """Analytic dQ/dK/dV of l = <dO, O> against central differences (h = 1e-6)
    on every input element of a tiny GQA problem."""
    rng = np.random.default_rng(17)
    L, B, hq, hkv, d = 8, 2, 2, 1, 4
    x = _inputs(rng, 1, L, hq, hkv, d)
    scale = 0.45
    r = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], x["doc"], x["dox"], B, scale)
    names = ["qc", "kc", "vc", "qx", "kx", "vx"]

    def loss(xs):
        oc, ox, _, _ = O.bdlm_fwd(xs["qc"], xs["kc"], xs["vc"], xs["qx"], xs["kx"], xs["vx"], B, scale)
        return (oc * x["doc"]).sum() + (ox * x["dox"]).sum()

    h = 1e-6
    for name in names:
        grad = np.zeros_like(x[name])
        for idx in itertools.product(*[range(s) for s in x[name].shape]):
            xp = {k: v.copy() for k, v in x.items()}
            xm = {k: v.copy() for k, v in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            grad[idx] = (loss(xp) - loss(xm)) / (2 * h)
        an = r["d" + name]
        err = np.abs(grad - an).max() / max(np.abs(an).max(), 1e-30)
        assert err < 1e-7, (name, err)


# ------------------------------------------------------------- exactness identities
@pytest.mark.parametrize("L,B,hq,hkv,d", [(16, 4, 4, 2, 8), (24, 8, 2, 2, 4), (18, 3, 3, 1, 5)])
def test_bp_exactness_full_equals_per_block(L, B, hq, hkv, d):
    """The full 2L masked computation equals the block-separated computation
    (clean dK/dV summed over the clean stream and every later block)."""
    rng = np.random.default_rng(18)
    x = _inputs(rng, 2, L, hq, hkv, d)
    a = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], x["doc"], x["dox"], B, 0.3)
    b = O.bdlm_fwd_bwd_per_block(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"],
                                 x["doc"], x["dox"], B, 0.3)
    for k in ("oc", "ox", "lse_c", "lse_x", "dqc", "dqx", "dkc", "dkx", "dvc", "dvx"):
        np.testing.assert_allclose(a[k], b[k], atol=1e-13, rtol=0, err_msg=k)


def _share_case(seed, L=64, B=8, nlocal=3, hq=2, hkv=1, d=4):
    rng = np.random.default_rng(seed)
    ids = np.sort(rng.choice(L // B, size=nlocal, replace=False))
    T = nlocal * B
    kc, vc = _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    qx, kx, vx = _rand(rng, 1, T, hq, d), _rand(rng, 1, T, hkv, d), _rand(rng, 1, T, hkv, d)
    dox = _rand(rng, 1, T, hq, d)
    return ids, kc, vc, qx, kx, vx, dox


@pytest.mark.parametrize("chunk", [8, 16, 24, 64])
def test_chunked_prefix_merge_equals_single_pass(chunk):
    """Partials over clean chunks (some empty for early blocks) plus the
    own-block partial, merged by logsumexp, equal one pass over all keys, and
    equal the full 2L computation restricted to those corrupted blocks."""
    L, B = 64, 8
    ids, kc, vc, qx, kx, vx, dox = _share_case(19 + chunk, L=L, B=B)
    scale = 0.6
    parts = [O.share_fwd(qx, kx, vx, kc, vc, ids, B, j, min(j + chunk, L), 0, scale)
             for j in range(0, L, chunk)]
    parts.append(O.share_fwd(qx, kx, vx, kc, vc, ids, B, 0, 0, 1, scale))
    o_m, lse_m = O.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    o_1, lse_1 = O.share_fwd(qx, kx, vx, kc, vc, ids, B, 0, L, 1, scale)
    np.testing.assert_allclose(o_m, o_1, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse_m, lse_1, atol=1e-13, rtol=0)
    # the same blocks inside a full length-2L problem
    rng = np.random.default_rng(5)
    hq, hkv, d = qx.shape[2], kc.shape[2], qx.shape[3]
    qc_f = _rand(rng, 1, L, hq, d)
    qx_f, kx_f, vx_f = _rand(rng, 1, L, hq, d), _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    for i, bid in enumerate(ids):
        qx_f[0, bid * B:(bid + 1) * B] = qx[0, i * B:(i + 1) * B]
        kx_f[0, bid * B:(bid + 1) * B] = kx[0, i * B:(i + 1) * B]
        vx_f[0, bid * B:(bid + 1) * B] = vx[0, i * B:(i + 1) * B]
    full = O.bdlm_fwd_bwd(qc_f, kc, vc, qx_f, kx_f, vx_f, None, None, B, scale)
    for i, bid in enumerate(ids):
        np.testing.assert_allclose(o_m[0, i * B:(i + 1) * B], full["ox"][0, bid * B:(bid + 1) * B],
                                   atol=1e-14)
        np.testing.assert_allclose(lse_m[0, :, i * B:(i + 1) * B],
                                   full["lse_x"][0, :, bid * B:(bid + 1) * B], atol=1e-13)


@pytest.mark.parametrize("chunk", [16, 24])
def test_chunked_backward_sums_to_per_block_backward(chunk):
    """Per-chunk backward with the final LSE/O: dQ contributions add up to the
    one-pass dQ; window dK/dV tile the clean dK/dV; own-block dK/dV match."""
    L, B = 64, 8
    ids, kc, vc, qx, kx, vx, dox = _share_case(40 + chunk, L=L, B=B)
    scale = 0.6
    o_f, lse_f = O.share_fwd(qx, kx, vx, kc, vc, ids, B, 0, L, 1, scale)
    one = O.share_bwd(qx, kx, vx, kc, vc, ids, B, 0, L, 1, o_f, lse_f, dox, scale)
    dq = np.zeros_like(qx)
    dkc = np.zeros_like(kc)
    dvc = np.zeros_like(vc)
    for j in range(0, L, chunk):
        e = min(j + chunk, L)
        r = O.share_bwd(qx, kx, vx, kc, vc, ids, B, j, e, 0, o_f, lse_f, dox, scale)
        dq += r[0]
        dkc[:, j:e] = r[1]
        dvc[:, j:e] = r[2]
        assert not r[3].any() and not r[4].any()
    own = O.share_bwd(qx, kx, vx, kc, vc, ids, B, 0, 0, 1, o_f, lse_f, dox, scale)
    dq += own[0]
    np.testing.assert_allclose(dq, one[0], atol=1e-13)
    np.testing.assert_allclose(dkc, one[1], atol=1e-13)
    np.testing.assert_allclose(dvc, one[2], atol=1e-13)
    np.testing.assert_allclose(own[3], one[3], atol=1e-13)
    np.testing.assert_allclose(own[4], one[4], atol=1e-13)
    # and the one-pass share backward equals plain attention backward per block
    hq, hkv = qx.shape[2], kc.shape[2]
    for i, bid in enumerate(ids):
        r = slice(i * B, (i + 1) * B)
        for h in range(hq):
            g = h * hkv // hq
            keys = np.concatenate([kc[0, :bid * B, g], kx[0, r, g]])
            vals = np.concatenate([vc[0, :bid * B, g], vx[0, r, g]])
            qt = torch.tensor(qx[0, r, h], requires_grad=True)
            kt = torch.tensor(keys, requires_grad=True)
            vt = torch.tensor(vals, requires_grad=True)
            o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                                 scale=scale)[0]
            (o * torch.tensor(dox[0, r, h])).sum().backward()
            np.testing.assert_allclose(one[0][0, r, h], qt.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("chunk", [8, 24, 64])
def test_clean_query_share_equals_full_clean_stream(chunk):
    """The rank's clean query blocks, streamed over clean chunks and merged,
    give the full 2L computation's clean-stream rows (forward), and the summed
    chunk backwards give its dQ rows and its clean dK/dV when only those rows
    carry an upstream gradient."""
    L, B, hq, hkv, d = 64, 8, 2, 1, 4
    rng = np.random.default_rng(70 + chunk)
    ids = np.sort(rng.choice(L // B, size=3, replace=False))
    T = len(ids) * B
    kc, vc = _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    qc_f = _rand(rng, 1, L, hq, d)
    qx_f, kx_f, vx_f = _rand(rng, 1, L, hq, d), _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    qs = np.concatenate([qc_f[:, b * B:(b + 1) * B] for b in ids], axis=1)
    dos = _rand(rng, 1, T, hq, d)
    scale = 0.6
    wins = [(j, min(j + chunk, L)) for j in range(0, L, chunk)]
    parts = [O.share_fwd(qs, None, None, kc, vc, ids, B, j, e, 0, scale, clean_queries=True) for j, e in wins]
    o_m, lse_m = O.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    doc_f = np.zeros_like(qc_f)
    for i, b in enumerate(ids):
        doc_f[0, b * B:(b + 1) * B] = dos[0, i * B:(i + 1) * B]
    full = O.bdlm_fwd_bwd(qc_f, kc, vc, qx_f, kx_f, vx_f, doc_f, np.zeros_like(qx_f), B, scale)
    for i, b in enumerate(ids):
        np.testing.assert_allclose(o_m[0, i * B:(i + 1) * B], full["oc"][0, b * B:(b + 1) * B], atol=1e-14)
        np.testing.assert_allclose(lse_m[0, :, i * B:(i + 1) * B], full["lse_c"][0, :, b * B:(b + 1) * B],
                                   atol=1e-13)
    dq = np.zeros_like(qs)
    dkc = np.zeros_like(kc)
    dvc = np.zeros_like(vc)
    for j, e in wins:
        r = O.share_bwd(qs, None, None, kc, vc, ids, B, j, e, 0, o_m, lse_m, dos, scale, clean_queries=True)
        dq += r[0]
        dkc[:, j:e] = r[1]
        dvc[:, j:e] = r[2]
        assert not r[3].any() and not r[4].any()
    for i, b in enumerate(ids):
        np.testing.assert_allclose(dq[0, i * B:(i + 1) * B], full["dqc"][0, b * B:(b + 1) * B], atol=1e-13)
    np.testing.assert_allclose(dkc, full["dkc"], atol=1e-13)
    np.testing.assert_allclose(dvc, full["dvc"], atol=1e-13)
    assert not full["dkx"].any() and not full["dvx"].any()


def test_clean_query_share_block_is_attention_over_its_inclusive_prefix():
    """Each clean query block of a one-pass clean-query share is plain attention
    (torch SDPA in fp64) over the clean keys of its own and earlier blocks."""
    L, B, hq, hkv, d = 48, 8, 2, 1, 4
    rng = np.random.default_rng(77)
    ids = np.array([0, 2, 5])
    kc, vc = _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    qs = _rand(rng, 1, len(ids) * B, hq, d)
    o, lse = O.share_fwd(qs, None, None, kc, vc, ids, B, 0, L, 0, 0.7, clean_queries=True)
    for i, b in enumerate(ids):
        r = slice(i * B, (i + 1) * B)
        for h in range(hq):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.tensor(qs[0, r, h])[None], torch.tensor(kc[0, :(b + 1) * B, 0])[None],
                torch.tensor(vc[0, :(b + 1) * B, 0])[None], scale=0.7)[0]
            np.testing.assert_allclose(o[0, r, h], ref.numpy(), atol=1e-14)


def test_merge_edge_cases():
    rng = np.random.default_rng(20)
    o1, o2 = _rand(rng, 1, 3, 2, 4), _rand(rng, 1, 3, 2, 4)
    l1 = _rand(rng, 1, 2, 3)
    ninf = np.full((1, 2, 3), -np.inf)
    # a single part is returned unchanged
    o, l = O.merge_partials([o1], [l1])
    np.testing.assert_allclose(o, o1)
    np.testing.assert_allclose(l, l1)
    # an empty partial has weight 0
    o, l = O.merge_partials([o1, np.zeros_like(o2)], [l1, ninf])
    np.testing.assert_allclose(o, o1)
    np.testing.assert_allclose(l, l1)
    # all-empty rows stay (0, -inf)
    o, l = O.merge_partials([np.zeros_like(o1), np.zeros_like(o2)], [ninf, ninf])
    assert (o == 0).all() and np.isneginf(l).all()
    # two equal LSEs: plain average, LSE + log 2
    o, l = O.merge_partials([o1, o2], [l1, l1])
    np.testing.assert_allclose(o, 0.5 * (o1 + o2), atol=1e-15)
    np.testing.assert_allclose(l, l1 + np.log(2.0), atol=1e-15)


def test_share_empty_window_rows_are_empty_partials():
    L, B = 64, 8
    ids, kc, vc, qx, kx, vx, dox = _share_case(21, L=L, B=B)
    # a window above every block's prefix: no visible key anywhere
    lo = int(ids.max()) * B
    o, lse = O.share_fwd(qx, kx, vx, kc, vc, ids, B, lo, L, 0, 0.5)
    assert (o == 0).all() and np.isneginf(lse).all()


# -------------------------------------------------------------- sampled oracle
def test_sampled_units_equal_full_computation():
    rng = np.random.default_rng(22)
    L, B, hq, hkv, d = 32, 8, 4, 2, 4
    x = _inputs(rng, 2, L, hq, hkv, d)
    full = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], x["doc"], x["dox"], B, 0.5)
    units = np.array([(0, 0, 0, 1), (1, 1, 3, 2), (0, 1, 0, 0), (1, 0, 3, 3), (0, 1, 2, 1)])
    res, dk_s, dv_s = O.sampled_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"],
                                        x["doc"], x["dox"], B, 0.5, units)
    for r in res:
        b, st, blk, h = r["unit"]
        t = slice(blk * B, (blk + 1) * B)
        s = "c" if st == 0 else "x"
        np.testing.assert_allclose(r["o"], full["o" + s][b, t, h], atol=1e-14)
        np.testing.assert_allclose(r["lse"], full["lse_" + s][b, h, t], atol=1e-14)
        np.testing.assert_allclose(r["dq"], full["dq" + s][b, t, h], atol=1e-13)
    # dK/dV of the sampled rows == full backward with dO zeroed elsewhere
    doc, dox = np.zeros_like(x["doc"]), np.zeros_like(x["dox"])
    for b, st, blk, h in units:
        t = slice(blk * B, (blk + 1) * B)
        (doc if st == 0 else dox)[b, t, h] = (x["doc"] if st == 0 else x["dox"])[b, t, h]
    m = O.bdlm_fwd_bwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], doc, dox, B, 0.5)
    np.testing.assert_allclose(dk_s, np.concatenate([m["dkc"], m["dkx"]], 1), atol=1e-13)
    np.testing.assert_allclose(dv_s, np.concatenate([m["dvc"], m["dvx"]], 1), atol=1e-13)


@pytest.mark.parametrize("chunk", [16, 64])
def test_share_backward_own_block_equals_full_problem(chunk):
    """The share-mode backward's own-block dK/dV (and its clean windows) equal
    the full length-2L backward's dK/dV when the local corrupted blocks are
    scattered into a full problem whose dO is zero everywhere else: only those
    rows then carry a gradient, so the full dK/dV are exactly their
    contributions (BP exactness, review Strengths, Prop. 1 / App. A).  The
    per-block dK/dV are also checked against torch SDPA autograd over each
    block's keys [clean prefix ; own block], summed over the GQA group."""
    L, B, hq, hkv, d = 64, 8, 4, 2, 4
    rng = np.random.default_rng(90 + chunk)
    ids = np.sort(rng.choice(L // B, size=3, replace=False))
    T = len(ids) * B
    kc, vc = _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    qx, kx, vx = _rand(rng, 1, T, hq, d), _rand(rng, 1, T, hkv, d), _rand(rng, 1, T, hkv, d)
    dox = _rand(rng, 1, T, hq, d)
    scale = 0.55
    o_f, lse_f = O.share_fwd(qx, kx, vx, kc, vc, ids, B, 0, L, 1, scale)
    own = O.share_bwd(qx, kx, vx, kc, vc, ids, B, 0, 0, 1, o_f, lse_f, dox, scale)
    dkc = np.zeros_like(kc)
    dvc = np.zeros_like(vc)
    for j in range(0, L, chunk):
        e = min(j + chunk, L)
        r = O.share_bwd(qx, kx, vx, kc, vc, ids, B, j, e, 0, o_f, lse_f, dox, scale)
        dkc[:, j:e] = r[1]
        dvc[:, j:e] = r[2]
    # scatter into a full problem with dO zero outside the local corrupted blocks
    qc_f = _rand(rng, 1, L, hq, d)
    qx_f, kx_f, vx_f = _rand(rng, 1, L, hq, d), _rand(rng, 1, L, hkv, d), _rand(rng, 1, L, hkv, d)
    dox_f = np.zeros((1, L, hq, d))
    for i, bid in enumerate(ids):
        src, dst = slice(i * B, (i + 1) * B), slice(bid * B, (bid + 1) * B)
        qx_f[0, dst], kx_f[0, dst], vx_f[0, dst] = qx[0, src], kx[0, src], vx[0, src]
        dox_f[0, dst] = dox[0, src]
    full = O.bdlm_fwd_bwd(qc_f, kc, vc, qx_f, kx_f, vx_f, np.zeros_like(qc_f), dox_f, B, scale)
    for i, bid in enumerate(ids):
        src, dst = slice(i * B, (i + 1) * B), slice(bid * B, (bid + 1) * B)
        np.testing.assert_allclose(own[3][0, src], full["dkx"][0, dst], atol=1e-13, err_msg="dkx")
        np.testing.assert_allclose(own[4][0, src], full["dvx"][0, dst], atol=1e-13, err_msg="dvx")
    np.testing.assert_allclose(dkc, full["dkc"], atol=1e-13, err_msg="dkc")
    np.testing.assert_allclose(dvc, full["dvc"], atol=1e-13, err_msg="dvc")
    # SDPA autograd per (block, head): dK/dV over [clean prefix ; own block]
    rep = hq // hkv
    for i, bid in enumerate(ids):
        r = slice(i * B, (i + 1) * B)
        for g in range(hkv):
            kt = torch.tensor(np.concatenate([kc[0, :bid * B, g], kx[0, r, g]]), requires_grad=True)
            vt = torch.tensor(np.concatenate([vc[0, :bid * B, g], vx[0, r, g]]), requires_grad=True)
            for h in range(g * rep, (g + 1) * rep):
                o = torch.nn.functional.scaled_dot_product_attention(
                    torch.tensor(qx[0, r, h])[None], kt[None], vt[None], scale=scale)[0]
                (o * torch.tensor(dox[0, r, h])).sum().backward()
            np.testing.assert_allclose(own[3][0, r, g], kt.grad.numpy()[bid * B:], atol=1e-12)
            np.testing.assert_allclose(own[4][0, r, g], vt.grad.numpy()[bid * B:], atol=1e-12)
