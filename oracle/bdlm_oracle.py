"""fp64 CPU oracle for BDLM masked attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never imports it, links it or calls it, and it
shares no code with the GPU library (no kernels, helpers, tables or constants).

What it follows
---------------
"Block Parallelism For Efficient Distributed Long-Context Diffusion Language
Model Training" (arXiv 2609.19242), as described by its abstract (arXiv and
NeurIPS 2026 pages) and by the evolve.pub review (Summary, Key claims,
Strengths: "Exactness is proven", FAQ "What is CSBP?"):

* A block diffusion LM keeps autoregressive dependencies across blocks and
  denoises the tokens of one block in parallel (abstract).  Training attends
  over the concatenated clean-plus-corrupted sequence [x0 ; xt] of length 2L
  (abstract; review Strengths, Prop. 1 / App. A, "reference length-2L
  computation").
* Clean K/V is shared by all later blocks while each corrupted block's K/V is
  private to that block (abstract; FAQ on CSBP).
* The objective separates over target blocks, so a whole corrupted block can
  be computed on one rank against the clean prefix (BP), and the clean
  sequence can be sharded (CSBP) with results that equal the length-2L
  computation up to floating-point reduction order (review Key claims,
  Strengths; FAQ "Does CSBP change training results").

Readings where the pages are silent (the pages print no equation):
  R1 mask: token t of [x0 ; xt] has stream C if t < L else X and block
     (t mod L) div B.  A clean query in block b sees clean keys of blocks
     <= b; a corrupted query in block b sees clean keys of blocks < b and the
     corrupted keys of its own block b; clean queries never see corrupted keys.
  R2 scores S = scale * <q, k>, natural-log LSE, softmax over visible keys only.
  R3 GQA: q-head h reads kv-head h div (Hq / Hkv).
  R4 a row with no visible key (only possible for a partial over a key chunk)
     has O = 0 and LSE = -inf; merging gives such a partial weight 0.
  R5 the backward of a key chunk uses the final (merged) LSE and
     D = rowsum(dO * O_final) -- the stored-LSE recompute.
Everything is fp64; inputs are the exact values the GPU receives.
"""
import numpy as np

__all__ = [
    "token_stream_block", "bdlm_mask", "bdlm_mask_rows", "attention_fwd", "attention_bwd",
    "bdlm_fwd", "bdlm_fwd_bwd", "bdlm_fwd_bwd_per_block", "merge_partials",
    "share_keys", "share_fwd", "share_bwd", "unit_rows_fwd_bwd", "sampled_fwd_bwd",
    "kv_head_of",
]


# --------------------------------------------------------------------------- mask
def token_stream_block(L, B):
    """Stream (0 = clean x0, 1 = corrupted xt) and block index of each of the 2L
    tokens of [x0 ; xt] (reading R1)."""
    t = np.arange(2 * L)
    stream = (t >= L).astype(np.int64)
    block = (t % L) // B
    return stream, block


def _visible(q_stream, q_block, k_stream, k_block):
    """Element-wise visibility rule R1 (broadcasting arrays)."""
    clean_clean = (q_stream == 0) & (k_stream == 0) & (k_block <= q_block)
    noisy_clean = (q_stream == 1) & (k_stream == 0) & (k_block < q_block)
    noisy_noisy = (q_stream == 1) & (k_stream == 1) & (k_block == q_block)
    return clean_clean | noisy_clean | noisy_noisy


def bdlm_mask(L, B):
    """Explicit 2L x 2L boolean mask of the BDLM attention (True = visible)."""
    if L % B:
        raise ValueError("L must be a multiple of B")
    s, b = token_stream_block(L, B)
    return _visible(s[:, None], b[:, None], s[None, :], b[None, :])


def bdlm_mask_rows(L, B, rows):
    """Rows `rows` (indices into the 2L sequence) of the explicit mask."""
    s, b = token_stream_block(L, B)
    rows = np.asarray(rows)
    return _visible(s[rows][:, None], b[rows][:, None], s[None, :], b[None, :])


def kv_head_of(h, hq, hkv):
    """Reading R3: contiguous query-head groups share one kv head."""
    return h // (hq // hkv)


# ---------------------------------------------------------------- plain attention
def attention_fwd(q, k, v, mask, scale):
    """Naive masked softmax attention for one head.

    q [Tq, d], k/v [Tk, d], mask [Tq, Tk] bool.  Returns O [Tq, d], natural-log
    LSE [Tq] and the probabilities P [Tq, Tk].  Rows with no visible key give
    O = 0, LSE = -inf, P = 0 (reading R4)."""
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    has = np.isfinite(m)
    m_ref = np.where(has, m, 0.0)
    e = np.exp(s - m_ref[:, None])          # masked entries -> exp(-inf) = 0
    l = e.sum(axis=1)
    l_safe = np.where(has, l, 1.0)
    p = e / l_safe[:, None]
    lse = np.where(has, m_ref + np.log(l_safe), -np.inf)
    o = p @ v
    return o, lse, p


def attention_bwd(q, k, v, p, o, do, scale, delta=None):
    """Analytic backward of attention_fwd for one head given its P.

    D = rowsum(dO * O); dP = dO V^T; dS = P (dP - D); dQ = scale dS K;
    dK = scale dS^T Q; dV = P^T dO.  `delta` overrides D (reading R5)."""
    d_row = (do * o).sum(axis=1) if delta is None else delta
    dp = do @ v.T
    ds = p * (dp - d_row[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return dq, dk, dv


# ------------------------------------------------------------- full length-2L form
def _cat(a, b):
    return np.concatenate([a, b], axis=1)


def bdlm_fwd(qc, kc, vc, qx, kx, vx, block, scale):
    """Forward of the reference length-2L computation with the explicit mask.

    Inputs [batch, L, H, d] (H = Hq for Q, Hkv for K/V).  Returns
    (oc, ox, lse_c, lse_x) with O [batch, L, Hq, d] and LSE [batch, Hq, L]."""
    r = bdlm_fwd_bwd(qc, kc, vc, qx, kx, vx, None, None, block, scale)
    return r["oc"], r["ox"], r["lse_c"], r["lse_x"]


def bdlm_fwd_bwd(qc, kc, vc, qx, kx, vx, doc, dox, block, scale):
    """Forward (and backward when doc/dox are given) over [x0 ; xt] with the
    explicit 2L x 2L mask, one (batch, q-head) at a time.  dK/dV of a kv head
    sum the contributions of every q head that reads it."""
    bsz, L, hq, d = qc.shape
    hkv = kc.shape[2]
    mask = bdlm_mask(L, block)
    q = _cat(qc, qx).astype(np.float64)
    k = _cat(kc, kx).astype(np.float64)
    v = _cat(vc, vx).astype(np.float64)
    want_bwd = doc is not None
    if want_bwd:
        do = _cat(doc, dox).astype(np.float64)
    o = np.zeros((bsz, 2 * L, hq, d))
    lse = np.zeros((bsz, hq, 2 * L))
    dq = np.zeros_like(o)
    dk = np.zeros((bsz, 2 * L, hkv, d))
    dv = np.zeros_like(dk)
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            oh, lh, ph = attention_fwd(q[b, :, h], k[b, :, g], v[b, :, g], mask, scale)
            o[b, :, h] = oh
            lse[b, h] = lh
            if want_bwd:
                dqh, dkh, dvh = attention_bwd(q[b, :, h], k[b, :, g], v[b, :, g], ph, oh,
                                              do[b, :, h], scale)
                dq[b, :, h] = dqh
                dk[b, :, g] += dkh
                dv[b, :, g] += dvh
            del ph
    out = {"oc": o[:, :L], "ox": o[:, L:], "lse_c": lse[:, :, :L], "lse_x": lse[:, :, L:]}
    if want_bwd:
        out.update(dqc=dq[:, :L], dqx=dq[:, L:], dkc=dk[:, :L], dkx=dk[:, L:],
                   dvc=dv[:, :L], dvx=dv[:, L:])
    return out


# ------------------------------------------------------ per-block (BP) separated form
def bdlm_fwd_bwd_per_block(qc, kc, vc, qx, kx, vx, doc, dox, block, scale):
    """The block-separated form that BP computes (review Strengths, Prop. 1):

    * the clean stream is block-causal attention over x0 alone;
    * corrupted block b is *unmasked* attention of its queries over the clean
      prefix K_C[0 : bB] followed by its own corrupted K/V;
    * clean dK/dV collect the clean stream's contribution plus that of every
      later corrupted block; a corrupted block's dK/dV stay with the block.
    Written without the 2L x 2L mask, so equality with bdlm_fwd_bwd is the
    BP-exactness identity."""
    bsz, L, hq, d = qc.shape
    hkv = kc.shape[2]
    n = L // block
    blk = np.arange(L) // block
    causal = blk[None, :] <= blk[:, None]
    out = {k_: np.zeros((bsz, L, hq, d)) for k_ in ("oc", "ox", "dqc", "dqx")}
    out["lse_c"] = np.zeros((bsz, hq, L))
    out["lse_x"] = np.zeros((bsz, hq, L))
    for k_ in ("dkc", "dvc", "dkx", "dvx"):
        out[k_] = np.zeros((bsz, L, hkv, d))
    for b in range(bsz):
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            o, lse, p = attention_fwd(qc[b, :, h], kc[b, :, g], vc[b, :, g], causal, scale)
            out["oc"][b, :, h] = o
            out["lse_c"][b, h] = lse
            dq, dk, dv = attention_bwd(qc[b, :, h], kc[b, :, g], vc[b, :, g], p, o,
                                       doc[b, :, h], scale)
            out["dqc"][b, :, h] = dq
            out["dkc"][b, :, g] += dk
            out["dvc"][b, :, g] += dv
            for i in range(n):
                r = slice(i * block, (i + 1) * block)
                keys = np.concatenate([kc[b, : i * block, g], kx[b, r, g]], axis=0)
                vals = np.concatenate([vc[b, : i * block, g], vx[b, r, g]], axis=0)
                full = np.ones((block, keys.shape[0]), dtype=bool)
                o, lse, p = attention_fwd(qx[b, r, h], keys, vals, full, scale)
                out["ox"][b, r, h] = o
                out["lse_x"][b, h, r] = lse
                dq, dk, dv = attention_bwd(qx[b, r, h], keys, vals, p, o, dox[b, r, h], scale)
                out["dqx"][b, r, h] = dq
                out["dkc"][b, : i * block, g] += dk[: i * block]
                out["dvc"][b, : i * block, g] += dv[: i * block]
                out["dkx"][b, r, g] += dk[i * block:]
                out["dvx"][b, r, g] += dv[i * block:]
    return out


# ------------------------------------------------------------ (O, LSE) partial merge
def merge_partials(o_parts, lse_parts):
    """Combine attention partials over disjoint key sets.

    o_parts: list of [..., T, H, d]; lse_parts: list of [..., H, T].
    LSE = log sum_j exp(LSE_j); O = sum_j exp(LSE_j - LSE) O_j.  Partials with
    LSE = -inf weigh 0; a row whose partials are all empty stays (0, -inf)."""
    lse = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])   # [N, ..., H, T]
    m = lse.max(axis=0)
    has = np.isfinite(m)
    m_ref = np.where(has, m, 0.0)
    w = np.exp(lse - m_ref)                                                  # 0 for -inf parts
    tot = w.sum(axis=0)
    lse_out = np.where(has, m_ref + np.log(np.where(has, tot, 1.0)), -np.inf)
    frac = np.where(has, w / np.where(has, tot, 1.0), 0.0)                   # [N, ..., H, T]
    o_out = np.zeros_like(np.asarray(o_parts[0], dtype=np.float64))
    for j, oj in enumerate(o_parts):
        fj = np.swapaxes(frac[j], -1, -2)[..., None]                          # [..., T, H, 1]
        o_out = o_out + fj * np.asarray(oj, dtype=np.float64)
    return o_out, lse_out


# --------------------------------------------------------------- CSBP share partials
def share_keys(block_id, block, local_index, kv_begin, kv_end, own_block, clean_queries=False):
    """Key sets of local block `local_index` (global id `block_id`) in one
    share-mode call: clean tokens [kv_begin, kv_end) cut to the block's clean
    prefix, and its own corrupted rows [local_index*B, (local_index+1)*B) of the
    local arrays when own_block.  The prefix is the mask's: a corrupted block
    sees the clean blocks before it, [0, block_id*B); a clean block (the clean
    stream in context-parallel form, clean_queries) sees the clean blocks up to
    and including itself, [0, (block_id+1)*B), and no corrupted keys."""
    c_lo = max(kv_begin, 0)
    c_hi = min(kv_end, (block_id + (1 if clean_queries else 0)) * block)
    clean = np.arange(c_lo, c_hi) if c_hi > c_lo else np.arange(0)
    own = (np.arange(local_index * block, (local_index + 1) * block) if own_block
           else np.arange(0))
    return clean, own


def share_fwd(qx, kx, vx, kc, vc, block_ids, block, kv_begin, kv_end, own_block, scale,
              clean_queries=False):
    """Partial (O, LSE) of a rank's local blocks over one key chunk.

    qx/kx/vx [batch, nlocal*B, H, d] are the local blocks in id order; kc/vc
    [batch, L, Hkv, d] the clean sequence (kx/vx are unused, may be None, for
    clean query blocks).  Returns O [batch, nlocal*B, Hq, d] and LSE
    [batch, Hq, nlocal*B]; rows without a visible key get (0, -inf)."""
    bsz, T, hq, d = qx.shape
    hkv = kc.shape[2]
    o = np.zeros((bsz, T, hq, d))
    lse = np.full((bsz, hq, T), -np.inf)
    for i, bid in enumerate(block_ids):
        r = slice(i * block, (i + 1) * block)
        ci, xi = share_keys(int(bid), block, i, kv_begin, kv_end, own_block, clean_queries)
        for b in range(bsz):
            for h in range(hq):
                g = kv_head_of(h, hq, hkv)
                keys, vals = kc[b, ci, g], vc[b, ci, g]
                if len(xi):
                    keys = np.concatenate([keys, kx[b, xi, g]], axis=0)
                    vals = np.concatenate([vals, vx[b, xi, g]], axis=0)
                full = np.ones((block, keys.shape[0]), dtype=bool)
                oh, lh, _ = attention_fwd(qx[b, r, h], keys, vals, full, scale)
                o[b, r, h] = oh
                lse[b, h, r] = lh
    return o, lse


def share_bwd(qx, kx, vx, kc, vc, block_ids, block, kv_begin, kv_end, own_block,
              o_final, lse_final, dox, scale, clean_queries=False):
    """Backward of one share-mode key chunk with the final (merged) O and LSE.

    P = exp(S - LSE_final) on the chunk's keys, D = rowsum(dO * O_final)
    (reading R5).  Returns the chunk's dQ contribution [batch, T, Hq, d],
    dK/dV of the clean window [batch, kv_end-kv_begin, Hkv, d] and dK/dV of the
    local corrupted rows [batch, T, Hkv, d] (zero unless own_block)."""
    bsz, T, hq, d = qx.shape
    hkv = kc.shape[2]
    W = max(kv_end - kv_begin, 0)
    dq = np.zeros((bsz, T, hq, d))
    dkc = np.zeros((bsz, W, hkv, d))
    dvc = np.zeros_like(dkc)
    dkx = np.zeros((bsz, T, hkv, d))
    dvx = np.zeros_like(dkx)
    for i, bid in enumerate(block_ids):
        r = slice(i * block, (i + 1) * block)
        ci, xi = share_keys(int(bid), block, i, kv_begin, kv_end, own_block, clean_queries)
        nc = len(ci)
        if nc + len(xi) == 0:
            continue
        for b in range(bsz):
            for h in range(hq):
                g = kv_head_of(h, hq, hkv)
                keys, vals = kc[b, ci, g], vc[b, ci, g]
                if len(xi):
                    keys = np.concatenate([keys, kx[b, xi, g]], axis=0)
                    vals = np.concatenate([vals, vx[b, xi, g]], axis=0)
                s = scale * (qx[b, r, h] @ keys.T)
                p = np.exp(s - lse_final[b, h, r][:, None])
                delta = (dox[b, r, h] * o_final[b, r, h]).sum(axis=1)
                dqh, dkh, dvh = attention_bwd(qx[b, r, h], keys, vals, p, o_final[b, r, h],
                                              dox[b, r, h], scale, delta=delta)
                dq[b, r, h] += dqh
                dkc[b, ci - kv_begin, g] += dkh[:nc]
                dvc[b, ci - kv_begin, g] += dvh[:nc]
                dkx[b, xi, g] += dkh[nc:]
                dvx[b, xi, g] += dvh[nc:]
    return dq, dkc, dvc, dkx, dvx


# ------------------------------------------------------------------ sampled units
def unit_rows_fwd_bwd(q_rows, k_all, v_all, mask_rows, do_rows, scale):
    """O, LSE, dQ and the dK/dV contributions of a set of query rows of one head
    against all 2L keys of its kv head.  Rows are independent in the forward
    and in dQ, so these equal the full computation's values on those rows."""
    o, lse, p = attention_fwd(q_rows, k_all, v_all, mask_rows, scale)
    if do_rows is None:
        return o, lse, None, None, None
    dq, dk, dv = attention_bwd(q_rows, k_all, v_all, p, o, do_rows, scale)
    return o, lse, dq, dk, dv


def sampled_fwd_bwd(qc, kc, vc, qx, kx, vx, doc, dox, block, scale, units, row_offsets=None):
    """Oracle values on sampled units (batch, stream, block, q-head).

    `row_offsets` (optional, offsets inside the block) restricts every unit to
    those rows; rows are independent, so their values are still exact.
    Returns a list of per-unit dicts (o, lse, dq for the unit's rows) and the
    summed dK/dV contributions of all sampled rows, [batch, 2L, Hkv, d] -- what
    a backward whose dO is zero outside the sampled rows produces."""
    bsz, L, hq, d = qc.shape
    hkv = kc.shape[2]
    res = []
    dk_sum = np.zeros((bsz, 2 * L, hkv, d))
    dv_sum = np.zeros_like(dk_sum)
    kv_cache = {}
    for (b, st, blk, h) in np.asarray(units).tolist():
        g = kv_head_of(h, hq, hkv)
        if (b, g) not in kv_cache:
            kv_cache.clear()
            kv_cache[(b, g)] = (np.concatenate([kc[b, :, g], kx[b, :, g]]).astype(np.float64),
                                np.concatenate([vc[b, :, g], vx[b, :, g]]).astype(np.float64))
        k_all, v_all = kv_cache[(b, g)]
        offs = np.arange(block) if row_offsets is None else np.asarray(row_offsets)
        tok = blk * block + offs
        rows = st * L + tok
        q_src = qc if st == 0 else qx
        do_src = doc if st == 0 else dox
        do_rows = None if do_src is None else np.asarray(do_src[b, tok, h], dtype=np.float64)
        o, lse, dq, dk, dv = unit_rows_fwd_bwd(np.asarray(q_src[b, tok, h], dtype=np.float64),
                                               k_all, v_all, bdlm_mask_rows(L, block, rows),
                                               do_rows, scale)
        res.append({"unit": (b, st, blk, h), "o": o, "lse": lse, "dq": dq})
        if dk is not None:
            dk_sum[b, :, g] += dk
            dv_sum[b, :, g] += dv
    return res, dk_sum, dv_sum
