"""Seeded input generators.

Every tensor is drawn from torch's counter-based generator (Philox on the GPU,
its CPU generator on the host) seeded from (workload seed, tensor index), so a
tensor's values do not depend on which other tensors were drawn.  The draw is
fp32 N(0, 1) times a std, then cast to the workload dtype (bf16 casts round to
nearest even).  Both the oracle side and the GPU side read the *cast* values,
so they see bit-identical inputs.

Nothing here computes attention: draws, scalings of draws and casts only.
"""
from typing import Dict, Optional, Sequence

import numpy as np
import torch

TENSOR_ORDER = ("qc", "kc", "vc", "qx", "kx", "vx", "doc", "dox")
_OUTLIER_INDEX = len(TENSOR_ORDER)


def _torch_dtype(dtype: str) -> torch.dtype:
    if dtype == "bf16":
        return torch.bfloat16
    if dtype == "f32":
        return torch.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def _generator(device, seed: int, index: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1009 + int(index))
    return g


def draw_normal(shape: Sequence[int], seed: int, index: int, device="cpu",
                std: float = 1.0) -> torch.Tensor:
    """fp32 N(0, std^2) draw of `shape` for tensor number `index` of a workload."""
    g = _generator(device, seed, index)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _scale_outlier_rows(kc: torch.Tensor, kx: torch.Tensor, frac: float, mult: float,
                        seed: int) -> None:
    """Scale round(frac * rows) key rows, chosen without replacement over both
    streams, by `mult` (in fp32, before the dtype cast).  A row is one
    (stream, batch, token, kv-head) key vector."""
    if frac <= 0.0:
        return
    d = kc.shape[-1]
    rows_c = kc.reshape(-1, d)
    rows_x = kx.reshape(-1, d)
    n_c = rows_c.shape[0]
    n = n_c + rows_x.shape[0]
    count = int(round(frac * n))
    g = _generator(kc.device, seed, _OUTLIER_INDEX)
    pick = torch.randperm(n, generator=g, device=kc.device)[:count]
    pc = pick[pick < n_c]
    px = pick[pick >= n_c] - n_c
    rows_c[pc] *= mult
    rows_x[px] *= mult


def make_full_inputs(w, device="cpu", sharp: bool = False, seqlen: Optional[int] = None,
                     block: Optional[int] = None, batch: Optional[int] = None,
                     seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Inputs of a full-mode call: Q/K/V and upstream dO for both streams.

    Layout is [batch, tokens, heads, head_dim] (row-major).  `sharp` draws Q
    and K unscaled (N(0,1)) so that the logits at scale 1/sqrt(d) are ~N(0,1);
    the pre-scaled draws make the softmax nearly uniform.
    """
    L = seqlen or w.seqlen
    b = batch or w.batch
    s = w.seed if seed is None else seed
    td = _torch_dtype(w.dtype)
    qshape = (b, L, w.hq, w.head_dim)
    kshape = (b, L, w.hkv, w.head_dim)
    qk_std = 1.0 if sharp else w.q_std
    stds = {"qc": qk_std, "kc": qk_std, "vc": w.q_std, "qx": qk_std, "kx": qk_std,
            "vx": w.q_std, "doc": 1.0, "dox": 1.0}
    out = {}
    for i, name in enumerate(TENSOR_ORDER):
        shape = qshape if name in ("qc", "qx", "doc", "dox") else kshape
        out[name] = draw_normal(shape, s, i, device, stds[name])
    _scale_outlier_rows(out["kc"], out["kx"], w.outlier_frac, w.outlier_mult, s)
    for name in TENSOR_ORDER:
        out[name] = out[name].to(td).contiguous()
    return out


def draw_block_positions(nblocks: int, count: int, seed: int) -> np.ndarray:
    """`count` distinct block ids drawn without replacement from [0, nblocks), sorted."""
    rng = np.random.default_rng(seed)
    ids = rng.choice(nblocks, size=count, replace=False)
    return np.sort(ids).astype(np.int32)


def make_share_inputs(w, device="cpu", sharp: bool = False, seqlen: Optional[int] = None,
                      nlocal: Optional[int] = None, block: Optional[int] = None,
                      seed: Optional[int] = None) -> Dict[str, object]:
    """Inputs of one rank's CSBP share: the full clean K/V, the rank's local
    corrupted blocks' Q/K/V and dO, and the blocks' sorted global ids."""
    L = seqlen or w.seqlen
    B = block or w.block
    nl = nlocal or w.share_blocks
    s = w.seed if seed is None else seed
    td = _torch_dtype(w.dtype)
    qk_std = 1.0 if sharp else w.q_std
    T = nl * B
    out = {
        "kc": draw_normal((1, L, w.hkv, w.head_dim), s, 1, device, qk_std),
        "vc": draw_normal((1, L, w.hkv, w.head_dim), s, 2, device, w.q_std),
        "qx": draw_normal((1, T, w.hq, w.head_dim), s, 3, device, qk_std),
        "kx": draw_normal((1, T, w.hkv, w.head_dim), s, 4, device, qk_std),
        "vx": draw_normal((1, T, w.hkv, w.head_dim), s, 5, device, w.q_std),
        "dox": draw_normal((1, T, w.hq, w.head_dim), s, 7, device, 1.0),
    }
    for k in list(out):
        out[k] = out[k].to(td).contiguous()
    out["block_ids"] = draw_block_positions(L // B, nl, s)
    if w.clean_share:
        ids = clean_shard_ids(L // B, w.share_ranks, 0)
        Tc = len(ids) * B
        out["qs"] = draw_normal((1, Tc, w.hq, w.head_dim), s, 8, device, qk_std).to(td).contiguous()
        out["dos"] = draw_normal((1, Tc, w.hq, w.head_dim), s, 9, device, 1.0).to(td).contiguous()
        out["clean_ids"] = ids
    return out


def clean_shard_ids(nblocks: int, nranks: int, rank: int) -> np.ndarray:
    """Clean blocks of `rank` when the clean sequence is sharded over `nranks`
    ranks in the zigzag layout: the blocks are cut into 2*nranks equal runs and
    rank r takes runs r and 2*nranks-1-r, which gives every rank the same
    number of visible (query, key) pairs under the clean stream's block-causal
    rule (a block b sees b+1 blocks).  Sorted block ids."""
    if nblocks % (2 * nranks):
        raise ValueError("nblocks must be a multiple of 2*nranks")
    run = nblocks // (2 * nranks)
    a = np.arange(rank * run, (rank + 1) * run)
    b = np.arange((2 * nranks - 1 - rank) * run, (2 * nranks - rank) * run)
    return np.concatenate([a, b]).astype(np.int64)


def draw_units(nblocks: int, hq: int, batch: int, count: int, seed: int,
               streams: Sequence[int] = (0, 1)) -> np.ndarray:
    """Sampled oracle units (batch, stream, block, q-head), stream 0 = clean,
    1 = corrupted.  The first and last block of each stream are always in the
    sample; the rest are drawn without repetition.  Returns int64 [count, 4]."""
    rng = np.random.default_rng(seed + 100)
    forced = []
    for st in streams:
        for blk in (0, nblocks - 1):
            forced.append((int(rng.integers(batch)), st, blk, int(rng.integers(hq))))
    seen = set(forced)
    units = list(dict.fromkeys(forced))
    total = batch * len(streams) * nblocks * hq
    count = min(count, total)
    while len(units) < count:
        u = (int(rng.integers(batch)), int(streams[rng.integers(len(streams))]),
             int(rng.integers(nblocks)), int(rng.integers(hq)))
        if u not in seen:
            seen.add(u)
            units.append(u)
    return np.asarray(units[:count], dtype=np.int64)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy on the host (bf16 and fp32 both widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
