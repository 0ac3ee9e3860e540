"""One rank's context-sharded block-parallel (CSBP) attention share, on one GPU.

Block parallelism gives a rank whole corrupted blocks; CSBP additionally shards
the shared clean sequence, so the rank sees the clean K/V prefix as a stream of
chunks ("Block Parallelism For Efficient Distributed Long-Context Diffusion
Language Model Training": abstract; review FAQ "What is CSBP?").  This module
drives that stream with the C-ABI calls:

forward   own-block partial, then per clean chunk a share-mode forward that
          merges its partial into the running (O, LSE) in place, inside the
          kernel's epilogue (accumulate = 1); a final one-part merge writes O in
          the input dtype.
backward  per clean chunk a share-mode backward with the final O and LSE (dQ
          added into one fp32 buffer, the chunk's clean dK/dV written at its
          window), plus the own-block backward.

Chunks that no local block can see (start >= max(block_ids) * B) are skipped.
Inside a chunk, blocks whose clean prefix ends before the chunk get the empty
partial (O = 0, LSE = -inf), which the merge kernel recognises without reading
its O.

The rank's own shard of the clean stream is the context-parallel half of the
same step (the clean sequence sharded across the ranks, Sec. 4 / Fig. 3 of the
paper): its clean query blocks attend to the clean keys of their own and every
earlier block, streamed in the same chunks (clean_share_forward /
clean_share_backward: the share-mode calls with clean_queries = 1, no
own-block term).
"""
from typing import List, Optional, Sequence, Tuple

import torch

from .api import bdlm_attn_bwd, bdlm_attn_fwd, bdlm_attn_merge_partials, desc_for, workspace


class ShareBuffers:
    """Preallocated buffers of a share step (so the timed loop allocates nothing)."""

    def __init__(self, qx: torch.Tensor, kc: torch.Tensor, kx: Optional[torch.Tensor] = None):
        b, T, hq, d = qx.shape
        dev = qx.device
        self.acc_o = torch.empty((b, T, hq, d), dtype=torch.float32, device=dev)
        self.acc_lse = torch.empty((b, hq, T), dtype=torch.float32, device=dev)
        self.o = torch.empty_like(qx)
        self.lse = torch.empty_like(self.acc_lse)
        self.dqx = torch.empty((b, T, hq, d), dtype=torch.float32, device=dev)
        self.dkc = torch.zeros_like(kc)
        self.dvc = torch.zeros_like(kc)
        self.dkx = torch.empty_like(kx) if kx is not None else None
        self.dvx = torch.empty_like(kx) if kx is not None else None
        self.ws = None


def _chunks(L: int, chunk: int, ids: Sequence[int], B: int) -> List[Tuple[int, int]]:
    """Chunks [start, end) of the clean sequence that at least one local block sees."""
    top = max(ids) * B
    return [(j, min(j + chunk, L)) for j in range(0, min(L, top), chunk)]


def share_forward(qx, kx, vx, kc, vc, ids: Sequence[int], B: int, chunk: int,
                  scale: Optional[float] = None, bufs: Optional[ShareBuffers] = None, stream=None):
    """Final (O, LSE) of the local corrupted blocks over their whole visible key
    set, assembled from streamed chunk partials.  Returns (O in qx.dtype, LSE)."""
    if qx.shape[0] != 1:
        raise ValueError("the share step streams one sequence (batch 1)")
    ids = [int(i) for i in ids]
    L = kc.shape[1]
    bufs = bufs or ShareBuffers(qx, kc, kx)
    d_own = desc_for(qx, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=0, kv_end=0, own_block=1)
    bdlm_attn_fwd(d_own, None, kc, vc, qx, kx, vx, None, bufs.acc_o, None, bufs.acc_lse, None, stream)
    for (j0, j1) in _chunks(L, chunk, ids, B):
        d = desc_for(qx, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=j0, kv_end=j1, own_block=0,
                     accumulate=1)
        bdlm_attn_fwd(d, None, kc, vc, qx, kx, vx, None, bufs.acc_o, None, bufs.acc_lse, None, stream)
    bdlm_attn_merge_partials([bufs.acc_o], [bufs.acc_lse], bufs.o, bufs.lse, stream)
    return bufs.o, bufs.lse


def share_backward(qx, kx, vx, kc, vc, ids: Sequence[int], B: int, chunk: int, o, lse, dox,
                   scale: Optional[float] = None, bufs: Optional[ShareBuffers] = None, stream=None):
    """Gradients of the share: returns (dqx fp32, dkc, dvc, dkx, dvx).  dkc/dvc
    rows that no local block sees are zero."""
    ids = [int(i) for i in ids]
    L = kc.shape[1]
    bufs = bufs or ShareBuffers(qx, kc, kx)
    bufs.dqx.zero_()
    top = max(ids) * B
    if top < L:
        bufs.dkc[:, top:].zero_()
        bufs.dvc[:, top:].zero_()
    d_full = desc_for(qx, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=0, kv_end=L, own_block=1)
    if bufs.ws is None:
        bufs.ws = workspace(d_full, True, qx.device)
    for (j0, j1) in _chunks(L, chunk, ids, B):
        d = desc_for(qx, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=j0, kv_end=j1, own_block=0)
        bdlm_attn_bwd(d, None, kc, vc, qx, kx, vx, None, o, None, lse, None, dox,
                      None, bufs.dkc, bufs.dvc, bufs.dqx, None, None, bufs.ws, stream)
    d_own = desc_for(qx, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=0, kv_end=0, own_block=1)
    bdlm_attn_bwd(d_own, None, kc, vc, qx, kx, vx, None, o, None, lse, None, dox,
                  None, bufs.dkc, bufs.dvc, bufs.dqx, bufs.dkx, bufs.dvx, bufs.ws, stream)
    return bufs.dqx, bufs.dkc, bufs.dvc, bufs.dkx, bufs.dvx


def _clean_chunks(L: int, chunk: int, ids: Sequence[int], B: int) -> List[Tuple[int, int]]:
    """Chunks that at least one local clean block sees (its prefix includes itself)."""
    top = (max(ids) + 1) * B
    return [(j, min(j + chunk, L)) for j in range(0, min(L, top), chunk)]


def clean_share_forward(qs, kc, vc, ids: Sequence[int], B: int, chunk: int,
                        scale: Optional[float] = None, bufs: Optional[ShareBuffers] = None, stream=None):
    """Final (O, LSE) of the rank's clean query blocks qs [1, n*B, Hq, d] (global
    clean block ids `ids`) over the clean keys of their own and every earlier
    block, assembled from streamed chunk partials."""
    if qs.shape[0] != 1:
        raise ValueError("the share step streams one sequence (batch 1)")
    ids = [int(i) for i in ids]
    L = kc.shape[1]
    bufs = bufs or ShareBuffers(qs, kc)
    for n, (j0, j1) in enumerate(_clean_chunks(L, chunk, ids, B)):
        d = desc_for(qs, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=j0, kv_end=j1, own_block=0,
                     clean_queries=1, accumulate=int(n > 0))
        bdlm_attn_fwd(d, None, kc, vc, qs, None, None, None, bufs.acc_o, None, bufs.acc_lse, None, stream)
    bdlm_attn_merge_partials([bufs.acc_o], [bufs.acc_lse], bufs.o, bufs.lse, stream)
    return bufs.o, bufs.lse


def clean_share_backward(qs, kc, vc, ids: Sequence[int], B: int, chunk: int, o, lse, dos,
                         scale: Optional[float] = None, bufs: Optional[ShareBuffers] = None, stream=None):
    """Gradients of the clean-query share: returns (dq fp32, dkc, dvc).  dkc/dvc
    rows that no local block sees are zero."""
    ids = [int(i) for i in ids]
    L = kc.shape[1]
    bufs = bufs or ShareBuffers(qs, kc)
    bufs.dqx.zero_()
    top = (max(ids) + 1) * B
    if top < L:
        bufs.dkc[:, top:].zero_()
        bufs.dvc[:, top:].zero_()
    d_full = desc_for(qs, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=0, kv_end=L, own_block=0,
                      clean_queries=1)
    if bufs.ws is None:
        bufs.ws = workspace(d_full, True, qs.device)
    for (j0, j1) in _clean_chunks(L, chunk, ids, B):
        d = desc_for(qs, kc, B, scale, seqlen=L, block_ids=ids, kv_begin=j0, kv_end=j1, own_block=0,
                     clean_queries=1)
        bdlm_attn_bwd(d, None, kc, vc, qs, None, None, None, o, None, lse, None, dos,
                      None, bufs.dkc, bufs.dvc, bufs.dqx, None, None, bufs.ws, stream)
    return bufs.dqx, bufs.dkc, bufs.dvc


# ------------------------------------------------- staged clean chunks (bounded)
class StagedBuffers(ShareBuffers):
    """Buffers of a share step whose clean K/V never reside whole on the rank:
    two chunk-sized staging slots for K/V (the one being consumed and the one
    being received) and two for the chunk's clean dK/dV (the one being written
    and the one being sent), as an all-gather / reduce-scatter pair would use
    them.  The local corrupted blocks' buffers are those of ShareBuffers."""

    def __init__(self, qx: torch.Tensor, kx: Optional[torch.Tensor], hkv: int, chunk: int):
        b, T, hq, d = qx.shape
        dev, dt = qx.device, qx.dtype
        shape = (b, chunk, hkv, d)
        self.k_stage = [torch.empty(shape, dtype=dt, device=dev) for _ in range(2)]
        self.v_stage = [torch.empty(shape, dtype=dt, device=dev) for _ in range(2)]
        self.dk_stage = [torch.empty(shape, dtype=dt, device=dev) for _ in range(2)]
        self.dv_stage = [torch.empty(shape, dtype=dt, device=dev) for _ in range(2)]
        self.chunk = chunk
        self.acc_o = torch.empty((b, T, hq, d), dtype=torch.float32, device=dev)
        self.acc_lse = torch.empty((b, hq, T), dtype=torch.float32, device=dev)
        self.o = torch.empty_like(qx)
        self.lse = torch.empty_like(self.acc_lse)
        self.dqx = torch.empty((b, T, hq, d), dtype=torch.float32, device=dev)
        self.dkc = self.dvc = None
        self.dkx = torch.empty_like(kx) if kx is not None else None
        self.dvx = torch.empty_like(kx) if kx is not None else None
        self.ws = None


def share_forward_staged(qx, kx, vx, L: int, ids: Sequence[int], B: int, chunk: int, fetch,
                         scale: Optional[float] = None, bufs: Optional[StagedBuffers] = None,
                         stream=None, clean_queries: int = 0):
    """share_forward / clean_share_forward with the clean K/V delivered chunk
    by chunk into a staging slot: fetch(j0, j1, k_dst, v_dst) fills k_dst, v_dst
    [batch, j1 - j0, Hkv, d] with clean rows [j0, j1) on `stream` (on one GPU
    a copy stands in for the all-gather's receive).  Returns (O, LSE)."""
    if qx.shape[0] != 1:
        raise ValueError("the share step streams one sequence (batch 1)")
    ids = [int(i) for i in ids]
    own = 0 if clean_queries else 1
    wins = _clean_chunks(L, chunk, ids, B) if clean_queries else _chunks(L, chunk, ids, B)
    first = True
    if own:
        ks, vs = bufs.k_stage[0][:, :0], bufs.v_stage[0][:, :0]      # the own-block call reads no clean key
        d = desc_for(qx, ks, B, scale, seqlen=L, block_ids=ids, kv_begin=0, kv_end=0, own_block=1, kv_staged=1)
        bdlm_attn_fwd(d, None, ks, vs, qx, kx, vx, None, bufs.acc_o, None, bufs.acc_lse, None, stream)
        first = False
    for n, (j0, j1) in enumerate(wins):
        ks, vs = bufs.k_stage[n % 2][:, :j1 - j0], bufs.v_stage[n % 2][:, :j1 - j0]
        fetch(j0, j1, ks, vs)
        d = desc_for(qx, ks, B, scale, seqlen=L, block_ids=ids, kv_begin=j0, kv_end=j1, own_block=0,
                     clean_queries=clean_queries, accumulate=0 if first else 1, kv_staged=1)
        bdlm_attn_fwd(d, None, ks, vs, qx, kx if own else None, vx if own else None, None, bufs.acc_o, None,
                      bufs.acc_lse, None, stream)
        first = False
    bdlm_attn_merge_partials([bufs.acc_o], [bufs.acc_lse], bufs.o, bufs.lse, stream)
    return bufs.o, bufs.lse


def share_backward_staged(qx, kx, vx, L: int, ids: Sequence[int], B: int, chunk: int, o, lse, dox, fetch,
                          deliver, scale: Optional[float] = None, bufs: Optional[StagedBuffers] = None,
                          stream=None, clean_queries: int = 0):
    """share_backward / clean_share_backward with staged chunks: each chunk's
    clean K/V are fetched again (fetch as in share_forward_staged) and its clean
    dK/dV, written into a staging slot, are handed to deliver(j0, j1, dk, dv)
    (on one GPU a copy stands in for the reduce-scatter's send).  Returns
    (dqx fp32, dkx, dvx); dkx, dvx are None for clean query blocks."""
    ids = [int(i) for i in ids]
    own = 0 if clean_queries else 1
    wins = _clean_chunks(L, chunk, ids, B) if clean_queries else _chunks(L, chunk, ids, B)
    bufs.dqx.zero_()
    if bufs.ws is None:
        d_full = desc_for(qx, bufs.k_stage[0], B, scale, seqlen=L, block_ids=ids, kv_begin=0,
                          kv_end=min(chunk, L), own_block=own, clean_queries=clean_queries, kv_staged=1)
        bufs.ws = workspace(d_full, True, qx.device)
    for n, (j0, j1) in enumerate(wins):
        W = j1 - j0
        ks, vs = bufs.k_stage[n % 2][:, :W], bufs.v_stage[n % 2][:, :W]
        dks, dvs = bufs.dk_stage[n % 2][:, :W], bufs.dv_stage[n % 2][:, :W]
        fetch(j0, j1, ks, vs)
        d = desc_for(qx, ks, B, scale, seqlen=L, block_ids=ids, kv_begin=j0, kv_end=j1, own_block=0,
                     clean_queries=clean_queries, kv_staged=1)
        bdlm_attn_bwd(d, None, ks, vs, qx, kx if own else None, vx if own else None, None, o, None, lse, None,
                      dox, None, dks, dvs, bufs.dqx, None, None, bufs.ws, stream)
        deliver(j0, j1, dks, dvs)
    if own:
        ks, vs = bufs.k_stage[0][:, :0], bufs.v_stage[0][:, :0]
        dks, dvs = bufs.dk_stage[0][:, :0], bufs.dv_stage[0][:, :0]
        d = desc_for(qx, ks, B, scale, seqlen=L, block_ids=ids, kv_begin=0, kv_end=0, own_block=1, kv_staged=1)
        bdlm_attn_bwd(d, None, ks, vs, qx, kx, vx, None, o, None, lse, None, dox,
                      None, dks, dvs, bufs.dqx, bufs.dkx, bufs.dvx, bufs.ws, stream)
    return bufs.dqx, bufs.dkx, bufs.dvx


# ------------------------------------------------------------------ rank layout
def rank_blocks(nblocks: int, nranks: int, rank: int, layout: str = "zigzag") -> List[int]:
    """Blocks a rank owns (its corrupted target blocks and its shard of the
    clean sequence).  Block b costs b + 1 block-pairs in either half (a
    corrupted block sees b clean blocks plus itself; a clean block sees the
    clean blocks up to itself), so a contiguous cut loads the last rank about
    twice the mean.  "zigzag" cuts the blocks into 2R equal runs and gives
    rank r runs r and 2R-1-r, which equalises the cost exactly; "contiguous"
    gives rank r the r-th of R equal runs."""
    if nblocks % (2 * nranks) or not 0 <= rank < nranks:
        raise ValueError("need nblocks % (2*nranks) == 0 and 0 <= rank < nranks")
    if layout == "contiguous":
        run = nblocks // nranks
        return list(range(rank * run, (rank + 1) * run))
    if layout != "zigzag":
        raise ValueError(f"unknown layout {layout!r}")
    run = nblocks // (2 * nranks)
    return list(range(rank * run, (rank + 1) * run)) + \
        list(range((2 * nranks - 1 - rank) * run, (2 * nranks - rank) * run))


def rank_cost(ids: Sequence[int]) -> int:
    """Visible block-pairs of a rank's blocks in one half of its share."""
    return sum(int(b) + 1 for b in ids)
