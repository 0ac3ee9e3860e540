"""Thin torch-facing binding of the C ABI.

The functions named like the C entry points (bdlm_attn_fwd, bdlm_attn_bwd,
bdlm_attn_merge_partials, bdlm_attn_workspace_bytes) pass tensor data pointers
and the current HIP stream straight through.  The convenience wrappers
(attention_fwd, attention_bwd, share_fwd, share_bwd, merge_partials) only
allocate outputs and workspaces with torch before making the same calls.
Every step of the computation runs in the HIP kernels of libbdlm_attn.so.
"""
import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import BDLM_BF16, BDLM_F32, check, load, make_desc

_DT = {torch.bfloat16: BDLM_BF16, torch.float32: BDLM_F32}


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (row-major [batch, tokens, heads, head_dim])")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref: torch.Tensor):
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}: use torch.bfloat16 or torch.float32")
    return _DT[dt]


def desc_for(q: torch.Tensor, k: torch.Tensor, block: int, scale: Optional[float] = None,
             seqlen: Optional[int] = None, block_ids=None, kv_begin=0, kv_end=0, own_block=0,
             clean_queries=0, accumulate=0):
    """Descriptor from Q [batch, tokens, Hq, d] and K [batch, L, Hkv, d]."""
    b, _, hq, d = q.shape
    hkv = k.shape[2]
    L = seqlen if seqlen is not None else k.shape[1]
    if scale is None:
        scale = d ** -0.5
    return make_desc(b, L, block, hq, hkv, d, dtype_code(q.dtype), scale, block_ids,
                     kv_begin, kv_end, own_block, clean_queries, accumulate)


# ---------------------------------------------------------------- C-ABI calls
def bdlm_attn_workspace_bytes(desc, for_bwd: bool) -> int:
    return int(load().bdlm_attn_workspace_bytes(ctypes.byref(desc), int(bool(for_bwd))))


def bdlm_attn_fwd(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, ws=None, stream=None):
    ref = qx
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().bdlm_attn_fwd(ctypes.byref(desc), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(qx), _ptr(kx),
                              _ptr(vx), _ptr(oc), _ptr(ox), _ptr(lse_c), _ptr(lse_x), _ptr(ws), wsb,
                              _stream(stream, ref))
    check("bdlm_attn_fwd", st)


def bdlm_attn_bwd(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox,
                  dqc, dkc, dvc, dqx, dkx, dvx, ws=None, stream=None):
    ref = qx
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().bdlm_attn_bwd(ctypes.byref(desc), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(qx), _ptr(kx),
                              _ptr(vx), _ptr(oc), _ptr(ox), _ptr(lse_c), _ptr(lse_x), _ptr(doc),
                              _ptr(dox), _ptr(dqc), _ptr(dkc), _ptr(dvc), _ptr(dqx), _ptr(dkx),
                              _ptr(dvx), _ptr(ws), wsb, _stream(stream, ref))
    check("bdlm_attn_bwd", st)


def bdlm_attn_merge_partials(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor],
                             o_out: torch.Tensor, lse_out: torch.Tensor, stream=None):
    n = len(o_parts)
    if n != len(lse_parts) or n == 0:
        raise ValueError("need the same positive number of O and LSE partials")
    b, T, H, d = o_parts[0].shape
    op = (ctypes.c_void_p * n)(*[_ptr(t).value for t in o_parts])
    lp = (ctypes.c_void_p * n)(*[_ptr(t).value for t in lse_parts])
    st = load().bdlm_attn_merge_partials(n, b, T, H, d, op, lp, _ptr(o_out), dtype_code(o_out.dtype),
                                         _ptr(lse_out), _stream(stream, o_out))
    check("bdlm_attn_merge_partials", st)


# --------------------------------------------------------- convenience wrappers
def workspace(desc, for_bwd: bool, device) -> Optional[torch.Tensor]:
    n = bdlm_attn_workspace_bytes(desc, for_bwd)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def attention_fwd(qc, kc, vc, qx, kx, vx, block: int, scale: Optional[float] = None, stream=None):
    """Full-mode forward: returns (oc, ox, lse_c, lse_x)."""
    desc = desc_for(qc, kc, block, scale)
    b, L, hq, _ = qc.shape
    oc, ox = torch.empty_like(qc), torch.empty_like(qx)
    lse_c = torch.empty((b, hq, L), dtype=torch.float32, device=qc.device)
    lse_x = torch.empty_like(lse_c)
    bdlm_attn_fwd(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, None, stream)
    return oc, ox, lse_c, lse_x


def attention_bwd(qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox, block: int,
                  scale: Optional[float] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Full-mode backward: returns (dqc, dkc, dvc, dqx, dkx, dvx)."""
    desc = desc_for(qc, kc, block, scale)
    if ws is None:
        ws = workspace(desc, True, qc.device)
    dqc, dqx = torch.empty_like(qc), torch.empty_like(qx)
    dkc, dvc, dkx, dvx = (torch.empty_like(kc) for _ in range(4))
    bdlm_attn_bwd(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox,
                  dqc, dkc, dvc, dqx, dkx, dvx, ws, stream)
    return dqc, dkc, dvc, dqx, dkx, dvx


def share_fwd(qx, kx, vx, kc, vc, block_ids, block: int, kv_begin: int, kv_end: int,
              own_block: int, scale: Optional[float] = None, out=None, stream=None, clean_queries: int = 0,
              accumulate: int = 0):
    """Share-mode partial over one key window: returns (O_part fp32, LSE_part).

    clean_queries=1: qx holds clean query blocks (each sees the clean keys of its
    own and every earlier block); kx, vx may then be None.  accumulate=1: merge
    the partial into the (O, LSE) already held in `out` instead."""
    desc = desc_for(qx, kc, block, scale, block_ids=block_ids, kv_begin=kv_begin, kv_end=kv_end,
                    own_block=own_block, clean_queries=clean_queries, accumulate=accumulate)
    b, T, hq, d = qx.shape
    if out is None:
        o = torch.empty((b, T, hq, d), dtype=torch.float32, device=qx.device)
        lse = torch.empty((b, hq, T), dtype=torch.float32, device=qx.device)
    else:
        o, lse = out
    bdlm_attn_fwd(desc, None, kc, vc, qx, kx, vx, None, o, None, lse, None, stream)
    return o, lse


def share_bwd(qx, kx, vx, kc, vc, block_ids, block: int, kv_begin: int, kv_end: int, own_block: int,
              o_final, lse_final, dox, dqx_acc, dkc, dvc, dkx=None, dvx=None,
              scale: Optional[float] = None, ws: Optional[torch.Tensor] = None, stream=None,
              clean_queries: int = 0):
    """Share-mode backward of one key window (adds into dqx_acc, writes the window of dkc/dvc)."""
    desc = desc_for(qx, kc, block, scale, block_ids=block_ids, kv_begin=kv_begin, kv_end=kv_end,
                    own_block=own_block, clean_queries=clean_queries)
    if ws is None:
        ws = workspace(desc, True, qx.device)
    bdlm_attn_bwd(desc, None, kc, vc, qx, kx, vx, None, o_final, None, lse_final, None, dox,
                  None, dkc, dvc, dqx_acc, dkx, dvx, ws, stream)


def merge_partials(o_parts: List[torch.Tensor], lse_parts: List[torch.Tensor],
                   out_dtype: torch.dtype = torch.float32, out=None, stream=None):
    """Merge (O, LSE) partials; returns (O, LSE)."""
    if out is None:
        o = torch.empty(o_parts[0].shape, dtype=out_dtype, device=o_parts[0].device)
        lse = torch.empty_like(lse_parts[0])
    else:
        o, lse = out
    bdlm_attn_merge_partials(o_parts, lse_parts, o, lse, stream)
    return o, lse


# ---------------------------------------------------------------- diagnostics
def schedule_walk(desc, for_bwd: bool, want_cover: bool = True):
    """Host walk of the kernels' work decomposition (batch 0, q-head 0).

    Returns (cover uint8 [rows, keys] or None, stats dict)."""
    import numpy as np
    lib = load()
    rows = desc.seqlen * 2 if desc.num_local_blocks == 0 else desc.num_local_blocks * desc.block
    keys = desc.seqlen * 2 if desc.num_local_blocks == 0 else desc.seqlen + desc.num_local_blocks * desc.block
    cover = np.zeros((rows, keys), dtype=np.uint8) if want_cover else None
    stats = (ctypes.c_int64 * 5)()
    st = lib.bdlm_attn_schedule_walk(ctypes.byref(desc), int(bool(for_bwd)),
                                     cover.ctypes.data_as(ctypes.c_void_p) if want_cover else None,
                                     cover.size if want_cover else 0, stats)
    check("bdlm_attn_schedule_walk", st)
    names = ("workgroups", "tile_visits", "masked_visits", "pairs", "errors")
    return cover, dict(zip(names, [int(x) for x in stats]))


class KernelTimer:
    """Context manager around bdlm_attn_profile_begin/end: per-kernel HIP-event
    totals of every launch the library makes inside the block."""

    def __init__(self, max_launches: int = 4096):
        self.max_launches = max_launches
        self.times = {}

    def __enter__(self):
        check("bdlm_attn_profile_begin", load().bdlm_attn_profile_begin(self.max_launches))
        return self

    def __exit__(self, *exc):
        arr = (_lib.BdlmKernelTime * 32)()
        n = ctypes.c_int32(0)
        check("bdlm_attn_profile_end", load().bdlm_attn_profile_end(arr, 32, ctypes.byref(n)))
        self.times = {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms))
                      for i in range(n.value)}
        return False
