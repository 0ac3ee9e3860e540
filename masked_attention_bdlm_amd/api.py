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
    if t.numel() == 0:
        # torch reports address 0 for an empty tensor; an empty view (say a
        # staged window of no rows) still has the address of its storage
        return ctypes.c_void_p(t.untyped_storage().data_ptr() + t.storage_offset() * t.element_size())
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
             clean_queries=0, accumulate=0, kv_staged=0):
    """Descriptor from Q [batch, tokens, Hq, d] and K [batch, L, Hkv, d] (with
    kv_staged, K holds only the window and `seqlen` must be given)."""
    b, _, hq, d = q.shape
    hkv = k.shape[2]
    if kv_staged and seqlen is None:
        raise ValueError("a staged window needs the clean sequence length (seqlen)")
    L = seqlen if seqlen is not None else k.shape[1]
    if scale is None:
        scale = d ** -0.5
    return make_desc(b, L, block, hq, hkv, d, dtype_code(q.dtype), scale, block_ids,
                     kv_begin, kv_end, own_block, clean_queries, accumulate, kv_staged)


# ------------------------------------------------------------ argument checks
# The C ABI takes raw pointers and derives every size from the descriptor, so a
# tensor of the wrong dtype or shape would be read or written out of bounds.
# These checks run on the host before any pointer is passed on.
_TORCH_OF = {BDLM_BF16: torch.bfloat16, BDLM_F32: torch.float32}


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype, device=None, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device} (all tensors on one device)")


def _forbid(**named):
    for k, v in named.items():
        if v is not None:
            raise ValueError(f"{k} must be None in share mode")


def _shapes(desc):
    b, L, hq, hkv, d = desc.batch, desc.seqlen, desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    rows = L if desc.num_local_blocks == 0 else desc.num_local_blocks * desc.block
    kvrows = desc.kv_end - desc.kv_begin if (desc.num_local_blocks and desc.kv_staged) else L
    return (b, rows, hq, d), (b, kvrows, hkv, d), (b, rows, hkv, d), (b, hq, rows)


def check_fwd_args(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x):
    """Shapes, dtypes and device of a bdlm_attn_fwd call against `desc`."""
    dt = _TORCH_OF.get(desc.dtype)
    if dt is None:
        raise ValueError(f"descriptor dtype {desc.dtype} is not BDLM_F32 or BDLM_BF16")
    qs, kcs, kxs, ls = _shapes(desc)
    dev = qx.device if qx is not None else None
    _expect(qx, "qx", qs, dt, dev)
    _expect(kc, "kc", kcs, dt, dev)
    _expect(vc, "vc", kcs, dt, dev)
    if desc.num_local_blocks == 0:
        for n, t, shp in (("qc", qc, qs), ("kx", kx, kxs), ("vx", vx, kxs), ("oc", oc, qs), ("ox", ox, qs)):
            _expect(t, n, shp, dt, dev)
        _expect(lse_c, "lse_c", ls, torch.float32, dev)
    else:
        _forbid(qc=qc, oc=oc, lse_c=lse_c)
        opt = not desc.own_block
        _expect(kx, "kx", kxs, dt, dev, optional=opt)
        _expect(vx, "vx", kxs, dt, dev, optional=opt)
        _expect(ox, "ox (share-mode partial, fp32)", qs, torch.float32, dev)
    _expect(lse_x, "lse_x", ls, torch.float32, dev)


def check_bwd_args(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox,
                   dqc, dkc, dvc, dqx, dkx, dvx):
    """Shapes, dtypes and device of a bdlm_attn_bwd call against `desc`."""
    dt = _TORCH_OF.get(desc.dtype)
    if dt is None:
        raise ValueError(f"descriptor dtype {desc.dtype} is not BDLM_F32 or BDLM_BF16")
    qs, kcs, kxs, ls = _shapes(desc)
    dev = qx.device if qx is not None else None
    for n, t, shp in (("qx", qx, qs), ("kc", kc, kcs), ("vc", vc, kcs), ("ox", ox, qs), ("dox", dox, qs),
                      ("dkc", dkc, kcs), ("dvc", dvc, kcs)):
        _expect(t, n, shp, dt, dev)
    _expect(lse_x, "lse_x", ls, torch.float32, dev)
    if desc.num_local_blocks == 0:
        for n, t, shp in (("qc", qc, qs), ("kx", kx, kxs), ("vx", vx, kxs), ("oc", oc, qs), ("doc", doc, qs),
                          ("dqc", dqc, qs), ("dqx", dqx, qs), ("dkx", dkx, kxs), ("dvx", dvx, kxs)):
            _expect(t, n, shp, dt, dev)
        _expect(lse_c, "lse_c", ls, torch.float32, dev)
    else:
        _forbid(qc=qc, oc=oc, lse_c=lse_c, doc=doc, dqc=dqc)
        _expect(dqx, "dqx (share-mode accumulator, fp32)", qs, torch.float32, dev)
        opt = not desc.own_block
        for n, t in (("kx", kx), ("vx", vx), ("dkx", dkx), ("dvx", dvx)):
            _expect(t, n, kxs, dt, dev, optional=opt)


def check_merge_args(o_parts, lse_parts, o_out, lse_out):
    """All partials fp32 of one shape [b, T, H, d] / [b, H, T] on one device."""
    if len(o_parts) != len(lse_parts) or len(o_parts) == 0:
        raise ValueError("need the same positive number of O and LSE partials")
    b, T, H, d = o_parts[0].shape
    dev = o_parts[0].device
    for j, (o, l) in enumerate(zip(o_parts, lse_parts)):
        _expect(o, f"o_parts[{j}]", (b, T, H, d), torch.float32, dev)
        _expect(l, f"lse_parts[{j}]", (b, H, T), torch.float32, dev)
    if o_out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"o_out: dtype {o_out.dtype}, expected float32 or bfloat16")
    _expect(o_out, "o_out", (b, T, H, d), o_out.dtype, dev)
    _expect(lse_out, "lse_out", (b, H, T), torch.float32, dev)


# ---------------------------------------------------------------- C-ABI calls
def bdlm_attn_workspace_bytes(desc, for_bwd: bool) -> int:
    return int(load().bdlm_attn_workspace_bytes(ctypes.byref(desc), int(bool(for_bwd))))


def bdlm_attn_fwd(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, ws=None, stream=None):
    check_fwd_args(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x)
    ref = qx
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().bdlm_attn_fwd(ctypes.byref(desc), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(qx), _ptr(kx),
                              _ptr(vx), _ptr(oc), _ptr(ox), _ptr(lse_c), _ptr(lse_x), _ptr(ws), wsb,
                              _stream(stream, ref))
    check("bdlm_attn_fwd", st)


def bdlm_attn_bwd(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox,
                  dqc, dkc, dvc, dqx, dkx, dvx, ws=None, stream=None):
    check_bwd_args(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox, dqc, dkc, dvc, dqx, dkx, dvx)
    ref = qx
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().bdlm_attn_bwd(ctypes.byref(desc), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(qx), _ptr(kx),
                              _ptr(vx), _ptr(oc), _ptr(ox), _ptr(lse_c), _ptr(lse_x), _ptr(doc),
                              _ptr(dox), _ptr(dqc), _ptr(dkc), _ptr(dvc), _ptr(dqx), _ptr(dkx),
                              _ptr(dvx), _ptr(ws), wsb, _stream(stream, ref))
    check("bdlm_attn_bwd", st)


def bdlm_attn_bwd_noalloc(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox,
                          dqc, dkc, dvc, dqx, dkx, dvx, stream=None):
    """bdlm_attn_bwd with the library's fixed per-GPU workspace array (no
    workspace argument, nothing allocated)."""
    check_bwd_args(desc, qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox, dqc, dkc, dvc, dqx, dkx, dvx)
    st = load().bdlm_attn_bwd_noalloc(ctypes.byref(desc), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(qx), _ptr(kx),
                                      _ptr(vx), _ptr(oc), _ptr(ox), _ptr(lse_c), _ptr(lse_x), _ptr(doc),
                                      _ptr(dox), _ptr(dqc), _ptr(dkc), _ptr(dvc), _ptr(dqx), _ptr(dkx),
                                      _ptr(dvx), _stream(stream, qx))
    check("bdlm_attn_bwd_noalloc", st)


def bdlm_attn_merge_partials(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor],
                             o_out: torch.Tensor, lse_out: torch.Tensor, stream=None):
    check_merge_args(o_parts, lse_parts, o_out, lse_out)
    n = len(o_parts)
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


class _BdlmAttention(torch.autograd.Function):
    """Full-mode BDLM attention as an autograd function.  Forward and backward
    are the library's bdlm_attn_fwd and bdlm_attn_bwd; the saved tensors are
    the inputs, O and the LSE rows (the backward recomputes P from them)."""

    @staticmethod
    def forward(ctx, qc, kc, vc, qx, kx, vx, block, scale):
        oc, ox, lse_c, lse_x = attention_fwd(qc, kc, vc, qx, kx, vx, block, scale)
        ctx.save_for_backward(qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x)
        ctx.block, ctx.scale = block, scale
        return oc, ox

    @staticmethod
    def backward(ctx, doc, dox):
        qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x = ctx.saved_tensors
        doc = torch.zeros_like(oc) if doc is None else doc.contiguous()
        dox = torch.zeros_like(ox) if dox is None else dox.contiguous()
        grads = attention_bwd(qc, kc, vc, qx, kx, vx, oc, ox, lse_c, lse_x, doc, dox, ctx.block, ctx.scale)
        return (*grads, None, None)


def bdlm_attention(qc, kc, vc, qx, kx, vx, block: int, scale: Optional[float] = None):
    """Differentiable full-mode BDLM attention over [x0 ; xt]: returns (oc, ox).
    Inputs are [batch, L, heads, d] device tensors as for attention_fwd; the
    gradients of qc, kc, vc, qx, kx, vx come from bdlm_attn_bwd."""
    return _BdlmAttention.apply(qc, kc, vc, qx, kx, vx, block, scale)


def share_fwd(qx, kx, vx, kc, vc, block_ids, block: int, kv_begin: int, kv_end: int,
              own_block: int, scale: Optional[float] = None, out=None, stream=None, clean_queries: int = 0,
              accumulate: int = 0, seqlen: Optional[int] = None, kv_staged: int = 0):
    """Share-mode partial over one key window: returns (O_part fp32, LSE_part).

    clean_queries=1: qx holds clean query blocks (each sees the clean keys of its
    own and every earlier block); kx, vx may then be None.  accumulate=1: merge
    the partial into the (O, LSE) already held in `out` instead.  kv_staged=1:
    kc, vc hold only the window's rows (then `seqlen` = L is required)."""
    desc = desc_for(qx, kc, block, scale, seqlen=seqlen, block_ids=block_ids, kv_begin=kv_begin, kv_end=kv_end,
                    own_block=own_block, clean_queries=clean_queries, accumulate=accumulate, kv_staged=kv_staged)
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
              clean_queries: int = 0, seqlen: Optional[int] = None, kv_staged: int = 0):
    """Share-mode backward of one key window (adds into dqx_acc, writes the window of dkc/dvc;
    with kv_staged=1, kc/vc/dkc/dvc hold only the window's rows)."""
    desc = desc_for(qx, kc, block, scale, seqlen=seqlen, block_ids=block_ids, kv_begin=kv_begin, kv_end=kv_end,
                    own_block=own_block, clean_queries=clean_queries, kv_staged=kv_staged)
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
def schedule_walk(desc, for_bwd: int, want_cover: bool = True):
    """Host walk of a kernel's work decomposition (batch 0, q-head 0): for_bwd
    0 = forward, 1 = dK/dV kernel, 2 = dQ kernel.

    Returns (cover uint8 [rows, keys] or None, stats dict)."""
    import numpy as np
    lib = load()
    rows = desc.seqlen * 2 if desc.num_local_blocks == 0 else desc.num_local_blocks * desc.block
    keys = desc.seqlen * 2 if desc.num_local_blocks == 0 else desc.seqlen + desc.num_local_blocks * desc.block
    cover = np.zeros((rows, keys), dtype=np.uint8) if want_cover else None
    stats = (ctypes.c_int64 * 5)()
    if for_bwd not in (0, 1, 2):
        raise ValueError("for_bwd: 0 forward, 1 dK/dV kernel, 2 dQ kernel")
    st = lib.bdlm_attn_schedule_walk(ctypes.byref(desc), int(for_bwd),
                                     cover.ctypes.data_as(ctypes.c_void_p) if want_cover else None,
                                     cover.size if want_cover else 0, stats)
    check("bdlm_attn_schedule_walk", st)
    names = ("workgroups", "tile_visits", "masked_visits", "pairs", "errors")
    return cover, dict(zip(names, [int(x) for x in stats]))


def bdlm_calib_mfma(mode: int, workgroups: int, iters: int, cycles: torch.Tensor, sink: torch.Tensor,
                    stream=None):
    """Calibration launch of the sustained bf16 MFMA probe (modes 0-3, see
    include/bdlm_attn.h); cycles: int64 [workgroups * 16], sink: float32
    [workgroups * 512], both on the GPU."""
    _expect(cycles, "cycles", (workgroups * 16,), torch.int64)
    _expect(sink, "sink", (workgroups * 512,), torch.float32, cycles.device)
    st = load().bdlm_calib_mfma(int(mode), int(workgroups), int(iters), _ptr(cycles), _ptr(sink),
                                _stream(stream, cycles))
    check("bdlm_calib_mfma", st)


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
