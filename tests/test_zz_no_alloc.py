"""bdlm_attn_bwd_noalloc (the backward with the library's fixed per-GPU
workspace array) against bdlm_attn_bwd with a caller-allocated workspace,
through the C ABI: the same kernels run, so the gradients must be
bit-identical; they are also held to the bf16 tolerances against each other.
Two calls in a row, the second on a smaller problem (the array keeps the first
call's contents), plus a share-mode call and the size limit."""
import ctypes

import pytest
import torch

import masked_attention_bdlm_amd as M
from masked_attention_bdlm_amd import api
from masked_attention_bdlm_amd._lib import make_desc
from synth import Workload, make_full_inputs, make_share_inputs
from tests.gpu_util import announce, check_outputs, host, require_gpu

pytestmark = pytest.mark.gpu


def _full_case(L, B, hq, hkv, d, seed):
    w = Workload(name="noalloc", batch=1, seqlen=L, block=B, hq=hq, hkv=hkv, head_dim=d, dtype="bf16",
                 seed=seed, q_std=d ** -0.5)
    x = make_full_inputs(w, device="cuda", sharp=True)
    oc, ox, lc, lx = M.attention_fwd(x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], B, w.scale)
    return w, x, (oc, ox, lc, lx)


def _grads(x):
    return (torch.empty_like(x["qc"]), torch.empty_like(x["kc"]), torch.empty_like(x["kc"]),
            torch.empty_like(x["qx"]), torch.empty_like(x["kx"]), torch.empty_like(x["kx"]))


def _compare(w, x, fw):
    oc, ox, lc, lx = fw
    desc = api.desc_for(x["qc"], x["kc"], w.block, w.scale)
    ref = _grads(x)
    ws = api.workspace(desc, True, x["qc"].device)
    api.bdlm_attn_bwd(desc, x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], oc, ox, lc, lx,
                      x["doc"], x["dox"], *ref, ws)
    got = _grads(x)
    api.bdlm_attn_bwd_noalloc(desc, x["qc"], x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], oc, ox, lc, lx,
                              x["doc"], x["dox"], *got)
    torch.cuda.synchronize()
    names = ("dqc", "dkc", "dvc", "dqx", "dkx", "dvx")
    for n, a, b in zip(names, got, ref):
        assert torch.equal(a, b), n
    check_outputs(host(dict(zip(names, got))), host(dict(zip(names, ref))), "bf16", where="noalloc")


def test_noalloc_backward_equals_workspace_backward_twice():
    require_gpu()
    announce("noalloc: L=2048 B=64 then L=512 B=32")
    w1, x1, f1 = _full_case(2048, 64, 8, 2, 128, 31)
    _compare(w1, x1, f1)
    w2, x2, f2 = _full_case(512, 32, 4, 1, 64, 32)       # smaller: the array holds the first call's values
    _compare(w2, x2, f2)


def test_noalloc_share_mode_and_size_limit():
    require_gpu()
    announce("noalloc: share mode and the size limit")
    L, B, n, C = 2048, 128, 4, 512
    w = Workload(name="noalloc_share", batch=1, seqlen=L, block=B, hq=4, hkv=2, head_dim=128, dtype="bf16",
                 seed=33, q_std=128 ** -0.5, share_blocks=n, share_chunk=C)
    x = make_share_inputs(w, device="cuda", sharp=True)
    ids = [int(i) for i in x["block_ids"]]
    o, lse = M.share_fwd(x["qx"], x["kx"], x["vx"], x["kc"], x["vc"], ids, B, 0, L, 1, w.scale)
    o = o.to(x["qx"].dtype)
    desc = api.desc_for(x["qx"], x["kc"], B, w.scale, block_ids=ids, kv_begin=0, kv_end=L, own_block=1)
    outs = []
    for noalloc in (False, True):
        dq = torch.zeros(x["qx"].shape, dtype=torch.float32, device="cuda")
        dkc, dvc = torch.zeros_like(x["kc"]), torch.zeros_like(x["vc"])
        dkx, dvx = torch.empty_like(x["kx"]), torch.empty_like(x["vx"])
        args = (desc, None, x["kc"], x["vc"], x["qx"], x["kx"], x["vx"], None, o, None, lse, None, x["dox"],
                None, dkc, dvc, dq, dkx, dvx)
        if noalloc:
            api.bdlm_attn_bwd_noalloc(*args)
        else:
            api.bdlm_attn_bwd(*args, api.workspace(desc, True, "cuda"))
        outs.append((dq, dkc, dvc, dkx, dvx))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    # a workspace larger than the array is refused before anything is enqueued
    lib = M.load()
    big = make_desc(1, 262144, 1024, 32, 8, 128, 1, 128 ** -0.5)
    assert lib.bdlm_attn_workspace_bytes(ctypes.byref(big), 1) > lib.bdlm_attn_noalloc_scratch_bytes()
    p = ctypes.c_void_p(4096)
    assert lib.bdlm_attn_bwd_noalloc(ctypes.byref(big), *([p] * 18), None) == 2
