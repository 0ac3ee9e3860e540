"""Property test of the oracle over small random shapes: the explicit-mask form
equals torch SDPA with the same mask (library routine) and the block-separated
form (BP exactness)."""
import numpy as np
import torch
from hypothesis import given, settings, strategies as st

from oracle import bdlm_oracle as O


@settings(max_examples=25, deadline=None)
@given(n=st.integers(1, 4), B=st.integers(1, 5), rep=st.integers(1, 3), hkv=st.integers(1, 2),
       d=st.integers(1, 6), seed=st.integers(0, 2**31 - 1))
def test_small_shapes(n, B, rep, hkv, d, seed):
    L, hq = n * B, rep * hkv
    rng = np.random.default_rng(seed)
    qc, qx, doc, dox = (rng.standard_normal((1, L, hq, d)) for _ in range(4))
    kc, kx, vc, vx = (rng.standard_normal((1, L, hkv, d)) for _ in range(4))
    a = O.bdlm_fwd_bwd(qc, kc, vc, qx, kx, vx, doc, dox, B, 0.8)
    b = O.bdlm_fwd_bwd_per_block(qc, kc, vc, qx, kx, vx, doc, dox, B, 0.8)
    for k in a:
        np.testing.assert_allclose(a[k], b[k], atol=1e-12, err_msg=k)
    m = torch.tensor(O.bdlm_mask(L, B))
    q = torch.tensor(np.concatenate([qc, qx], 1)[0].transpose(1, 0, 2))
    k = torch.tensor(np.concatenate([kc, kx], 1)[0].transpose(1, 0, 2)).repeat_interleave(rep, 0)
    v = torch.tensor(np.concatenate([vc, vx], 1)[0].transpose(1, 0, 2)).repeat_interleave(rep, 0)
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=m,
                                                         scale=0.8)[0].numpy().transpose(1, 0, 2)
    np.testing.assert_allclose(np.concatenate([a["oc"][0], a["ox"][0]]), o, atol=1e-12)
