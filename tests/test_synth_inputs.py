"""Host checks of the seeded input generators (no attention arithmetic here)."""
import numpy as np
import torch

from synth import WORKLOADS, draw_block_positions, draw_units, make_full_inputs, make_share_inputs


def test_full_inputs_deterministic_and_shaped():
    w = WORKLOADS["tiny_f32"]
    a = make_full_inputs(w)
    b = make_full_inputs(w)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["qc"].shape == (1, 256, 2, 64) and a["qc"].dtype == torch.float32
    assert abs(float(a["qc"].std()) - 1 / 8) < 0.01


def test_bf16_cast_and_outlier_rows():
    w = WORKLOADS["gqa_64k"]
    x = make_full_inputs(w, seqlen=1024, block=64)
    assert x["kc"].dtype == torch.bfloat16
    norms = torch.cat([x["kc"], x["kx"]], 1).float().reshape(-1, 128).norm(dim=1)
    big = int((norms > 4.0).sum())        # unit-std rows have norm ~1, outliers ~8
    assert big == round(0.01 * 2 * 1024 * 8)


def test_block_positions_and_units():
    ids = draw_block_positions(256, 16, 4)
    assert len(set(ids.tolist())) == 16 and (np.diff(ids) > 0).all() and ids.max() < 256
    u = draw_units(512, 32, 1, 64, 3)
    assert u.shape == (64, 4) and len({tuple(r) for r in u.tolist()}) == 64
    firsts = {(int(s), int(b)) for _, s, b, _ in u[:4]}
    assert firsts == {(0, 0), (0, 511), (1, 0), (1, 511)}


def test_share_inputs():
    w = WORKLOADS["csbp_share_256k"]
    x = make_share_inputs(w, seqlen=8192, nlocal=4, block=256)
    assert x["qx"].shape == (1, 1024, 32, 128) and x["kc"].shape == (1, 8192, 8, 128)
    assert len(x["block_ids"]) == 4


def test_clean_shard_ids_zigzag_is_balanced_and_partitions():
    from synth import clean_shard_ids
    nb, nr = 256, 16
    shards = [clean_shard_ids(nb, nr, r) for r in range(nr)]
    allb = np.sort(np.concatenate(shards))
    np.testing.assert_array_equal(allb, np.arange(nb))        # a partition of the blocks
    work = [int((s + 1).sum()) for s in shards]                 # block b sees b + 1 clean blocks
    assert len(set(work)) == 1
    assert list(shards[0][:3]) == [0, 1, 2] and shards[0][-1] == nb - 1


def test_rank_share_inputs_include_the_clean_shard():
    w = WORKLOADS["csbp_rank_256k"]
    x = make_share_inputs(w, seqlen=65536, nlocal=4)       # 64 blocks over 16 ranks: 4 each
    assert x["qs"].shape == (1, 4 * w.block, w.hq, w.head_dim) and x["qs"].dtype == torch.bfloat16
    assert x["dos"].shape == x["qs"].shape
    assert list(x["clean_ids"]) == [0, 1, 62, 63]
