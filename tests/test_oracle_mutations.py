"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check
that at least one pin fails for each: the pins are not vacuous."""
import numpy as np
import pytest

from oracle import bdlm_oracle as O
import tests.test_oracle_pins as P


def _mask_lt(q_stream, q_block, k_stream, k_block):       # clean sees only strictly earlier blocks
    cc = (q_stream == 0) & (k_stream == 0) & (k_block < q_block)
    xc = (q_stream == 1) & (k_stream == 0) & (k_block < q_block)
    xx = (q_stream == 1) & (k_stream == 1) & (k_block == q_block)
    return cc | xc | xx


def _mask_noisy_own_clean(q_stream, q_block, k_stream, k_block):   # corrupted sees its own clean block
    cc = (q_stream == 0) & (k_stream == 0) & (k_block <= q_block)
    xc = (q_stream == 1) & (k_stream == 0) & (k_block <= q_block)
    xx = (q_stream == 1) & (k_stream == 1) & (k_block == q_block)
    return cc | xc | xx


def _bwd_no_delta(q, k, v, p, o, do, scale, delta=None):
    dp = do @ v.T
    ds = p * dp
    return scale * (ds @ k), scale * (ds.T @ q), p.T @ do


def _bwd_dk_unscaled(q, k, v, p, o, do, scale, delta=None):
    d_row = (do * o).sum(axis=1) if delta is None else delta
    ds = p * (do @ v.T - d_row[:, None])
    return scale * (ds @ k), ds.T @ q, p.T @ do


def _bwd_dv_transposed(q, k, v, p, o, do, scale, delta=None):
    d_row = (do * o).sum(axis=1) if delta is None else delta
    ds = p * (do @ v.T - d_row[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), (p.T @ do)[::-1]


def _kv_head_mod(h, hq, hkv):
    return h % hkv


def _merge_no_weights(o_parts, lse_parts):
    lse = np.stack(lse_parts)
    m = lse.max(axis=0)
    o = sum(o_parts) / len(o_parts)
    return o, m


def _fwd_lse_log2(q, k, v, mask, scale):
    o, lse, p = _ORIG_FWD(q, k, v, mask, scale)
    return o, lse / np.log(2.0), p


_ORIG_FWD = O.attention_fwd
_ORIG_SHARE_BWD = O.share_bwd


def _share_bwd_own_swapped(*a, **k):          # own-block dK and dV exchanged
    dq, dkc, dvc, dkx, dvx = _ORIG_SHARE_BWD(*a, **k)
    return dq, dkc, dvc, dvx, dkx


def _share_bwd_own_rows_rolled(*a, **k):      # own-block rows written one block off
    dq, dkc, dvc, dkx, dvx = _ORIG_SHARE_BWD(*a, **k)
    B = a[6]
    return dq, dkc, dvc, np.roll(dkx, B, axis=1), np.roll(dvx, B, axis=1)


def _share_bwd_window_dk_unscaled(*a, **k):   # clean-window dK missing the softmax scale
    dq, dkc, dvc, dkx, dvx = _ORIG_SHARE_BWD(*a, **k)
    return dq, dkc / a[13], dvc, dkx, dvx

MUTATIONS = [
    ("_visible", _mask_lt, [P.test_mask_matches_hand_written_fixture, ("mask_L4_B2.txt", 4, 2)]),
    ("_visible", _mask_noisy_own_clean, [P.test_visible_pair_count_closed_form, (8, 2)]),
    ("attention_bwd", _bwd_no_delta, [P.test_backward_matches_central_finite_differences]),
    ("attention_bwd", _bwd_dk_unscaled, [P.test_backward_equals_sdpa_autograd, (16, 4, 4, 2, 8)]),
    ("attention_bwd", _bwd_dv_transposed, [P.test_backward_equals_sdpa_autograd, (20, 5, 2, 2, 6)]),
    ("kv_head_of", _kv_head_mod, [P.test_forward_equals_sdpa_with_explicit_mask, (24, 8, 4, 2, 16)]),
    ("kv_head_of", _kv_head_mod, [P.test_backward_equals_sdpa_autograd, (16, 4, 4, 2, 8)]),
    ("merge_partials", _merge_no_weights, [P.test_chunked_prefix_merge_equals_single_pass, (16,)]),
    ("attention_fwd", _fwd_lse_log2, [P.test_zero_query_closed_form]),
    ("share_bwd", _share_bwd_own_swapped, [P.test_share_backward_own_block_equals_full_problem, (16,)]),
    ("share_bwd", _share_bwd_own_rows_rolled, [P.test_share_backward_own_block_equals_full_problem, (64,)]),
    ("share_bwd", _share_bwd_window_dk_unscaled, [P.test_share_backward_own_block_equals_full_problem, (16,)]),
]


@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_planted_mistake_is_caught(i, monkeypatch):
    name, fn, (check, *args) = MUTATIONS[i]
    monkeypatch.setattr(O, name, fn)
    with pytest.raises(AssertionError):
        check(*(args[0] if args else ()))
