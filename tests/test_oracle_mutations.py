"""The pins must be able to fail: plant plausible mistakes in the oracle (on
the CPU, via monkeypatching) and check that some pin catches each one."""

import numpy as np
import pytest

import oracle
import oracle.attention as oa
import tests.test_oracle_pins as pins


def _wrong_visible_offset(q_pos, nk, causal, window, offset=0):
    return _ORIG_VISIBLE(q_pos, nk, causal, window, offset=0)  # forgets bottom-right alignment


def _wrong_window(q_pos, nk, causal, window, offset=0):
    return _ORIG_VISIBLE(q_pos, nk, causal, window + 1 if window else 0, offset)  # off by one


def _no_scale_scores(q, k, scale, causal, window, q_pos, nq):
    return _ORIG_SCORES(q, k, 1.0, causal, window, q_pos, nq)


def _transposed_bwd(q, k, v, dout, scale, causal=False, window=0):
    dq, dk, dv = _ORIG_BWD(q, k, v, dout, scale, causal, window)
    return dq, dk, dv[::-1].copy()  # rows of dV in the wrong order


def _bwd_drops_d(q, k, v, dout, scale, causal=False, window=0):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    p = oa.attention_probs(q, k, scale, causal, window)
    ds = p * (do @ v.T)  # dP - D with the D term dropped
    return scale * ds @ k, scale * ds.T @ q, p.T @ do


_ORIG_VISIBLE = oa.visible
_ORIG_SCORES = oa._scores
_ORIG_BWD = oa.attention_bwd


def _blocked_no_rescale(q, k, v, scale, causal=False, window=0, br=16, bc=16):
    """The per-block softmax of jsqmd.com 2.2.1 taken literally: no alpha."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for r0 in range(0, nq, br):
        rows = np.arange(r0, min(r0 + br, nq))
        acc = np.zeros((rows.size, v.shape[1]))
        l = np.zeros(rows.size)
        for c0 in range(0, nk, bc):
            cols = np.arange(c0, min(c0 + bc, nk))
            ok = oa.visible(rows, nk, causal, window, offset=nk - nq)[:, cols]
            s = np.where(ok, scale * q[rows] @ k[cols].T, -np.inf)
            m = np.where(np.isfinite(s.max(1)), s.max(1), 0)
            pt = np.exp(s - m[:, None])
            acc += pt @ v[cols]
            l += pt.sum(1)
        o[rows] = acc / np.maximum(l, 1e-300)[:, None]
    return o, lse


def _merge_unnormalised(o_parts, lse_parts):
    o = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    m = lse.max(axis=0)
    w = np.exp(lse - m[None])
    return (w[..., None] * o).sum(axis=0), m + np.log(w.sum(axis=0))  # weights not divided by their sum


def _merge_lse_without_max(o_parts, lse_parts):
    o, _ = _ORIG_MERGE(o_parts, lse_parts)
    lse = np.asarray(lse_parts, dtype=np.float64)
    return o, np.log(np.exp(lse - lse.max(axis=0)[None]).sum(axis=0))  # the max is not added back


def _kvcache_forgets_new_keys(q, k_cache, v_cache, cache_seqlens, scale, causal=False, window=0, k_new=None,
                              v_new=None):
    # appends, but attends over the old length only
    o, lse, kc, vc = _ORIG_KVCACHE(q, k_cache, v_cache, cache_seqlens, scale, causal, window, k_new, v_new)
    o2, lse2, _, _ = _ORIG_KVCACHE(q, kc, vc, np.maximum(np.asarray(cache_seqlens), 1), scale, causal, window)
    return o2, lse2, kc, vc


def _paged_gather_swaps_index(blocks, block_table, page):
    blocks = np.asarray(blocks)
    table = np.asarray(block_table, dtype=np.int64)
    b_, mb = table.shape
    out = np.empty((b_, mb * page) + blocks.shape[2:], dtype=blocks.dtype)
    for b in range(b_):
        for j in range(mb * page):
            out[b, j] = blocks[table[b, j % mb], j // mb]  # page and row index confused
    return out


def _philox_no_key_bump(counter, key, rounds=10):
    m32 = np.uint64(0xFFFFFFFF)
    c = np.asarray(counter, dtype=np.uint64) & m32
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = np.uint64(int(key[0])), np.uint64(int(key[1]))
    for _ in range(rounds):  # the key schedule is forgotten
        p0 = np.uint64(0xD2511F53) * c0
        p1 = np.uint64(0xCD9E8D57) * c2
        c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & m32, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & m32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def _bwd_mask_only_in_dv(q, k, v, dout, scale, causal=False, window=0, drop=None):
    dq, dk, dv = _ORIG_BWD(q, k, v, dout, scale, causal, window, drop=None)  # dP, D without the mask
    if drop is not None:
        p = oa.attention_probs(q, k, scale, causal, window)
        dv = (p * drop[0] * drop[1]).T @ np.asarray(dout, dtype=np.float64)
    return dq, dk, dv


_ORIG_DROPOUT_INDEX = oa.dropout_index


def _dropout_index_shares_bytes(slot, q_rows, nk, offset):
    """Word (j mod 16) div 4 instead of (j mod 32) div 8: keys j and j + 16 of
    the first half of every 32-key block then draw the same byte, which leaves
    every marginal statistic of the bytes intact."""
    ctr, word, byte = _ORIG_DROPOUT_INDEX(slot, q_rows, nk, offset)
    j = np.arange(nk)
    return ctr, np.broadcast_to((j % 16) // 4, word.shape), byte


_ORIG_MERGE = oa.merge_partials
_ORIG_KVCACHE = oa.kvcache_fwd

MUTATIONS = [
    ("visible", _wrong_visible_offset, lambda: pins.test_forward_matches_torch_sdpa(17, 29, True, 0)),
    ("visible", _wrong_window, lambda: pins.test_scale_zero_is_mean_over_visible_keys(True, 4)),
    ("_scores", _no_scale_scores, lambda: pins.test_single_key()),
    ("attention_bwd", _transposed_bwd, lambda: pins.test_backward_matches_torch_autograd(True, 0)),
    ("attention_bwd", _bwd_drops_d, lambda: pins.test_backward_identities(True, 0)),
    ("blocked_fwd", _blocked_no_rescale,
     lambda: pins.test_blocked_online_softmax_equals_direct(37, 8, 5, False, 0)),
    ("merge_partials", _merge_unnormalised, lambda: pins.test_merge_closed_forms()),
    ("merge_partials", _merge_lse_without_max,
     lambda: pins.test_merge_of_key_chunks_equals_full_attention(False, 0, [0, 7, 19, 40])),
    ("philox4x32", _philox_no_key_bump, lambda: pins.test_philox_known_answers()),
    ("attention_bwd", _bwd_mask_only_in_dv, lambda: pins.test_dropout_backward_finite_differences(True, 0)),
    ("dropout_index", _dropout_index_shares_bytes, lambda: pins.test_dropout_map_is_injective()),
    ("dropout_index", _dropout_index_shares_bytes, lambda: pins.test_dropout_bytes_pairwise_independent()),
    ("dropout_index", _dropout_index_shares_bytes, lambda: pins.test_dropout_bytes_map_and_uniformity()),
    ("paged_gather", _paged_gather_swaps_index, lambda: pins.test_paged_kvcache_equals_contiguous(4)),
    ("kvcache_fwd", _kvcache_forgets_new_keys,
     lambda: pins.test_kvcache_decode_equals_rows_of_the_full_sequence(1, True, 0)),
]


@pytest.mark.parametrize("attr,mutant,pin", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, attr, mutant, pin):
    monkeypatch.setattr(oa, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant, raising=False)
    with pytest.raises(AssertionError):
        pin()
