"""Pins of the CPU oracle against things other than itself (no GPU).

Each test ties an oracle function to a closed form, a hand-derived value, an
invariant, finite differences or an independent library routine (torch's CPU
attention and autograd), chosen so that a plausible mistake in the oracle --
a dropped scale, a wrong mask sign or offset, a transposed operand, a missing
rescale in the blocked recurrence, a wrong gradient term -- fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
_EXPR_ENV = {"log": math.log, "sqrt": math.sqrt}


def _ev(x):
    if isinstance(x, list):
        return np.array([_ev(e) for e in x], dtype=np.float64)
    return float(eval(x, {"__builtins__": {}}, _EXPR_ENV))  # fixture expressions only


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# hand-derived worked examples (tests/golden/hand_examples.json)
# --------------------------------------------------------------------------
def _golden_cases():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_forward(case):
    q, k, v = _ev(case["q"]), _ev(case["k"]), _ev(case["v"])
    o, lse = oracle.attention_fwd(q, k, v, _ev(case["scale"]), case["causal"], case["window"])
    np.testing.assert_allclose(o, _ev(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _ev(case["lse"]), rtol=0, atol=1e-12)
    ob, lseb = oracle.blocked_fwd(q, k, v, _ev(case["scale"]), case["causal"], case["window"], br=1, bc=1)
    np.testing.assert_allclose(ob, _ev(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lseb, _ev(case["lse"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", [c for c in _golden_cases() if "dq" in c], ids=lambda c: c["name"])
def test_golden_backward(case):
    q, k, v, do = _ev(case["q"]), _ev(case["k"]), _ev(case["v"]), _ev(case["dout"])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, _ev(case["scale"]), case["causal"], case["window"])
    np.testing.assert_allclose(dq, _ev(case["dq"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, _ev(case["dk"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, _ev(case["dv"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------
MASKS = [(False, 0), (True, 0), (True, 5), (False, 4)]


@pytest.mark.parametrize("causal,window", MASKS)
def test_rows_sum_to_one(causal, window):
    rng = np.random.default_rng(1)
    q, k = _rand(rng, 23, 16), _rand(rng, 23, 16)
    p = oracle.attention_probs(q, k, 0.3, causal, window)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-14)
    assert (p >= 0).all()


@pytest.mark.parametrize("causal,window", MASKS)
def test_constant_v_returns_v(causal, window):
    rng = np.random.default_rng(2)
    q, k = _rand(rng, 19, 8), _rand(rng, 19, 8)
    row = _rand(rng, 8)
    v = np.tile(row, (19, 1))
    o, _ = oracle.attention_fwd(q, k, v, 0.5, causal, window)
    np.testing.assert_allclose(o, np.tile(row, (19, 1)), atol=1e-13)


def test_single_key():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 7, 8), _rand(rng, 1, 8), _rand(rng, 1, 5)
    o, lse = oracle.attention_fwd(q, k, v, 0.7)
    np.testing.assert_allclose(o, np.tile(v[0], (7, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * (q @ k[0]), atol=1e-13)


@pytest.mark.parametrize("window", [0, 3])
def test_causal_row0_is_v0(window):
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 9, 8), _rand(rng, 9, 8), _rand(rng, 9, 6)
    o, lse = oracle.attention_fwd(q, k, v, 0.4, True, window)
    assert np.array_equal(o[0], v[0])
    np.testing.assert_allclose(lse[0], 0.4 * q[0] @ k[0], atol=1e-14)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 4), (False, 3), (False, 0)])
def test_scale_zero_is_mean_over_visible_keys(causal, window):
    """scale = 0: uniform weights over the visible keys -> cumulative/windowed mean."""
    rng = np.random.default_rng(5)
    n = 13
    q, k, v = _rand(rng, n, 4), _rand(rng, n, 4), _rand(rng, n, 3)
    o, lse = oracle.attention_fwd(q, k, v, 0.0, causal, window)
    for i in range(n):
        lo = max(0, i - window + 1) if window > 0 else 0
        hi = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v[lo:hi].mean(axis=0), atol=1e-14)
        assert lse[i] == pytest.approx(math.log(hi - lo), abs=1e-14)


def test_shift_invariance_large_offset():
    """Adding the same vector u to every key shifts each row's logits by a
    constant, which softmax ignores; a huge u exercises the max subtraction."""
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 11, 8), _rand(rng, 11, 8), _rand(rng, 11, 8)
    u = 300.0 * _rand(rng, 8)
    for causal, window in MASKS:
        o1, lse1 = oracle.attention_fwd(q, k, v, 0.9, causal, window)
        o2, lse2 = oracle.attention_fwd(q, k + u, v, 0.9, causal, window)
        assert np.isfinite(o2).all()
        np.testing.assert_allclose(o2, o1, atol=1e-10)
        np.testing.assert_allclose(lse2 - lse1, 0.9 * q @ u, atol=1e-9)


def test_fully_masked_row_zero_and_neg_inf():
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 4, 4), _rand(rng, 2, 4), _rand(rng, 2, 4)
    # causal, Nq=4 > Nk=2: bottom-right alignment -> rows 0,1 see nothing
    o, lse = oracle.attention_fwd(q, k, v, 1.0, True, 0)
    assert (o[:2] == 0).all() and np.isneginf(lse[:2]).all()
    assert np.isfinite(o[2:]).all()
    ob, lseb = oracle.blocked_fwd(q, k, v, 1.0, True, 0, br=3, bc=1)
    np.testing.assert_allclose(ob, o, atol=1e-14)
    assert np.isneginf(lseb[:2]).all()


@pytest.mark.parametrize("n,br,bc,causal,window", [
    (37, 8, 5, False, 0), (37, 8, 5, True, 0), (64, 16, 16, True, 0), (64, 8, 16, True, 9),
    (37, 5, 8, True, 6), (50, 7, 3, False, 11), (1, 4, 4, True, 0),
])
def test_blocked_online_softmax_equals_direct(n, br, bc, causal, window):
    rng = np.random.default_rng(8 + n + br)
    q, k, v = 2 * _rand(rng, n, 16), 2 * _rand(rng, n, 16), _rand(rng, n, 12)
    o, lse = oracle.attention_fwd(q, k, v, 0.25, causal, window)
    ob, lseb = oracle.blocked_fwd(q, k, v, 0.25, causal, window, br=br, bc=bc)
    np.testing.assert_allclose(ob, o, atol=1e-13)
    np.testing.assert_allclose(lseb, lse, atol=1e-13)


def test_sampled_rows_match_full():
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 30, 8), _rand(rng, 30, 8), _rand(rng, 30, 8)
    o, lse = oracle.attention_fwd(q, k, v, 0.3, True, 7)
    idx = np.array([0, 5, 17, 29])
    os_, ls_ = oracle.attention_fwd(q[idx], k, v, 0.3, True, 7, q_pos=idx, nq=30)
    np.testing.assert_allclose(os_, o[idx], atol=1e-15)
    np.testing.assert_allclose(ls_, lse[idx], atol=1e-15)


# --------------------------------------------------------------------------
# torch's CPU attention routine and autograd as an independent reference
# --------------------------------------------------------------------------
def _torch_mask(nq, nk, causal, window):
    i = torch.arange(nq)[:, None] + (nk - nq)
    j = torch.arange(nk)[None, :]
    ok = torch.ones(nq, nk, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window > 0:
        ok &= j > i - window
    return ok


@pytest.mark.parametrize("nq,nk,causal,window", [
    (33, 33, False, 0), (33, 33, True, 0), (40, 40, True, 8), (17, 29, True, 0), (16, 48, True, 5),
])
def test_forward_matches_torch_sdpa(nq, nk, causal, window):
    g = torch.Generator().manual_seed(nq * 7 + nk)
    q = torch.randn(nq, 16, generator=g, dtype=torch.float64)
    k = torch.randn(nk, 16, generator=g, dtype=torch.float64)
    v = torch.randn(nk, 10, generator=g, dtype=torch.float64)
    mask = _torch_mask(nq, nk, causal, window)
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None], scale=0.35)[0]
    o, lse = oracle.attention_fwd(q.numpy(), k.numpy(), v.numpy(), 0.35, causal, window)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    s = (0.35 * q @ k.T).masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 6)])
def test_backward_matches_torch_autograd(causal, window):
    g = torch.Generator().manual_seed(11)
    n, d = 21, 8
    q = torch.randn(n, d, generator=g, dtype=torch.float64, requires_grad=True)
    k = torch.randn(n, d, generator=g, dtype=torch.float64, requires_grad=True)
    v = torch.randn(n, d, generator=g, dtype=torch.float64, requires_grad=True)
    do = torch.randn(n, d, generator=g, dtype=torch.float64)
    mask = _torch_mask(n, n, causal, window)
    out = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None], scale=0.6)[0]
    out.backward(do)
    dq, dk, dv = oracle.attention_bwd(q.detach().numpy(), k.detach().numpy(), v.detach().numpy(),
                                      do.numpy(), 0.6, causal, window)
    np.testing.assert_allclose(dq, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, v.grad.numpy(), atol=1e-12)


def test_mha_layout_matches_torch_bhnd():
    """mha_fwd takes [B, N, H, d]; torch's routine takes [B, H, N, d]."""
    g = torch.Generator().manual_seed(12)
    q = torch.randn(2, 24, 3, 8, generator=g, dtype=torch.float64)
    k = torch.randn(2, 24, 3, 8, generator=g, dtype=torch.float64)
    v = torch.randn(2, 24, 3, 8, generator=g, dtype=torch.float64)
    ref = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                         is_causal=True, scale=0.5).transpose(1, 2)
    o, lse = oracle.mha_fwd(q.numpy(), k.numpy(), v.numpy(), 0.5, causal=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    assert lse.shape == (2, 3, 24)


def test_varlen_matches_block_diagonal_sdpa():
    """Packed sequences attend only within themselves: the same as one long
    sequence under a block-diagonal (and causal, windowed) mask."""
    lengths = [5, 1, 12, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    total = int(cu[-1])
    g = torch.Generator().manual_seed(13)
    q = torch.randn(total, 2, 8, generator=g, dtype=torch.float64)
    k = torch.randn(total, 2, 8, generator=g, dtype=torch.float64)
    v = torch.randn(total, 2, 8, generator=g, dtype=torch.float64)
    seg = torch.repeat_interleave(torch.arange(len(lengths)), torch.tensor(lengths))
    pos = torch.arange(total) - torch.tensor(cu[:-1])[seg]
    window = 4
    same = seg[:, None] == seg[None, :]
    causal = pos[None, :] <= pos[:, None]
    win = pos[None, :] > pos[:, None] - window
    mask = same & causal & win
    ref = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                         attn_mask=mask[None], scale=0.4).transpose(0, 1)
    o, lse = oracle.varlen_fwd(q.numpy(), k.numpy(), v.numpy(), cu, 0.4, True, window)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    assert lse.shape == (2, total)


# --------------------------------------------------------------------------
# backward: finite differences and identities
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 3)])
def test_backward_finite_differences(causal, window):
    rng = np.random.default_rng(14)
    n, d, scale, h = 6, 4, 0.7, 1e-6
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))

    def loss(qq, kk, vv):
        o, _ = oracle.attention_fwd(qq, kk, vv, scale, causal, window)
        return float((do * o).sum())

    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal, window)
    for which, g in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += h
            minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 2), (False, 0)])
def test_varlen_backward_finite_differences(causal, window):
    """Packed-sequence gradients against central differences of the packed
    forward: the loss L = sum(dO * O) runs through varlen_fwd, so a mistake
    in the per-sequence offsets, the masks or cross-sequence leakage shows."""
    rng = np.random.default_rng(17)
    cu = np.array([0, 3, 7, 8])  # lengths 3, 4, 1
    total, heads, d, scale, h = 8, 2, 3, 0.8, 1e-6
    q, k, v, do = (_rand(rng, total, heads, d) for _ in range(4))

    def loss(qq, kk, vv):
        o, _ = oracle.varlen_fwd(qq, kk, vv, cu, scale, causal, window)
        return float((do * o).sum())

    grads = oracle.varlen_bwd(q, k, v, do, cu, scale, causal, window)
    for which, g in enumerate(grads):
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += h
            minus[which][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 5)])
def test_backward_identities(causal, window):
    rng = np.random.default_rng(15)
    n, d = 17, 8
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, causal, window)
    # each softmax-Jacobian row sums to zero -> sum over keys of dK vanishes
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # every row of P sums to one -> sum over keys of dV equals sum over queries of dO
    np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # D_i = rowsum(dO * O) = sum_j P_ij dP_ij
    p = oracle.attention_probs(q, k, 0.5, causal, window)
    o, _ = oracle.attention_fwd(q, k, v, 0.5, causal, window)
    np.testing.assert_allclose((do * o).sum(1), (p * (do @ v.T)).sum(1), atol=1e-12)


def test_mha_bwd_layout():
    rng = np.random.default_rng(16)
    q, k, v, do = (_rand(rng, 1, 9, 2, 4) for _ in range(4))
    dq, dk, dv = oracle.mha_bwd(q, k, v, do, 0.5, causal=True)
    for h in range(2):
        r = oracle.attention_bwd(q[0, :, h], k[0, :, h], v[0, :, h], do[0, :, h], 0.5, True)
        np.testing.assert_allclose(dq[0, :, h], r[0], atol=0)
        np.testing.assert_allclose(dk[0, :, h], r[1], atol=0)
        np.testing.assert_allclose(dv[0, :, h], r[2], atol=0)


# --------------------------------------------------------------------------
# fp8 e4m3 decoding (OCP definition) vs torch's float8_e4m3fn
# --------------------------------------------------------------------------
def test_e4m3_decode_known_values():
    assert oracle.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert oracle.e4m3_decode(np.uint8(0xFE)) == -448.0
    assert oracle.e4m3_decode(np.uint8(0x38)) == 1.0
    assert oracle.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6
    assert oracle.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9
    assert oracle.e4m3_decode(np.uint8(0x00)) == 0.0
    assert np.isnan(oracle.e4m3_decode(np.uint8(0x7F)))
    assert np.isnan(oracle.e4m3_decode(np.uint8(0xFF)))


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert (both_nan | (ref == got)).all()


def test_fp8_dequant():
    codes = np.array([0x38, 0x40, 0xB8], dtype=np.uint8)  # 1, 2, -1
    np.testing.assert_array_equal(oracle.fp8_dequant(codes, 0.5), [0.5, 1.0, -0.5])


# --------------------------------------------------------------------------
# merge of partial (O, LSE) results
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal,window,cuts", [
    (False, 0, [0, 7, 19, 40]), (True, 0, [0, 13, 14, 40]), (True, 6, [0, 5, 22, 31, 40]), (False, 0, [0, 40]),
])
def test_merge_of_key_chunks_equals_full_attention(causal, window, cuts):
    """Attention over contiguous key chunks, each computed by torch's CPU routine
    (with torch.logsumexp for its LSE), merged by the oracle, equals torch's
    attention over all keys.  Chunks that a row cannot see give LSE = -inf."""
    g = torch.Generator().manual_seed(len(cuts) * 31 + window)
    n, d = 40, 12
    q = torch.randn(n, d, generator=g, dtype=torch.float64)
    k = torch.randn(n, d, generator=g, dtype=torch.float64)
    v = torch.randn(n, 9, generator=g, dtype=torch.float64)
    mask = _torch_mask(n, n, causal, window)
    s = (0.4 * q @ k.T).masked_fill(~mask, float("-inf"))
    o_parts, lse_parts = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        lse_p = torch.logsumexp(s[:, a:b], dim=1)
        p = torch.softmax(s[:, a:b], dim=1).nan_to_num(0.0)  # rows that see none of these keys: 0
        o_parts.append((p @ v[a:b]).numpy())
        lse_parts.append(lse_p.numpy())
    o, lse = oracle.merge_partials(np.stack(o_parts), np.stack(lse_parts))
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None], scale=0.4)[0]
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


def test_merge_closed_forms():
    rng = np.random.default_rng(5)
    o1 = rng.standard_normal((3, 4, 6))
    l1 = rng.standard_normal((3, 4))
    # one part: identity
    o, lse = oracle.merge_partials(o1[None], l1[None])
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1, atol=1e-15)
    # two equal parts: the same O, LSE + ln 2
    o, lse = oracle.merge_partials(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(o, o1, atol=1e-14)
    np.testing.assert_allclose(lse, l1 + math.log(2), atol=1e-14)
    # weights exp(LSE_p - LSE): with LSEs ln 1 and ln 3, O = (O_1 + 3 O_2) / 4, LSE = ln 4
    o2 = rng.standard_normal((3, 4, 6))
    o, lse = oracle.merge_partials(np.stack([o1, o2]), np.stack([np.zeros((3, 4)), np.full((3, 4), math.log(3))]))
    np.testing.assert_allclose(o, (o1 + 3 * o2) / 4, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(4), atol=1e-14)
    # a part with LSE = -inf adds nothing, whatever its O holds; all -inf gives 0 and -inf
    junk = np.full_like(o1, 1e300)
    o, lse = oracle.merge_partials(np.stack([o1, junk]), np.stack([l1, np.full((3, 4), -np.inf)]))
    np.testing.assert_allclose(o, o1, atol=1e-15)
    np.testing.assert_allclose(lse, l1, atol=1e-15)
    o, lse = oracle.merge_partials(np.stack([junk, junk]), np.full((2, 3, 4), -np.inf))
    assert (o == 0).all() and np.isneginf(lse).all()
    # a common shift of every LSE_p leaves O alone and shifts LSE; no overflow at 1000
    o, lse = oracle.merge_partials(np.stack([o1, o2]), np.stack([l1 + 1000.0, l1 + 1000.0 + math.log(3)]))
    np.testing.assert_allclose(o, (o1 + 3 * o2) / 4, atol=1e-13)
    np.testing.assert_allclose(lse, l1 + 1000.0 + math.log(4), atol=1e-12)


# --------------------------------------------------------------------------
# KV-cache decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("nq,causal,window", [(1, True, 0), (3, True, 0), (2, True, 4), (1, False, 0)])
def test_kvcache_decode_equals_rows_of_the_full_sequence(nq, causal, window):
    """Decoding the last nq tokens of a sequence against a cache holding the
    earlier ones (plus the appended new keys) gives the last nq rows of the
    full-sequence attention computed by torch's CPU routine.  Cache rows past
    the valid length hold NaN, so reading them would show."""
    g = torch.Generator().manual_seed(nq * 10 + window)
    lens = [9, 0, 17]  # tokens already cached per batch entry
    lmax, h, d = 24, 2, 8
    b_ = len(lens)
    x_q = torch.randn(b_, lmax, h, d, generator=g, dtype=torch.float64)
    x_k = torch.randn(b_, lmax, h, d, generator=g, dtype=torch.float64)
    x_v = torch.randn(b_, lmax, h, d, generator=g, dtype=torch.float64)
    k_cache = torch.full((b_, lmax, h, d), float("nan"), dtype=torch.float64)
    v_cache = torch.full((b_, lmax, h, d), float("nan"), dtype=torch.float64)
    q = torch.empty(b_, nq, h, d, dtype=torch.float64)
    k_new = torch.empty(b_, nq, h, d, dtype=torch.float64)
    v_new = torch.empty(b_, nq, h, d, dtype=torch.float64)
    for b, t in enumerate(lens):
        k_cache[b, :t], v_cache[b, :t] = x_k[b, :t], x_v[b, :t]
        q[b], k_new[b], v_new[b] = x_q[b, t:t + nq], x_k[b, t:t + nq], x_v[b, t:t + nq]
    o, lse, kc, vc = oracle.kvcache_fwd(q.numpy(), k_cache.numpy(), v_cache.numpy(), lens, 0.3, causal, window,
                                        k_new.numpy(), v_new.numpy())
    for b, t in enumerate(lens):
        n = t + nq
        np.testing.assert_array_equal(kc[b, :n], x_k[b, :n].numpy())
        np.testing.assert_array_equal(vc[b, :n], x_v[b, :n].numpy())
        assert np.isnan(kc[b, n:]).all()
        mask = _torch_mask(n, n, causal, window)
        for hh in range(h):
            ref = F.scaled_dot_product_attention(x_q[b, :n, hh][None], x_k[b, :n, hh][None], x_v[b, :n, hh][None],
                                                 attn_mask=mask[None], scale=0.3)[0]
            np.testing.assert_allclose(o[b, :, hh], ref[t:].numpy(), atol=1e-12)
            s = (0.3 * x_q[b, :n, hh] @ x_k[b, :n, hh].T).masked_fill(~mask, float("-inf"))
            np.testing.assert_allclose(lse[b, hh], torch.logsumexp(s, dim=1)[t:].numpy(), atol=1e-12)


def test_kvcache_without_new_keys_reads_the_first_seqlen_rows():
    """No new k, v: the queries attend over cache rows 0 .. seqlen-1 only, as
    the last nq positions of that key range; brute-force loops on a tiny case."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 2, 1, 3))
    kc = rng.standard_normal((1, 6, 1, 3))
    vc = rng.standard_normal((1, 6, 1, 3))
    kc[0, 4:], vc[0, 4:] = np.nan, np.nan
    o, lse, _, _ = oracle.kvcache_fwd(q, kc, vc, [4], 0.5, causal=True)
    for i in range(2):
        pos = 4 - 2 + i  # bottom-right: query i sits at key position i + Nk - Nq
        w = [math.exp(0.5 * sum(q[0, i, 0, c] * kc[0, j, 0, c] for c in range(3))) for j in range(pos + 1)]
        tot = sum(w)
        for c in range(3):
            assert abs(o[0, i, 0, c] - sum(w[j] * vc[0, j, 0, c] for j in range(pos + 1)) / tot) < 1e-12
        assert abs(lse[0, 0, i] - math.log(tot)) < 1e-12


@pytest.mark.parametrize("page", [1, 4, 8])
def test_paged_kvcache_equals_contiguous(page):
    """Pages filled by scattering a contiguous cache through a shuffled block
    table (written here, independently of the oracle's gather) give the
    contiguous decode's result, and the appended rows land in the pages the
    table names."""
    rng = np.random.default_rng(page)
    b_, h, d, nq, lmax = 3, 2, 4, 2, 24
    lens = [5, 0, 21]
    mb = lmax // page
    q = rng.standard_normal((b_, nq, h, d))
    kc = rng.standard_normal((b_, lmax, h, d))
    vc = rng.standard_normal((b_, lmax, h, d))
    kn = rng.standard_normal((b_, nq, h, d))
    vn = rng.standard_normal((b_, nq, h, d))
    table = rng.permutation(b_ * mb + 5)[:b_ * mb].reshape(b_, mb)  # 5 pages nobody uses
    kb = np.full((b_ * mb + 5, page, h, d), np.nan)
    vb = np.full((b_ * mb + 5, page, h, d), np.nan)
    for b in range(b_):
        for j in range(lmax):
            kb[table[b, j // page], j % page] = kc[b, j]
            vb[table[b, j // page], j % page] = vc[b, j]
    o, lse, kb2, vb2 = oracle.kvcache_paged_fwd(q, kb, vb, table, page, lens, 0.4, True, 0, kn, vn)
    ro, rl, rkc, _ = oracle.kvcache_fwd(q, kc, vc, lens, 0.4, True, 0, kn, vn)
    np.testing.assert_array_equal(o, ro)
    np.testing.assert_array_equal(lse, rl)
    for b, t in enumerate(lens):
        for i in range(nq):
            j = t + i
            np.testing.assert_array_equal(kb2[table[b, j // page], j % page], kn[b, i])
    unused = sorted(set(range(b_ * mb + 5)) - set(table.ravel().tolist()))
    assert np.isnan(kb2[unused]).all()


# --------------------------------------------------------------------------
# dropout: the counter-based generator and the dropped attention
# --------------------------------------------------------------------------
PHILOX_KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_kat.json")


def test_philox_known_answers():
    with open(PHILOX_KAT, encoding="utf-8") as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ctr = np.array([int(x, 16) for x in c["counter"]], dtype=np.uint64)
        key = [int(x, 16) for x in c["key"]]
        out = oracle.philox4x32(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in c["out"]]


def test_dropout_bytes_map_and_uniformity():
    """Each byte is the stated byte of the stated Philox word (checked element
    by element on a small block), and over 2^18 bytes every value is about
    equally frequent (chi-square, 255 degrees of freedom)."""
    seed, off, slot = 0x0123456789ABCDEF, 5, 9
    b = oracle.dropout_bytes(slot, [0, 1, 7, 40], 70, seed, off)
    for a, i in enumerate([0, 1, 7, 40]):
        for j in range(70):
            ctr = np.array([2 * (j // 32) + (j // 4) % 2, i, slot, off], dtype=np.uint64)
            w = oracle.philox4x32(ctr, (seed & 0xFFFFFFFF, seed >> 32))[(j % 32) // 8]
            assert b[a, j] == (int(w) >> (8 * (j % 4))) & 0xFF
    big = oracle.dropout_bytes(3, range(512), 512, 42, 0).ravel()
    counts = np.bincount(big, minlength=256)
    expect = big.size / 256
    chi2 = ((counts - expect) ** 2 / expect).sum()
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)


def test_dropout_map_is_injective():
    """No two elements share a random byte: over a 64 x 4096 block of two
    head slots and two offsets, every element has its own (counter, word,
    byte) triple."""
    rows = np.arange(64)
    seen = []
    for slot in (3, 4):
        for off in (1, 2):
            ctr, word, byte = oracle.dropout_index(slot, rows, 4096, off)
            assert ctr.shape == (64, 4096, 4) and word.shape == byte.shape == (64, 4096)
            assert ((0 <= word) & (word < 4)).all() and ((0 <= byte) & (byte < 4)).all()
            seen.append(np.concatenate([ctr.reshape(-1, 4), word.reshape(-1, 1), byte.reshape(-1, 1)], axis=1))
    triples = np.concatenate(seen).astype(np.uint64)
    assert np.unique(triples, axis=0).shape[0] == triples.shape[0]


def test_dropout_bytes_pairwise_independent():
    """Pairs of elements draw independent bytes: for every lag along the keys
    (1..63, which spans the 32-key blocks the map is built from) and along the
    rows (1..15), and between two head slots and two offsets, equal bytes occur
    at the rate 1/256 and the keep flags (p = 0.5) are uncorrelated, each
    within 5 sigma.  Two elements mapped to one byte would be equal always."""
    b = oracle.dropout_bytes(3, range(64), 4096, 0xFEEDF00D, 1).astype(np.int64)
    other = {"slot": oracle.dropout_bytes(4, range(64), 4096, 0xFEEDF00D, 1).astype(np.int64),
             "offset": oracle.dropout_bytes(3, range(64), 4096, 0xFEEDF00D, 2).astype(np.int64)}

    def check(x, y, what):
        n = x.size
        eq = (x == y).mean()
        sd = math.sqrt((1 / 256) * (255 / 256) / n)
        assert abs(eq - 1 / 256) < 5 * sd, f"{what}: equal-byte rate {eq:.5f}"
        kx, ky = (x < 128).astype(np.float64), (y < 128).astype(np.float64)
        corr = ((kx - kx.mean()) * (ky - ky.mean())).mean() / (kx.std() * ky.std())
        assert abs(corr) < 5 / math.sqrt(n), f"{what}: keep-flag correlation {corr:.4f}"

    for lag in range(1, 64):
        check(b[:, :-lag], b[:, lag:], f"key lag {lag}")
    for lag in range(1, 16):
        check(b[:-lag], b[lag:], f"row lag {lag}")
    for what, o in other.items():
        check(b, o, what)


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_dropout_keep_rate_and_scale(p):
    keep, s = oracle.dropout_keep(2, range(256), 1024, 7, 3, p)
    kthr = round(256 * (1 - p))
    assert s == 256 / kthr
    sigma = math.sqrt(kthr / 256 * (1 - kthr / 256) / keep.size)
    assert abs(keep.mean() - kthr / 256) < 5 * sigma
    # other seeds, offsets and slots give other masks
    assert (oracle.dropout_keep(2, range(256), 1024, 8, 3, p)[0] != keep).mean() > 0.05
    assert (oracle.dropout_keep(2, range(256), 1024, 7, 4, p)[0] != keep).mean() > 0.05
    assert (oracle.dropout_keep(3, range(256), 1024, 7, 3, p)[0] != keep).mean() > 0.05


def test_dropout_p_zero_keeps_everything():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((20, 8)) for _ in range(3))
    drop = oracle.dropout_keep(0, range(20), 20, 99, 0, 0.0)
    assert drop[0].all() and drop[1] == 1.0
    o1, l1 = oracle.attention_fwd(q, k, v, 0.3, True, 0, drop=drop)
    o2, l2 = oracle.attention_fwd(q, k, v, 0.3, True, 0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_dropout_is_unbiased():
    """The mean of O over many seeds approaches the undropped O (the scale
    256/K makes the expectation exact); LSE does not depend on the mask."""
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((12, 8)) for _ in range(3))
    o_ref, l_ref = oracle.attention_fwd(q, k, v, 0.5, True, 0)
    n = 600
    acc = np.zeros_like(o_ref)
    for seed in range(n):
        o, lse = oracle.attention_fwd(q, k, v, 0.5, True, 0, drop=oracle.dropout_keep(0, range(12), 12, seed, 0, 0.3))
        np.testing.assert_array_equal(lse, l_ref)
        acc += o
    # per element the mask variance is p/(1-p) of P^2 V^2 summed over keys; 6 sigma
    p_eff = 1 - round(256 * 0.7) / 256
    probs = oracle.attention_probs(q, k, 0.5, True, 0)
    sd = np.sqrt(p_eff / (1 - p_eff) * (probs ** 2) @ (v ** 2) / n)
    assert (np.abs(acc / n - o_ref) <= 6 * sd + 1e-12).all()


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 5)])
def test_dropout_backward_finite_differences(causal, window):
    """With the mask fixed, O is a smooth function of q, k, v: the oracle's
    gradients match central differences of L = sum(dO * O)."""
    rng = np.random.default_rng(3)
    n, d = 9, 4
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    drop = oracle.dropout_keep(1, range(n), n, 1234, 0, 0.4)
    assert not drop[0].all() and drop[0].any()
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.7, causal, window, drop=drop)

    def loss(qq, kk, vv):
        return (do * oracle.attention_fwd(qq, kk, vv, 0.7, causal, window, drop=drop)[0]).sum()

    eps = 1e-6
    for g, x, which in ((dq, q, 0), (dk, k, 1), (dv, v, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7)
