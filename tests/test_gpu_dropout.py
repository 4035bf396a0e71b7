"""GPU parity of dropout in the forward and backward (dense and packed)
against the fp64 oracle, which draws the same Philox4x32-10 mask from its own
implementation of the generator."""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_24_amd import fa_bwd, fa_fwd, fa_varlen_bwd, fa_varlen_fwd
from exact_attention_24_amd.inputs import WORKLOADS, dense_inputs, varlen_inputs, workload_inputs
from tests.parity import BF16_MAX_ABS, assert_close, assert_lse_close, f64, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _close_rel(got, ref, what):
    """|got - ref| <= 1e-2 + 2^-8 |ref|: bf16 rounding of large one-hot sums
    on top of the absolute bound; a wrong mask bit moves an element by at
    least amp * scale / (visible keys) >= 16 / 400, far outside it."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = BF16_MAX_ABS + np.abs(ref) * 2.0 ** -8
    assert (err <= bound).all(), f"{what}: max excess {(err - bound).max():.3e} at {np.unravel_index(np.argmax(err - bound), err.shape)}"


def _onehot(n, d, amp):
    """Rows amp * e_(j mod d): attention output column c then sums the dropped,
    rescaled probabilities of the keys j = c mod d, so one wrong mask bit moves
    an output by amp * scale / (visible keys), far above the tolerance."""
    x = torch.zeros(n, d)
    x[torch.arange(n), torch.arange(n) % d] = amp
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("nq,nk,causal,window,p", [
    (300, 192, False, 0, 0.1), (300, 300, True, 0, 0.3), (257, 257, True, 40, 0.5), (64, 200, True, 0, 0.1),
])
def test_forward_mask_is_the_oracle_mask(nq, nk, causal, window, p):
    """Uniform probabilities (scale 1e-30) and one-hot V rows: O shows the mask."""
    print(f"[dropout mask fwd] nq={nq} nk={nk} causal={causal} window={window} p={p}", flush=True)
    b, h, d = 2, 3, 64
    g = torch.Generator().manual_seed(nq + nk)
    q = torch.randn(b, nq, h, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, nk, h, d, generator=g).to(torch.bfloat16)
    v = _onehot(nk, d, 16.0)[None, :, None, :].expand(b, nk, h, d).contiguous()
    seed, off = 0x1234_5678_9ABC_DEF0 + nq, 7
    o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, softmax_scale=1e-30,
                    dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    ro, rl = oracle.mha_fwd(f64(q), f64(k), f64(v), 1e-30, causal, window, dropout=(p, seed, off))
    _close_rel(f64(o), ro, "O")
    assert_lse_close(f64(lse), rl)


@pytest.mark.parametrize("nq,nk,causal,window,p", [
    (300, 192, False, 0, 0.1), (300, 300, True, 0, 0.3), (257, 257, True, 40, 0.5), (150, 400, True, 0, 0.2),
])
def test_backward_mask_is_the_oracle_mask(nq, nk, causal, window, p):
    """Uniform probabilities and one-hot dO rows: dV = (P keep s)^T dO shows
    the mask in the key-major orientation of the dK/dV kernel; dQ, dK too."""
    print(f"[dropout mask bwd] nq={nq} nk={nk} causal={causal} window={window} p={p}", flush=True)
    b, h, d = 1, 2, 64
    g = torch.Generator().manual_seed(nq * 3 + nk)
    q = torch.randn(b, nq, h, d, generator=g).to(torch.bfloat16)
    k = torch.randn(b, nk, h, d, generator=g).to(torch.bfloat16)
    v = torch.randn(b, nk, h, d, generator=g).to(torch.bfloat16)
    do = _onehot(nq, d, 16.0)[None, :, None, :].expand(b, nq, h, d).contiguous()
    seed, off = 99 + nq, 3
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_fwd(qd, kd, vd, causal=causal, window=window, softmax_scale=1e-30, dropout_p=p, seed=seed, offset=off)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, window=window, softmax_scale=1e-30, dropout_p=p,
                        seed=seed, offset=off)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.mha_bwd(f64(q), f64(k), f64(v), f64(do), 1e-30, causal, window, dropout=(p, seed, off))
    _close_rel(f64(dv), rv, "dV")
    _close_rel(f64(dk), rk, "dK")
    _close_rel(f64(dq), rq, "dQ")


@pytest.mark.parametrize("b,nq,nk,h,d,causal,window,p", [
    (2, 1024, 1024, 16, 64, True, 0, 0.1),      # the packed-QKV API example of the MindSpore page
    (1, 300, 300, 2, 128, True, 0, 0.2),
    (1, 520, 520, 2, 128, True, 130, 0.1),
    (1, 257, 257, 3, 64, False, 0, 0.5),
    (1, 150, 400, 2, 128, True, 0, 0.1),
])
def test_dropout_random_inputs(b, nq, nk, h, d, causal, window, p):
    print(f"[dropout] b={b} nq={nq} nk={nk} h={h} d={d} causal={causal} window={window} p={p}", flush=True)
    q, _, _, do = dense_inputs(b, nq, h, d, "bf16", seed=nq + 17, with_dout=True)
    _, k, v = dense_inputs(b, nk, h, d, "bf16", seed=nk + 18)
    seed, off = 2024, nq
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_fwd(qd, kd, vd, causal=causal, window=window, dropout_p=p, seed=seed, offset=off)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=causal, window=window, dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    sc = 1 / np.sqrt(d)
    heads = [(0, 0), (b - 1, h - 1)] if b * h > 4 else None
    ro, rl = oracle.mha_fwd(f64(q), f64(k), f64(v), sc, causal, window, heads=heads, dropout=(p, seed, off))
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)
    rq, rk, rv = oracle.mha_bwd(f64(q), f64(k), f64(v), f64(do), sc, causal, window, heads=heads,
                                dropout=(p, seed, off))
    assert_close(f64(dq), rq, what="dQ")
    assert_close(f64(dk), rk, what="dK")
    assert_close(f64(dv), rv, what="dV")


def test_dropout_persistent_schedule():
    """B2 N1100 H48 d64 causal, p = 0.1: enough work units that the forward
    and the dQ kernel run their persistent schedules (5 query tiles, the
    middle one unpaired).  Sampled forward rows and whole-head gradients of
    a few (batch, head) slots against the oracle's own Philox mask."""
    b, n, h, d, p = 2, 1100, 48, 64, 0.1
    q, k, v, do = dense_inputs(b, n, h, d, "bf16", seed=55, with_dout=True)
    seed, off = 909, 3
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_fwd(qd, kd, vd, causal=True, dropout_p=p, seed=seed, offset=off)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=True, dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = f64(q), f64(k), f64(v), f64(do)
    o64, l64, dq64, dk64, dv64 = f64(o), f64(lse), f64(dq), f64(dk), f64(dv)
    sc = 1 / np.sqrt(d)
    for bi, hh in ((0, 0), (0, 29), (1, 7), (1, h - 1)):
        slot = bi * h + hh
        rows = np.union1d(sample_rows(n, 32, seed=slot), [255, 256, 1023, 1024])
        drop = oracle.dropout_keep(slot, rows, n, seed, off, p)
        ro, rl = oracle.attention_fwd(q64[bi, rows, hh], k64[bi, :, hh], v64[bi, :, hh], sc, True, 0, q_pos=rows, nq=n,
                                      drop=drop)
        assert_close(o64[bi, rows, hh], ro, what=f"O slot {slot}")
        assert_lse_close(l64[bi, hh, rows], rl)
        drop = oracle.dropout_keep(slot, range(n), n, seed, off, p)
        rq, rk, rv = oracle.attention_bwd(q64[bi, :, hh], k64[bi, :, hh], v64[bi, :, hh], do64[bi, :, hh], sc, True, 0,
                                          drop=drop)
        assert_close(dq64[bi, :, hh], rq, what=f"dQ slot {slot}")
        assert_close(dk64[bi, :, hh], rk, what=f"dK slot {slot}")
        assert_close(dv64[bi, :, hh], rv, what=f"dV slot {slot}")


def test_dropout_varlen():
    lengths = [300, 1, 77, 513, 0]
    q, k, v, cu, do = varlen_inputs(lengths, 2, 128, "bf16", seed=31, with_dout=True)
    mx = max(lengths)
    seed, off, p = 5, 11, 0.15
    qd, kd, vd, dod, cud = (x.to(DEV) for x in (q, k, v, do, cu))
    o, lse = fa_varlen_fwd(qd, kd, vd, cud, mx, causal=True, window=100, dropout_p=p, seed=seed, offset=off)
    dq, dk, dv = fa_varlen_bwd(dod, qd, kd, vd, o, lse, cud, mx, causal=True, window=100, dropout_p=p, seed=seed,
                               offset=off)
    torch.cuda.synchronize()
    sc = 1 / np.sqrt(128)
    ro, rl = oracle.varlen_fwd(f64(q), f64(k), f64(v), cu.numpy(), sc, True, 100, dropout=(p, seed, off))
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)
    rq, rk, rv = oracle.varlen_bwd(f64(q), f64(k), f64(v), f64(do), cu.numpy(), sc, True, 100, dropout=(p, seed, off))
    assert_close(f64(dq), rq, what="dQ")
    assert_close(f64(dk), rk, what="dK")
    assert_close(f64(dv), rv, what="dV")


def test_dropout_seed_and_offset():
    q, k, v = (x.to(DEV) for x in dense_inputs(1, 256, 2, 64, "bf16", seed=4))
    o1 = fa_fwd(q, k, v, causal=True, dropout_p=0.2, seed=1, offset=0, return_lse=False)
    o2 = fa_fwd(q, k, v, causal=True, dropout_p=0.2, seed=1, offset=0, return_lse=False)
    o3 = fa_fwd(q, k, v, causal=True, dropout_p=0.2, seed=1, offset=1, return_lse=False)
    o4 = fa_fwd(q, k, v, causal=True, dropout_p=0.2, seed=2, offset=0, return_lse=False)
    o0 = fa_fwd(q, k, v, causal=True, return_lse=False)
    o5 = fa_fwd(q, k, v, causal=True, dropout_p=0.001, seed=1, return_lse=False)  # rounds to no dropout
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert not torch.equal(o1, o3) and not torch.equal(o1, o4)
    assert torch.equal(o0, o5)


def test_dropout_n8192_full_size():
    """B1 H32 N8192 d128 causal, p = 0.1: sampled forward rows of 4 heads, and
    two whole heads of the backward, element by element."""
    w = WORKLOADS["bwd_n8192"]
    t = workload_inputs("bwd_n8192")
    seed, off, p = 77, 1, 0.1
    qd, kd, vd, dod = (t[x].to(DEV) for x in ("q", "k", "v", "dout"))
    print("[dropout n8192] launching", flush=True)
    o, lse = fa_fwd(qd, kd, vd, causal=True, dropout_p=p, seed=seed, offset=off)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=True, dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    q, k, v, do = (f64(t[x]) for x in ("q", "k", "v", "dout"))
    o64, l64 = f64(o), f64(lse)
    rows = sample_rows(8192, 40, seed=8)
    for h in (0, 11, 20, 31):
        drop = oracle.dropout_keep(h, rows, 8192, seed, off, p)
        ro, rl = oracle.attention_fwd(q[0, rows, h], k[0, :, h], v[0, :, h], w.scale, True, 0, q_pos=rows, nq=8192,
                                      drop=drop)
        assert_close(o64[0, rows, h], ro, what=f"O head {h}")
        assert_lse_close(l64[0, h, rows], rl)
    dq64, dk64, dv64 = f64(dq), f64(dk), f64(dv)
    for h in (0, 31):
        drop = oracle.dropout_keep(h, range(8192), 8192, seed, off, p)
        rq, rk, rv = oracle.attention_bwd(q[0, :, h], k[0, :, h], v[0, :, h], do[0, :, h], w.scale, True, 0, drop=drop)
        assert_close(dq64[0, :, h], rq, what=f"dQ head {h}")
        assert_close(dk64[0, :, h], rk, what=f"dK head {h}")
        assert_close(dv64[0, :, h], rv, what=f"dV head {h}")
