"""GPU parity of the backward under a causal sliding window narrower than one key tile.

With a causal window W < 64 every query row sees at most W keys, so its
probabilities are concentrated and |dS| is large; these are legal inputs of
the backward (causal mask plus sliding window, the FA-3 paragraph of
"Flash-Attention 2/3在ms-swift中的集成与性能提升").  Whole heads are checked
element by element against the oracle, dense, packed and with dropout.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_24_amd import fa_bwd, fa_fwd, fa_varlen_bwd, fa_varlen_fwd
from exact_attention_24_amd.inputs import dense_inputs, varlen_inputs
from tests.parity import assert_close, assert_lse_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("window", [1, 8, 33, 63])
@pytest.mark.parametrize("d", [64, 128])
def test_dense_small_window(window, d):
    b, n, h = 1, 1100, 8
    print(f"[bwd small window] W={window} d={d} n={n} h={h}", flush=True)
    q, k, v, do = dense_inputs(b, n, h, d, "bf16", seed=window * 10 + d, with_dout=True)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_fwd(qd, kd, vd, causal=True, window=window)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=True, window=window)
    torch.cuda.synchronize()
    sc = 1 / np.sqrt(d)
    ro, rl = oracle.mha_fwd(f64(q), f64(k), f64(v), sc, True, window)
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)
    rq, rk, rv = oracle.mha_bwd(f64(q), f64(k), f64(v), f64(do), sc, True, window)
    assert_close(f64(dq), rq, what="dQ")
    assert_close(f64(dk), rk, what="dK")
    assert_close(f64(dv), rv, what="dV")


@pytest.mark.parametrize("nq,nk,window", [(700, 1000, 20), (1000, 700, 63)])
def test_dense_small_window_unequal_lengths(nq, nk, window):
    """Bottom-right causal alignment with Nq != Nk."""
    print(f"[bwd small window] nq={nq} nk={nk} W={window}", flush=True)
    q, _, _, do = dense_inputs(1, nq, 4, 128, "bf16", seed=nq + window, with_dout=True)
    _, k, v = dense_inputs(1, nk, 4, 128, "bf16", seed=nk + window + 1)
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_fwd(qd, kd, vd, causal=True, window=window)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=True, window=window)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.mha_bwd(f64(q), f64(k), f64(v), f64(do), 1 / np.sqrt(128), True, window)
    assert_close(f64(dq), rq, what="dQ")
    assert_close(f64(dk), rk, what="dK")
    assert_close(f64(dv), rv, what="dV")


@pytest.mark.parametrize("window", [8, 63])
def test_varlen_small_window(window):
    lengths = [300, 1, 77, 513, 0, 64, 129]
    print(f"[varlen bwd small window] W={window} lengths={lengths}", flush=True)
    q, k, v, cu, do = varlen_inputs(lengths, 4, 128, "bf16", seed=window + 3, with_dout=True)
    qd, kd, vd, dod, cud = (x.to(DEV) for x in (q, k, v, do, cu))
    mx = max(lengths)
    o, lse = fa_varlen_fwd(qd, kd, vd, cud, mx, causal=True, window=window)
    dq, dk, dv = fa_varlen_bwd(dod, qd, kd, vd, o, lse, cud, mx, causal=True, window=window)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.varlen_bwd(f64(q), f64(k), f64(v), f64(do), cu.numpy(), 1 / np.sqrt(128), True, window)
    assert_close(f64(dq), rq, what="dQ")
    assert_close(f64(dk), rk, what="dK")
    assert_close(f64(dv), rv, what="dV")


@pytest.mark.parametrize("window,p", [(8, 0.2), (33, 0.1)])
def test_dropout_small_window(window, p):
    b, n, h, d = 1, 600, 4, 128
    print(f"[dropout bwd small window] W={window} p={p}", flush=True)
    q, k, v, do = dense_inputs(b, n, h, d, "bf16", seed=window + 77, with_dout=True)
    seed, off = 31337, 5
    qd, kd, vd, dod = (x.to(DEV) for x in (q, k, v, do))
    o, lse = fa_fwd(qd, kd, vd, causal=True, window=window, dropout_p=p, seed=seed, offset=off)
    dq, dk, dv = fa_bwd(dod, qd, kd, vd, o, lse, causal=True, window=window, dropout_p=p, seed=seed, offset=off)
    torch.cuda.synchronize()
    sc = 1 / np.sqrt(d)
    ro, rl = oracle.mha_fwd(f64(q), f64(k), f64(v), sc, True, window, dropout=(p, seed, off))
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)
    rq, rk, rv = oracle.mha_bwd(f64(q), f64(k), f64(v), f64(do), sc, True, window, dropout=(p, seed, off))
    assert_close(f64(dq), rq, what="dQ")
    assert_close(f64(dk), rk, what="dK")
    assert_close(f64(dv), rv, what="dV")
