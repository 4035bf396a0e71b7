"""GPU parity of the forward kernels against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_24_amd import fa_bwd, fa_fwd
from exact_attention_24_amd.inputs import WORKLOADS, dense_inputs, workload_inputs
from tests.parity import assert_close, assert_lse_close, f64, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(q, k, v, causal, window, scale=None):
    o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, softmax_scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _oracle(q, k, v, scale, causal, window):
    return oracle.mha_fwd(f64(q), f64(k), f64(v), scale, causal, window)


SMALL = [
    # (batch, nq, nk, heads, d, causal, window)
    (1, 1, 1, 1, 64, False, 0),
    (1, 17, 17, 2, 64, True, 0),
    (2, 300, 300, 3, 64, False, 0),
    (2, 300, 300, 3, 128, True, 0),
    (1, 257, 257, 2, 128, False, 0),
    (1, 513, 513, 2, 128, True, 100),
    (1, 384, 384, 2, 64, True, 64),
    (1, 200, 200, 2, 128, False, 37),
    (1, 130, 333, 2, 128, True, 0),   # Nq < Nk: bottom-right causal
    (1, 333, 130, 2, 64, True, 0),    # Nq > Nk: the first rows see no key
    (1, 1, 700, 3, 128, True, 0),     # one query (decode-like) over many keys
]


@pytest.mark.parametrize("b,nq,nk,h,d,causal,window", SMALL)
def test_bf16_small_elementwise(b, nq, nk, h, d, causal, window):
    print(f"[fwd bf16] b={b} nq={nq} nk={nk} h={h} d={d} causal={causal} window={window}", flush=True)
    q, _, _ = dense_inputs(b, nq, h, d, "bf16", seed=nq * 31 + nk)
    _, k, v = dense_inputs(b, nk, h, d, "bf16", seed=nq * 31 + nk + 1)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, causal, window)
    ro, rl = _oracle(q, k, v, scale, causal, window)
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)


@pytest.mark.parametrize("d", [64, 128])
def test_f32_small_elementwise(d):
    print(f"[fwd f32] d={d}", flush=True)
    q, k, v = dense_inputs(2, 150, 3, d, "f32", seed=7)
    o, lse = _run(q, k, v, True, 0)
    ro, rl = _oracle(q, k, v, 1 / np.sqrt(d), True, 0)
    assert_close(f64(o), ro, max_abs=1e-5, mean_abs=1e-6)
    assert_lse_close(f64(lse), rl, tol=1e-5)


@pytest.mark.parametrize("b,nq,nk,h,d,causal,window", SMALL)
def test_f32_shapes_elementwise(b, nq, nk, h, d, causal, window):
    """The fp32 kernel splits each tile's keys over its 4 waves and merges the
    waves' states: windows, tails, Nq != Nk and rows that see no key."""
    print(f"[fwd f32] b={b} nq={nq} nk={nk} h={h} d={d} causal={causal} window={window}", flush=True)
    q, _, _ = dense_inputs(b, nq, h, d, "f32", seed=nq * 17 + nk)
    _, k, v = dense_inputs(b, nk, h, d, "f32", seed=nq * 17 + nk + 1)
    o, lse = _run(q, k, v, causal, window)
    ro, rl = _oracle(q, k, v, 1 / np.sqrt(d), causal, window)
    assert_close(f64(o), ro, max_abs=1e-5, mean_abs=1e-6)
    assert_lse_close(f64(lse), rl, tol=1e-5)


def test_tiny_fp32_workload():
    """B1 H1 N256 d64 fp32, non-causal, scale 1/8: the whole output."""
    w = WORKLOADS["tiny_fp32"]
    t = workload_inputs("tiny_fp32")
    o, lse = _run(t["q"], t["k"], t["v"], w.causal, w.window)
    ro, rl = _oracle(t["q"], t["k"], t["v"], w.scale, w.causal, w.window)
    mx, mn = assert_close(f64(o), ro)
    assert mx < 1e-5, mx
    assert_lse_close(f64(lse), rl)


def test_b2_h16_n1024_workload():
    """B2 H16 N1024 d64 bf16 causal: every head, every element."""
    w = WORKLOADS["b2_h16_n1024"]
    t = workload_inputs("b2_h16_n1024")
    o, lse = _run(t["q"], t["k"], t["v"], w.causal, w.window)
    ro, rl = _oracle(t["q"], t["k"], t["v"], w.scale, w.causal, w.window)
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)


@pytest.mark.parametrize("name", ["llama_n8192", "llama_n8192_noncausal"])
def test_llama_n8192_sampled_rows(name):
    """B1 H32 N8192 d128 bf16 at full size: sampled rows of every head, checked
    one by one against the oracle, plus two whole heads."""
    w = WORKLOADS[name]
    t = workload_inputs(name)
    print(f"[fwd {name}] launching", flush=True)
    o, lse = _run(t["q"], t["k"], t["v"], w.causal, w.window)
    q, k, v = f64(t["q"]), f64(t["k"]), f64(t["v"])
    o64, lse64 = f64(o), f64(lse)
    for h in range(w.heads):
        rows = sample_rows(w.seqlen, 48, seed=h)
        ro, rl = oracle.attention_fwd(q[0, rows, h], k[0, :, h], v[0, :, h], w.scale, w.causal, w.window,
                                      q_pos=rows, nq=w.seqlen)
        assert_close(o64[0, rows, h], ro, what=f"O head {h}")
        assert_lse_close(lse64[0, h, rows], rl)
    for h in (0, w.heads - 1):
        ro, rl = oracle.attention_fwd(q[0, :, h], k[0, :, h], v[0, :, h], w.scale, w.causal, w.window)
        assert_close(o64[0, :, h], ro, what=f"O full head {h}")
        assert_lse_close(lse64[0, h], rl)


PERSISTENT = [
    # shapes with >= 256 work units (one per CU), so the bf16 forward runs its
    # persistent schedule: (batch, nq, nk, heads, d, causal, window)
    (2, 1100, 1100, 48, 64, True, 0),     # 5 query tiles: the middle one is unpaired; ragged last tile
    (3, 1300, 1300, 32, 128, True, 0),    # 6 query tiles, batch 3
    (2, 1536, 1536, 48, 128, True, 300),  # causal + sliding window
    (1, 1100, 1500, 64, 128, False, 0),   # non-causal, Nq < Nk
    (2, 900, 1400, 64, 64, True, 0),      # bottom-right causal, Nq < Nk
    (1, 1000, 1000, 64, 128, False, 200), # window without causal
    (2, 1000, 600, 64, 128, True, 0),     # Nq > Nk: whole query tiles see no key (items without key tiles)
    (2, 1100, 700, 48, 64, True, 0),      # the same at d = 64, 5 query tiles
]


@pytest.mark.parametrize("b,nq,nk,h,d,causal,window", PERSISTENT)
def test_bf16_persistent_schedule_sampled_rows(b, nq, nk, h, d, causal, window):
    print(f"[fwd persistent] b={b} nq={nq} nk={nk} h={h} d={d} causal={causal} window={window}", flush=True)
    q, _, _ = dense_inputs(b, nq, h, d, "bf16", seed=nq * 7 + h)
    _, k, v = dense_inputs(b, nk, h, d, "bf16", seed=nk * 7 + h + 1)
    scale = 1.0 / np.sqrt(d)
    o, lse = _run(q, k, v, causal, window)
    q64, k64, v64, o64, lse64 = f64(q), f64(k), f64(v), f64(o), f64(lse)
    for bi in range(b):
        for hh in sorted({0, h // 2 + bi, h - 1}):
            rows = sample_rows(nq, 24, seed=bi * 1000 + hh)
            rows = np.union1d(rows, [0, nq - 1, min(nq - 1, 255), min(nq - 1, 256)])
            ro, rl = oracle.attention_fwd(q64[bi, rows, hh], k64[bi, :, hh], v64[bi, :, hh], scale, causal, window,
                                          q_pos=rows, nq=nq)
            assert_close(o64[bi, rows, hh], ro, what=f"O batch {bi} head {hh}")
            assert_lse_close(lse64[bi, hh, rows], rl)


def test_causal_row0_is_v0_bitwise():
    """Causal row 0 sees only key 0: P~ = 1, l = 1, so O_0 is exactly V_0."""
    q, k, v = dense_inputs(2, 500, 4, 128, "bf16", seed=3)
    o, _ = _run(q, k, v, True, 0)
    assert torch.equal(o[:, 0], v[:, 0])


def test_constant_v_and_single_key_on_gpu():
    q, k, v = dense_inputs(1, 260, 2, 64, "bf16", seed=4)
    vc = torch.ones_like(v) * torch.tensor(0.625, dtype=torch.bfloat16)
    o, _ = _run(q, k, vc, True, 0)
    assert torch.equal(o, torch.full_like(o, 0.625))
    o1, lse1 = _run(q, k[:, :1], v[:, :1], False, 0)
    assert torch.equal(o1, v[:, :1].expand_as(o1))


def test_deterministic_repeat():
    q, k, v = dense_inputs(1, 1000, 4, 128, "bf16", seed=5)
    o1, l1 = _run(q, k, v, True, 0)
    o2, l2 = _run(q, k, v, True, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_packed_qkv_strides():
    """(batch, seqlen, 3, heads, head_dim) packed QKV through strided views."""
    g = torch.Generator().manual_seed(6)
    qkv = torch.randn(2, 200, 3, 4, 64, generator=g).to(torch.bfloat16)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    qkv_d = qkv.to(DEV)
    o, lse = fa_fwd(qkv_d[:, :, 0], qkv_d[:, :, 1], qkv_d[:, :, 2], causal=True)
    torch.cuda.synchronize()
    ro, rl = _oracle(q, k, v, 1 / 8, True, 0)
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)


def test_bhnd_layout_through_strides():
    q, k, v = dense_inputs(1, 256, 4, 128, "bf16", seed=8)
    qt, kt, vt = (x.transpose(1, 2).contiguous().to(DEV) for x in (q, k, v))  # [B,H,N,d] storage
    o, _ = fa_fwd(qt.transpose(1, 2), kt.transpose(1, 2), vt.transpose(1, 2), causal=False)
    torch.cuda.synchronize()
    ro, _ = _oracle(q, k, v, 1 / np.sqrt(128), False, 0)
    assert_close(f64(o), ro)


def test_empty_inputs():
    z = torch.empty(0, 16, 2, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = fa_fwd(z, z, z, causal=True)
    assert o.shape == z.shape
    q = torch.randn(1, 5, 2, 64, device=DEV).to(torch.bfloat16)
    kv = torch.empty(1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = fa_fwd(q, kv, kv)
    torch.cuda.synchronize()
    assert (o.float() == 0).all() and torch.isneginf(lse).all()


@pytest.mark.parametrize("causal,window,nq,nk", [(True, 0, 700, 700), (True, 40, 700, 700), (False, 100, 300, 500),
                                                 (True, 0, 200, 600)])
def test_scale_zero_is_the_mean_over_visible_keys(causal, window, nq, nk):
    """softmax_scale = 0 weighs every visible key equally: O is the mean of V
    over them and LSE = ln(their count) (a closed form the oracle is pinned
    to); this checks the masks and the running sums on every tile size."""
    q, _, _ = dense_inputs(1, nq, 3, 128, "bf16", seed=nq + 5)
    _, k, v = dense_inputs(1, nk, 3, 128, "bf16", seed=nk + 6)
    o, lse = _run(q, k, v, causal, window, scale=0.0)
    ro, rl = _oracle(q, k, v, 0.0, causal, window)
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)
    cnt = oracle.visible(np.arange(nq), nk, causal, window, offset=nk - nq).sum(axis=1)
    assert_lse_close(f64(lse)[0], np.broadcast_to(np.where(cnt > 0, np.log(np.maximum(cnt, 1)), -np.inf), (3, nq)))
    # backward: scale 0 makes dQ = dK = 0 exactly; dV = P^T dO with uniform P
    do = dense_inputs(1, nq, 3, 128, "bf16", seed=nq + 7)[0]
    dq, dk, dv = fa_bwd(do.to(DEV), q.to(DEV), k.to(DEV), v.to(DEV), o.to(DEV), lse.to(DEV), causal=causal,
                        window=window, softmax_scale=0.0)
    torch.cuda.synchronize()
    assert (dq.cpu() == 0).all() and (dk.cpu() == 0).all()
    _, _, rv = oracle.mha_bwd(f64(q), f64(k), f64(v), f64(do), 0.0, causal, window)
    assert_close(f64(dv), rv, what="dV")
