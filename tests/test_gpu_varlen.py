"""GPU parity of the packed variable-length forward (cu_seqlens) against the
fp64 oracle, and against the dense forward run on each sequence alone."""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_24_amd import fa_fwd, fa_varlen_fwd
from exact_attention_24_amd.inputs import WORKLOADS, varlen_inputs, workload_inputs
from tests.parity import assert_close, assert_lse_close, f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(q, k, v, cu, causal, window, dtype_out=None):
    mx = int((cu[1:] - cu[:-1]).max()) if cu.numel() > 1 else 0
    o, lse = fa_varlen_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), mx, causal=causal, window=window)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("lengths,h,d,causal,window,dt", [
    ([5, 1, 130, 257, 64], 2, 64, True, 0, "bf16"),
    ([300, 0, 77, 513], 2, 128, True, 100, "bf16"),
    ([200, 201, 1], 3, 128, False, 0, "bf16"),
    ([129, 40], 2, 128, False, 33, "bf16"),
    ([70, 3, 150], 2, 64, True, 0, "f32"),
    ([90, 0, 161, 33], 2, 128, True, 40, "f32"),
])
def test_varlen_small_elementwise(lengths, h, d, causal, window, dt):
    print(f"[varlen] lengths={lengths} h={h} d={d} causal={causal} window={window} {dt}", flush=True)
    q, k, v, cu = varlen_inputs(lengths, h, d, dt, seed=sum(lengths))
    o, lse = _run(q, k, v, cu, causal, window)
    ro, rl = oracle.varlen_fwd(f64(q), f64(k), f64(v), cu.numpy(), 1 / np.sqrt(d), causal, window)
    assert_close(f64(o), ro)
    assert_lse_close(f64(lse), rl)


def test_varlen_many_sequences_elementwise():
    """600 short sequences (more than one packed call schedules on the device,
    so the one-item-per-work-group launch runs), some empty, causal and not."""
    rng = np.random.default_rng(600)
    lengths = [int(x) for x in rng.integers(0, 40, size=600)]
    q, k, v, cu = varlen_inputs(lengths, 2, 64, "bf16", seed=600)
    for causal in (True, False):
        o, lse = _run(q, k, v, cu, causal, 0)
        ro, rl = oracle.varlen_fwd(f64(q), f64(k), f64(v), cu.numpy(), 1 / np.sqrt(64), causal, 0)
        assert_close(f64(o), ro, what=f"O causal={causal}")
        assert_lse_close(f64(lse), rl)


def test_varlen_equals_dense_per_sequence_bitwise():
    lengths = [300, 1, 513, 64]
    q, k, v, cu = varlen_inputs(lengths, 4, 128, "bf16", seed=9)
    o, lse = _run(q, k, v, cu, True, 128)
    for s in range(len(lengths)):
        a, b = int(cu[s]), int(cu[s + 1])
        od, ld = fa_fwd(q[a:b][None].to(DEV), k[a:b][None].to(DEV), v[a:b][None].to(DEV), causal=True, window=128)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], od[0].cpu())
        assert torch.equal(lse[:, a:b], ld[0].cpu())


def test_varlen_32k_window4096_sampled():
    """28 heads, d128, 32768 packed tokens (lengths U{512..8192}), causal +
    window 4096: every sequence, sampled rows of every 4th head."""
    w = WORKLOADS["varlen_32k"]
    t = workload_inputs("varlen_32k")
    print(f"[varlen 32k] lengths={t['lengths']}", flush=True)
    o, lse = _run(t["q"], t["k"], t["v"], t["cu_seqlens"], True, w.window)
    q, k, v = f64(t["q"]), f64(t["k"]), f64(t["v"])
    o64, l64 = f64(o), f64(lse)
    cu = t["cu_seqlens"].numpy()
    rng = np.random.default_rng(4)
    for s in range(len(t["lengths"])):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(24, n), replace=False)]))
        for h in range(s % 4, w.heads, 4):
            ro, rl = oracle.attention_fwd(q[a + rows, h], k[a:b, h], v[a:b, h], w.scale, True, w.window,
                                          q_pos=rows, nq=n)
            assert_close(o64[a + rows, h], ro, what=f"O seq {s} head {h}")
            assert_lse_close(l64[h, a + rows], rl)


def test_host_cu_seqlens_is_refused():
    """cu_seqlens left on the host raises before anything is launched."""
    q, k, v, cu = varlen_inputs([30, 10], 2, 64, "bf16", seed=1)
    with pytest.raises(ValueError, match="cu_seqlens"):
        fa_varlen_fwd(q.to(DEV), k.to(DEV), v.to(DEV), cu, 30, causal=True)
