"""GPU parity of the fp8 (OCP e4m3) forward against the fp64 oracle run on the
dequantised inputs (code * per-tensor scale, decoded by the oracle's own
e4m3 decoder)."""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_24_amd import fa_fwd
from exact_attention_24_amd.inputs import WORKLOADS, dense_inputs, quantize_e4m3, workload_inputs
from tests.parity import FP8_MAX_ABS, assert_close, assert_lse_close, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _codes(t):
    return t.view(torch.uint8).numpy()


def _deq(t, s):
    return oracle.fp8_dequant(_codes(t), s)


@pytest.mark.parametrize("b,n,h,d,causal,window", [
    (1, 1, 1, 128, False, 0),
    (1, 300, 2, 128, True, 0),
    (2, 257, 2, 128, False, 0),
    (1, 520, 2, 128, True, 100),
    (1, 333, 3, 64, True, 0),
])
def test_fp8_small_elementwise(b, n, h, d, causal, window):
    print(f"[fp8] b={b} n={n} h={h} d={d} causal={causal} window={window}", flush=True)
    q, k, v = dense_inputs(b, n, h, d, "bf16", seed=n + d)
    (q8, sq), (k8, sk), (v8, sv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    o, lse = fa_fwd(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=causal, window=window, descale=(sq, sk, sv))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    ro, rl = oracle.mha_fwd(_deq(q8, sq), _deq(k8, sk), _deq(v8, sv), 1 / np.sqrt(d), causal, window)
    assert_close(o.cpu().double().numpy(), ro, max_abs=FP8_MAX_ABS, mean_abs=None, what="O fp8")
    # LSE uses fp32 probabilities before quantisation: as accurate as bf16
    mx = assert_lse_close(lse.cpu().double().numpy(), rl)
    print(f"[fp8 small] LSE max abs error {mx:.2e}", flush=True)


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_n8192_sampled_rows(causal):
    w = WORKLOADS["fp8_n8192"]
    t = workload_inputs("fp8_n8192")
    ds = (t["q_scale"], t["k_scale"], t["v_scale"])
    print(f"[fp8 n8192 causal={causal}] launching", flush=True)
    o, lse = fa_fwd(t["q8"].to(DEV), t["k8"].to(DEV), t["v8"].to(DEV), causal=causal, descale=ds)
    torch.cuda.synchronize()
    q = _deq(t["q8"], ds[0])
    k = _deq(t["k8"], ds[1])
    v = _deq(t["v8"], ds[2])
    o64, lse64 = o.cpu().double().numpy(), lse.cpu().double().numpy()
    worst = 0.0
    for h in range(0, w.heads, 3):
        rows = sample_rows(w.seqlen, 48, seed=100 + h)
        ro, rl = oracle.attention_fwd(q[0, rows, h], k[0, :, h], v[0, :, h], w.scale, causal, 0,
                                      q_pos=rows, nq=w.seqlen)
        assert_close(o64[0, rows, h], ro, max_abs=FP8_MAX_ABS, mean_abs=None, what=f"O fp8 head {h}")
        worst = max(worst, assert_lse_close(lse64[0, h, rows], rl))
    print(f"[fp8 n8192 causal={causal}] LSE max abs error {worst:.2e}", flush=True)
    ro, _ = oracle.attention_fwd(q[0, :, 7], k[0, :, 7], v[0, :, 7], w.scale, causal, 0)
    assert_close(o64[0, :, 7], ro, max_abs=FP8_MAX_ABS, mean_abs=None, what="O fp8 full head 7")


@pytest.mark.parametrize("b,n,h,d,causal,window", [
    # >= 256 work units (one per CU): the persistent schedule
    (2, 1100, 48, 128, True, 0),     # 5 query tiles: the middle one unpaired; ragged tail
    (2, 1536, 48, 64, True, 300),    # causal + window, d64
    (1, 1100, 64, 128, False, 0),    # non-causal
])
def test_fp8_persistent_schedule_sampled_rows(b, n, h, d, causal, window):
    print(f"[fp8 persistent] b={b} n={n} h={h} d={d} causal={causal} window={window}", flush=True)
    q, k, v = dense_inputs(b, n, h, d, "bf16", seed=n + 3 * h)
    (q8, sq), (k8, sk), (v8, sv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    o, lse = fa_fwd(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=causal, window=window, descale=(sq, sk, sv))
    torch.cuda.synchronize()
    qd, kd, vd = _deq(q8, sq), _deq(k8, sk), _deq(v8, sv)
    o64, lse64 = o.cpu().double().numpy(), lse.cpu().double().numpy()
    for bi in range(b):
        for hh in sorted({0, (h // 2 + 5 * bi) % h, h - 1}):
            rows = np.union1d(sample_rows(n, 24, seed=bi * 100 + hh), [0, 255, 256, n - 1])
            ro, rl = oracle.attention_fwd(qd[bi, rows, hh], kd[bi, :, hh], vd[bi, :, hh], 1 / np.sqrt(d), causal, window,
                                          q_pos=rows, nq=n)
            assert_close(o64[bi, rows, hh], ro, max_abs=FP8_MAX_ABS, mean_abs=None, what=f"O fp8 batch {bi} head {hh}")
            assert_lse_close(lse64[bi, hh, rows], rl)


def test_fp8_causal_row0():
    """Row 0 sees only key 0: P~ = 1 exactly in e4m3, so O_0 = s_v * code(V_0) rounded to bf16."""
    q, k, v = dense_inputs(1, 100, 2, 128, "bf16", seed=5)
    (q8, sq), (k8, sk), (v8, sv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
    o, _ = fa_fwd(q8.to(DEV), k8.to(DEV), v8.to(DEV), causal=True, descale=(sq, sk, sv))
    torch.cuda.synchronize()
    ref = torch.from_numpy(_deq(v8, sv)[:, 0]).to(torch.bfloat16)
    assert torch.equal(o.cpu()[:, 0], ref)
