"""fa_bwd_noalloc (the backward without any allocation, for callers that
cannot allocate) against fa_bwd on the same inputs, through the C ABI."""

import ctypes

import pytest
import torch

from exact_attention_24_amd import binding as B
from exact_attention_24_amd import fa_bwd, fa_bwd_noalloc, fa_fwd
from exact_attention_24_amd.inputs import dense_inputs

DEV = "cuda:0"


def _case(b, n, h, d, causal, window, seed):
    q, k, v, do = (x.to(DEV) for x in dense_inputs(b, n, h, d, "bf16", seed=seed, with_dout=True))
    o, lse = fa_fwd(q, k, v, causal=causal, window=window)
    return q, k, v, do, o, lse


@pytest.mark.gpu
def test_noalloc_equals_fa_bwd_on_two_calls_in_a_row():
    """Two calls in a row on one device, the second smaller (and on the
    narrow-window kernels): each equals fa_bwd bitwise, so the second call
    does not see the first call's scratch contents."""
    for (b, n, h, d, causal, window, seed) in ((2, 1500, 16, 128, True, 0, 71), (1, 700, 4, 64, True, 40, 72)):
        print(f"[no-alloc bwd] b={b} n={n} h={h} d={d} causal={causal} window={window}", flush=True)
        q, k, v, do, o, lse = _case(b, n, h, d, causal, window, seed)
        ref = fa_bwd(do, q, k, v, o, lse, causal=causal, window=window, deterministic=True)
        got = tuple(torch.full_like(x, float("nan")) for x in ref)
        fa_bwd_noalloc(do, q, k, v, o, lse, *got, causal=causal, window=window, deterministic=True)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(g, r), f"{name} differs from fa_bwd"


def test_noalloc_refuses_calls_beyond_its_scratch():
    """More than 2^20 rows of batch x heads x seqlen_q: refused on the host
    with the documented error before any device call."""
    L = B.lib()
    q = torch.zeros(1, 16, 2, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 16, dtype=torch.float32)
    g = torch.zeros(1, 16, 2, 64, dtype=torch.float32)
    p = B.make_bwd_params(q, q, q, q, q, lse, g, g, g, causal=True)
    p.heads, p.seqlen_q, p.seqlen_k = 64, 20000, 20000  # 1.28e6 rows > 2^20
    for i in range(3):
        p.q_stride[i] = p.k_stride[i] = p.v_stride[i] = p.o_stride[i] = p.do_stride[i] = 0
        p.dq_stride[i] = p.dk_stride[i] = p.dv_stride[i] = 0
    p.q_stride[1] = p.k_stride[1] = p.v_stride[1] = p.o_stride[1] = p.do_stride[1] = 64
    p.dq_stride[1] = p.dk_stride[1] = p.dv_stride[1] = 64
    assert L.fa_check_bwd(ctypes.byref(p)) == B.FA_OK
    assert L.fa_bwd_noalloc(ctypes.byref(p), None) == B.FA_ERR_INVALID_ARGUMENT
    assert b"static" in L.fa_last_error()
