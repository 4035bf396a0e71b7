"""Packed calls whose tensors span more than 2 GiB per head: the kernels address
rows from each sequence's own start, so only a sequence's own extent is bound
by 32-bit offsets.  The sequences that start past the 2 GiB mark must come out
bitwise equal to the same sequences run alone."""

import pytest
import torch

from exact_attention_24_amd import fa_varlen_bwd, fa_varlen_fwd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

H, D, L, NSEQ = 32, 128, 8192, 33  # 33 x 8192 tokens x 32 heads x 128 x 2 B = 2.2 GB per tensor


def _randn(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)


def test_packed_beyond_2gib_equals_sequences_alone():
    total = NSEQ * L
    assert (total - L) * H * D * 2 >= 1 << 31  # the last sequence starts past 2 GiB
    print(f"[large packed] {NSEQ} x {L} tokens, H{H} d{D}, causal", flush=True)
    q, k, v, do = (_randn((total, H, D), 1000 + i) for i in range(4))
    cu = torch.arange(0, total + 1, L, dtype=torch.int32, device=DEV)
    o, lse = fa_varlen_fwd(q, k, v, cu, L, causal=True)
    dq, dk, dv = fa_varlen_bwd(do, q, k, v, o, lse, cu, L, causal=True)
    torch.cuda.synchronize()
    cu1 = torch.tensor([0, L], dtype=torch.int32, device=DEV)
    for s in (NSEQ - 2, NSEQ - 1):
        a, b = s * L, (s + 1) * L
        print(f"[large packed] sequence {s} alone (tokens {a}..{b - 1})", flush=True)
        qs, ks, vs, dos = (x[a:b].contiguous() for x in (q, k, v, do))
        os_, ls = fa_varlen_fwd(qs, ks, vs, cu1, L, causal=True)
        gs = fa_varlen_bwd(dos, qs, ks, vs, os_, ls, cu1, L, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], os_), f"O of sequence {s}"
        assert torch.equal(lse[:, a:b], ls), f"LSE of sequence {s}"
        for got, ref, n in zip((dq, dk, dv), gs, ("dQ", "dK", "dV")):
            assert torch.equal(got[a:b], ref), f"{n} of sequence {s}"
