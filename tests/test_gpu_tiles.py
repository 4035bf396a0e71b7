"""GPU parity of the forward for every query-tile size the launch table picks.

The tile size adapts to the input ("动态调整 tile size" in the FA-3 paragraph of
"Flash-Attention 2/3在ms-swift中的集成与性能提升"): bf16 calls take 256 query
rows per work-group when that launch has a unit of work per CU (256 on
MI355X; a causal dense unit is a pair of tiles); below that, short causal
calls without a window or dropout (at most 2048 rows, at most 4 blocks of 32
rows per CU) take 32-row work-groups whose 4 waves split the keys; else 128
rows if that gives a work-group per CU, else 64.  Each case below lands on
one of the choices (the rule is restated here only to label the cases) and is
checked element by element against the oracle, with and without dropout.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_attention_24_amd import fa_fwd
from exact_attention_24_amd.inputs import dense_inputs
from tests.parity import assert_close, assert_lse_close, f64, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CUS = 256


def _tile(bh, nq, causal, window, p):
    t256 = -(-nq // 256)
    if bh * ((t256 + 1) // 2 if causal else t256) >= CUS:
        return 256
    if causal and window == 0 and p == 0 and nq <= 2048 and bh * -(-nq // 32) <= 4 * CUS:
        return 32
    return 128 if bh * -(-nq // 128) >= CUS else 64


CASES = [
    # (batch, n, heads, d, causal, window, dropout_p, expected tile)
    (1, 300, 2, 128, True, 0, 0.0, 32),
    (1, 300, 2, 64, False, 77, 0.0, 64),
    (1, 257, 3, 128, True, 0, 0.2, 64),
    (2, 1024, 16, 64, True, 0, 0.0, 32),      # the MindSpore API example shape
    (2, 1024, 16, 128, True, 0, 0.0, 32),
    (1, 2048, 2, 128, True, 0, 0.0, 32),      # the longest split-key call
    (1, 2049, 1, 64, True, 0, 0.0, 64),       # one row past it
    (3, 1000, 5, 64, True, 0, 0.0, 32),
    (4, 700, 16, 128, False, 0, 0.0, 128),
    (4, 700, 16, 128, True, 150, 0.1, 128),
    (1, 1024, 64, 128, True, 0, 0.0, 128),    # causal: too few tile pairs for 256 rows
    (1, 1024, 128, 128, True, 0, 0.0, 256),
    (1, 1024, 64, 64, False, 200, 0.0, 256),
]


@pytest.mark.parametrize("b,n,h,d,causal,window,p,tile", CASES)
def test_forward_every_tile_size(b, n, h, d, causal, window, p, tile):
    assert _tile(b * h, n, causal, window, p) == tile
    print(f"[tiles] tile={tile} b={b} n={n} h={h} d={d} causal={causal} window={window} p={p}", flush=True)
    q, k, v = dense_inputs(b, n, h, d, "bf16", seed=n + h + d + tile)
    if p:  # kept weights grow by 1 / (1 - p): keep |O| < 4, where a bf16 output is within 1e-2
        v = (v.float() * 0.5).to(v.dtype)
    kw = dict(dropout_p=p, seed=77 + n, offset=2) if p else {}
    o, lse = fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal, window=window, **kw)
    torch.cuda.synchronize()
    sc = 1 / np.sqrt(d)
    q64, k64, v64, o64, l64 = f64(q), f64(k), f64(v), f64(o), f64(lse)
    heads = [(bi, hh) for bi in range(b) for hh in range(h)]
    if len(heads) > 6:
        heads = [heads[0], heads[len(heads) // 3], heads[len(heads) // 2], heads[-1]]
    for bi, hh in heads:
        rows = np.arange(n) if n <= 300 else sample_rows(n, 64, seed=bi * 100 + hh)
        rows = np.union1d(rows, [r for r in (63, 64, 127, 128, 255, 256) if r < n])
        drop = oracle.dropout_keep(bi * h + hh, rows, n, 77 + n, 2, p) if p else None
        ro, rl = oracle.attention_fwd(q64[bi, rows, hh], k64[bi, :, hh], v64[bi, :, hh], sc, causal, window,
                                      q_pos=rows, nq=n, drop=drop)
        assert_close(o64[bi, rows, hh], ro, what=f"O batch {bi} head {hh}")
        assert_lse_close(l64[bi, hh, rows], rl)
