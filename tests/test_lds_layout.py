"""CPU model of the XOR-swizzled LDS tiles used by the bf16 forward (ping-pong
kernel) and the backward kernels: 64 rows x d bf16, no padding, 16-byte chunk
c of row r stored at chunk c ^ swz(r).

Checked here, for d = 64 and d = 128:
  * the LDS DMA fill (lane l of 1 KB block q loads logical chunk
    (l % (d/8)) ^ swz(row) of row (512/d) q + l / (d/8)) writes every element of
    the tile exactly once, at its swizzled place;
  * the K fragment reads at (base ^ 16 kk) + 32 kb d return the 8 elements
    row 32 kb + (lane % 32), columns 16 kk + 8 (lane / 32) ...;
  * the transposed V reads at (base_half ^ 32 db) + 16 cc d return the same
    4 elements as the unswizzled layout would;
  * 16-lane passes of the 16-byte K reads and 32-lane passes of the 8-byte
    transposed reads touch 64 distinct 4-byte banks (no bank conflict).
The swizzle and offsets restate exact_attention_24_amd/csrc/fa_device.h
(swz, swz_off, tr_off) and the addressing of fwd_bf16_pp_kernel.
"""

import numpy as np
import pytest

BC = 64


def swz(d, row):
    if d == 128:
        return 4 * (row & 3) + ((row >> 2) & 3)
    return 4 * ((row >> 1) & 1) + ((row >> 2) & 1) + 2 * ((row >> 3) & 1)


def swz_off(d, row, chunk):
    return row * d + ((chunk ^ swz(d, row)) << 3)


def tr_off(d, lane, db, half):
    row = 8 * half + 4 * (lane >> 5) + ((lane & 15) >> 2)
    chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
    return swz_off(d, row, chunk) + 4 * (lane & 1)


def dma_fill(d):
    """LDS contents (logical element ids) after the DMA blocks of one tile."""
    ts = BC * d
    tile = np.arange(ts).reshape(BC, d)
    lds = -np.ones(ts, dtype=np.int64)
    rows_per_block, chunks = 512 // d, d // 8
    for q in range(ts * 2 // 1024):
        for lane in range(64):
            r = rows_per_block * q + lane // chunks
            lc = (lane % chunks) ^ swz(d, r)
            dst = q * 512 + 8 * lane
            lds[dst:dst + 8] = tile[r, lc * 8:lc * 8 + 8]
    return tile, lds


def k_addr(d, lane, kb, kk):
    ql, hf = lane & 31, lane >> 5
    return ((ql * d + 8 * (swz(d, ql) ^ hf)) ^ (16 * kk)) + 32 * kb * d


def v_addr(d, lane, cc, db, half):
    return (tr_off(d, lane, 0, half) ^ (32 * db)) + 16 * cc * d


@pytest.mark.parametrize("d", [64, 128])
def test_dma_fill_is_the_swizzled_tile(d):
    tile, lds = dma_fill(d)
    assert (lds >= 0).all() and np.unique(lds).size == lds.size
    for r in range(BC):
        for c in range(d // 8):
            o = swz_off(d, r, c)
            assert (lds[o:o + 8] == tile[r, 8 * c:8 * c + 8]).all()


@pytest.mark.parametrize("d", [64, 128])
def test_k_fragment_addresses(d):
    tile, lds = dma_fill(d)
    for lane in range(64):
        ql, hf = lane & 31, lane >> 5
        for kb in range(2):
            for kk in range(d // 16):
                a = k_addr(d, lane, kb, kk)
                col = 16 * kk + 8 * hf
                assert (lds[a:a + 8] == tile[32 * kb + ql, col:col + 8]).all()


@pytest.mark.parametrize("d", [64, 128])
def test_v_transposed_addresses(d):
    tile, lds = dma_fill(d)
    for lane in range(64):
        for half in range(2):
            for db in range(d // 32):
                for cc in range(4):
                    a = v_addr(d, lane, cc, db, half)
                    assert a == tr_off(d, lane, db, half) + 16 * cc * d
                    row = 16 * cc + 8 * half + 4 * (lane >> 5) + ((lane & 15) >> 2)
                    col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
                    assert (lds[a:a + 4] == tile[row, col:col + 4]).all()


def _banks(byte_addr, nbytes):
    return [(byte_addr // 4 + i) % 64 for i in range(nbytes // 4)]


@pytest.mark.parametrize("d", [64, 128])
def test_reads_are_bank_conflict_free(d):
    for kb in range(2):
        for kk in range(d // 16):
            for p0 in range(0, 64, 16):
                banks = [b for lane in range(p0, p0 + 16) for b in _banks(2 * k_addr(d, lane, kb, kk), 16)]
                assert sorted(banks) == list(range(64)), (kb, kk, p0)
    for cc in range(4):
        for db in range(d // 32):
            for half in range(2):
                for p0 in (0, 32):
                    banks = [b for lane in range(p0, p0 + 32) for b in _banks(2 * v_addr(d, lane, cc, db, half), 8)]
                    assert sorted(banks) == list(range(64)), (cc, db, half, p0)


def test_a_wrong_swizzle_is_caught():
    """The checks above are not vacuous: without the swizzle the 16-row K
    reads of d = 128 all start in the same bank group."""
    banks = set()
    for lane in range(16):
        banks.add(((lane & 31) * 128 * 2 // 16) % 16)
    assert len(banks) < 16
