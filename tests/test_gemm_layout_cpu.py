"""CPU check of the transposed-operand LDS layout of the deterministic GEMM
(csrc/det_gemm.hip): a slice of 64 contraction rows x kT values, chunk c of
row r at position c ^ h(r), h(r) = 2 ((r & 3) | ((r >> 3) & 1) << 2), filled
by direct loads (load j of loader wave w writes 1 KB, lane i taking row
kRpl (kL w + j) + i / kCpr and position i % kCpr) and read with
ds_read_b64_tr_b16 (in each 16-lane group, lane i gets element j of the
4-element block addressed by lane 4 j + i / 4, at position i % 4).

Checked: every (row, chunk) of a slice is loaded exactly once; each lane of a
16 x 16 x 32 operand fragment receives its own column and contraction values
8 (l / 16) + 4 t .. + 3 for the two reads t; the 32 lanes of each half of a
read touch 8 distinct 32-byte bank slots; and h(row) depends on the row only
through lane bits, so fragment offsets are fixed for the whole product.  The
GPU tests check the kernel itself against the oracle."""

import pytest


def h(row):
    return 2 * ((row & 3) | (((row >> 3) & 1) << 2))


@pytest.mark.parametrize("kT", [256, 128])
def test_transposed_slice_layout(kT):
    row_bytes = kT * 2
    cpr = kT // 8                      # 16-byte chunks per row
    rpl = 1024 // row_bytes            # rows per 1 KB load
    loads = kT * 64 * 2 // (4 * 1024)  # loads per loader wave (4 loader waves)
    where = {}
    for w in range(4):
        for j in range(loads):
            for lane in range(64):
                row = rpl * (w * loads + j) + lane // cpr
                pos = lane % cpr
                chunk = pos ^ h(row)
                assert 0 <= chunk < cpr
                lds = (w * loads + j) * 1024 + lane * 16
                assert lds == row * row_bytes + pos * 16
                assert (row, chunk) not in where
                where[(row, chunk)] = lds
    assert len(where) == 64 * cpr                       # every chunk exactly once

    for m in range(kT // 16):                           # 16-column fragment m
        for u in range(2):                              # 32-wide step of the stage
            for t in range(2):                          # the two reads of a fragment
                addr = {}
                for lane in range(64):
                    g, a = lane // 16, lane % 16
                    row = 32 * u + 8 * g + 4 * t + a // 4
                    col = 16 * m + 4 * (a % 4)
                    assert h(row) == h(8 * g + a // 4)   # lane-constant swizzle
                    pos = (col // 8) ^ h(row)
                    addr[lane] = (row, col, row * row_bytes + pos * 16 + (col % 8) * 2)
                    assert where[(row, col // 8)] == row * row_bytes + pos * 16
                for half in range(2):
                    slots = {addr[l][2] % 256 // 32 for l in range(32 * half, 32 * half + 32)}
                    assert len(slots) == 8                # no bank conflict
                for lane in range(64):
                    g, i = lane // 16, lane % 16
                    for jj in range(4):
                        src = 16 * g + 4 * jj + i // 4
                        r, c, _ = addr[src]
                        assert c + i % 4 == 16 * m + i            # the lane's own column
                        assert r == 32 * u + 8 * g + 4 * t + jj   # its contraction values
