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


@pytest.mark.parametrize("kVi,kTj,esz", [(8, 4, 2), (8, 4, 4), (4, 2, 2), (4, 2, 4)])
def test_store_epilogue_layout(kVi, kTj, esz):
    """The GEMM's store epilogue through LDS (det_gemm.hip): per pass, the waves
    holding the pass's rows write each accumulator's four values to row q, byte
    p * esz of the staging layout (16-byte chunk c of row r at position
    c ^ (r & swz) inside buffer r // rows_per_buffer); every wave then reads 16
    bytes per lane, lanes of one row taking its consecutive chunks.  Checked:
    every staging byte of a pass is written exactly once and stays inside the
    two stage buffers; the reads cover every (row, chunk) of the pass exactly
    once and find there the values of output row q0 + row, columns
    p0 + 16 c / esz .. + 16 / esz - 1; each read instruction covers whole rows."""
    kTP, kTQ = 32 * kVi, 64 * kTj
    slot_bytes = (kTP * 64 * 2) + (kTQ * 64 * 2)        # X slice + Y slice of a stage
    row_b = kTP * esz
    C = row_b // 16
    Rs = slot_bytes // row_b
    PR = min(2 * Rs, kTQ)
    passes = kTQ // PR
    wave_rows = 16 * kTj
    rpi = 64 // C
    reads = PR // 8 // rpi
    swzm = C - 1 if C < 32 else 31
    assert C <= 64 and 64 % C == 0 and PR % wave_rows == 0 and PR % (8 * rpi) == 0

    def lds_at(row, byte):
        r = row % Rs
        base = 0 if row < Rs else slot_bytes
        return base + r * row_b + (((byte >> 4) ^ (r & swzm)) << 4) + (byte & 15)

    covered_q = set()
    for ps in range(passes):
        row_lo = ps * PR
        owner = {}
        for wave in range(8):
            wv, wt = wave & 1, wave >> 1
            if not (row_lo <= wt * wave_rows < row_lo + PR):
                continue
            for lane in range(64):
                lr, lg = lane & 15, lane >> 4
                for tj in range(kTj):
                    for vi in range(kVi):
                        row = wt * wave_rows + tj * 16 + lr - row_lo
                        p = wv * 16 * kVi + vi * 16 + 4 * lg
                        for i in range(4):
                            for b in range(esz):
                                a = lds_at(row, (p + i) * esz + b)
                                assert 0 <= a < 2 * slot_bytes
                                assert a not in owner
                                owner[a] = (row_lo + row, p + i)      # (q, p) of the value
        assert len(owner) == PR * row_b
        seen = set()
        for wave in range(8):
            for k in range(reads):
                rows_here = set()
                for lane in range(64):
                    row = wave * (PR // 8) + k * rpi + lane // C
                    c = lane % C
                    rows_here.add(row)
                    assert (row, c) not in seen
                    seen.add((row, c))
                    for b in range(16):
                        q, p = owner[lds_at(row, c * 16 + b)]
                        assert q == row_lo + row and p == c * (16 // esz) + b // esz
                    covered_q.add(row_lo + row)
                assert len(rows_here) == rpi                 # whole rows per instruction
        assert len(seen) == PR * C
    assert covered_q == set(range(kTQ))
