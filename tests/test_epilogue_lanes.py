"""Host-side checks of the lane arithmetic of the direct epilogues
(csrc/epilogue.hpp), emulated in Python: the two quad-permuting DPP steps
form a 4 x 4 transpose across each group of four lanes, and the per-lane
8-byte store offsets of the tiled and mirrored writes land exactly on the
tiled layout's element offsets (tiled.hpp), covering every element of a
wavefront's 128 x 128 quarter once. The GPU tests check the same code end to
end against the oracle; these pin the index maps on any machine."""
import itertools

import numpy as np


def t32_swz(r):
    return ((r >> 1) ^ (r >> 2)) & 3


def t32_off(i, k, cp):
    """Element offset of (i, k) in the tiled layout of padded width cp: 32 x 32
    blocks of 1024 elements, 16-byte chunks of a block row XOR-permuted."""
    return ((((i >> 5) * (cp >> 5)) + (k >> 5)) << 10) + ((i & 31) << 5) + \
        ((((k >> 3) & 3) ^ t32_swz(i & 31)) << 3) + (k & 7)


def dpp_quad(vals, perm):
    """v_mov_b32_dpp quad_perm: lane 4a + b reads lane 4a + perm[b]."""
    return [vals[4 * (l // 4) + perm[l % 4]] for l in range(len(vals))]


XOR1, XOR2 = (1, 0, 3, 2), (2, 3, 0, 1)


def quad_transpose(x, q):
    """The kernel's butterfly on a wavefront: x[lane] = [x0, x1, x2, x3]."""
    n = len(x)
    b1 = [(q[l] & 1) != 0 for l in range(n)]
    b2 = [(q[l] & 2) != 0 for l in range(n)]
    r0 = dpp_quad([x[l][0] if b1[l] else x[l][1] for l in range(n)], XOR1)
    r1 = dpp_quad([x[l][2] if b1[l] else x[l][3] for l in range(n)], XOR1)
    nn = [[r0[l] if b1[l] else x[l][0], x[l][1] if b1[l] else r0[l],
           r1[l] if b1[l] else x[l][2], x[l][3] if b1[l] else r1[l]] for l in range(n)]
    s0 = dpp_quad([nn[l][0] if b2[l] else nn[l][2] for l in range(n)], XOR2)
    s1 = dpp_quad([nn[l][1] if b2[l] else nn[l][3] for l in range(n)], XOR2)
    return [[s0[l] if b2[l] else nn[l][0], s1[l] if b2[l] else nn[l][1],
             nn[l][2] if b2[l] else s0[l], nn[l][3] if b2[l] else s1[l]] for l in range(n)]


def mfma_rows(lane, g):
    """Rows of a 32 x 32 MFMA block a lane holds in accumulator group g
    (elements 4 g .. 4 g + 3), and its column."""
    h, c = lane >> 5, lane & 31
    return [8 * g + 4 * h + i for i in range(4)], c


def test_quad_transpose_is_a_transpose():
    lanes = list(range(64))
    q = [l & 3 for l in lanes]
    for g in range(4):
        # value of (row, col) of the block: a unique tag
        x = []
        for l in lanes:
            rows, c = mfma_rows(l, g)
            x.append([(r, c) for r in rows])
        y = quad_transpose(x, q)
        for l in lanes:
            h, r32 = l >> 5, l & 31
            qq, k = r32 & 3, r32 >> 2
            row = 8 * g + 4 * h + qq
            assert y[l] == [(row, 4 * k + e) for e in range(4)], (l, g)


def test_direct_tiled_offsets_cover_the_quarter_once():
    cp = 1280  # padded width: five 256-wide tile columns
    m0, n0 = 256, 512
    for wave in range(4):
        wm, wn = wave >> 1, wave & 1
        seen = set()
        for lane in range(64):
            h, r32 = lane >> 5, lane & 31
            q, k = r32 & 3, r32 >> 2
            base = (((m0 >> 5) + wm * 4) * (cp >> 5) + (n0 >> 5) + wn * 4) << 10
            for I, j, g in itertools.product(range(4), range(4), range(4)):
                r = 8 * g + 4 * h + q
                inner = r * 32 + (((k >> 1) ^ t32_swz(r)) << 3) + 4 * (k & 1)
                off = base + ((I * (cp >> 5) + j) << 10) + inner
                row = m0 + wm * 128 + I * 32 + r
                col = n0 + wn * 128 + j * 32 + 4 * k
                for e in range(4):
                    assert t32_off(row, col + e, cp) == off + e
                    seen.add((row, col + e))
        assert len(seen) == 128 * 128


def test_mirror_offsets_are_the_transposed_positions():
    cp = 1024
    m0, n0 = 512, 256  # a tile below the diagonal
    for wave in range(4):
        wm, wn = wave >> 1, wave & 1
        bi0, bj0 = (m0 >> 5) + wm * 4, (n0 >> 5) + wn * 4
        seen = set()
        for lane in range(64):
            h, r32 = lane >> 5, lane & 31
            for I, j, g in itertools.product(range(4), range(4), range(4)):
                innm = r32 * 32 + ((g ^ t32_swz(r32)) << 3) + 4 * h
                off = (((bj0 + j) * (cp >> 5) + bi0 + I) << 10) + innm
                rows, c = mfma_rows(lane, g)
                for e, r in enumerate(rows):
                    # element (row, col) of the product goes to (col, row)
                    row = m0 + wm * 128 + I * 32 + r
                    col = n0 + wn * 128 + j * 32 + c
                    assert t32_off(col, row, cp) == off + e
                    seen.add((col, row))
        assert len(seen) == 128 * 128


def test_diagonal_block_split_is_exact():
    """A diagonal 32 x 32 block: the transposed values keep row >= column, the
    mirror writes column > row, so every element is written exactly once."""
    count = np.zeros((32, 32), dtype=int)
    for lane in range(64):
        h, r32 = lane >> 5, lane & 31
        q, k = r32 & 3, r32 >> 2
        for g in range(4):
            r = 8 * g + 4 * h + q
            for e in range(4):
                if r >= 4 * k + e:
                    count[r, 4 * k + e] += 1          # from D
            c0 = 8 * g + 4 * h
            for i in range(4):
                if c0 + i > r32:
                    count[r32, c0 + i] += 1           # from the mirror
    assert np.all(count == 1)
