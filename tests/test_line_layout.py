"""The MFMA tiles' whole-line load layout, checked as index arithmetic.

v_mfma_f32_16x16x32_bf16 takes, in lane l, 16 bytes of row l%16 of a 16-row
tile (K group l/16). The kernel instead loads whole 128-byte lines: X holds
rows 0-7 and Y rows 8-15, lane l reading chunk c(l) of row l%8, and a
rotation by 8 lanes within each 16-lane row (DPP row_ror:8) followed by a
per-lane select turns X, Y into the two operands of the tile's two MFMAs.
These tests restate that arithmetic (moedecode.hip: line_row, line_chunk4,
line_chunk2, lines_to_operands) and check that every lane ends up with the
operand-order (row, chunk) pairs, and that each load instruction reads whole
lines.
"""
import itertools


def row_ror8(values):
    """DPP row_ror:8 over a wave: lane s of each 16-lane row reads lane (s + 8) % 16."""
    return [values[(l & ~15) | (((l & 15) + 8) & 15)] for l in range(64)]


def lines_to_operands(X, Y):
    xr, yr = row_ror8(X), row_ror8(Y)
    lo = [(l & 8) == 0 for l in range(64)]
    a = [X[l] if lo[l] else yr[l] for l in range(64)]
    b = [xr[l] if lo[l] else Y[l] for l in range(64)]
    return a, b


def chunk4(l):
    return (l >> 4) + 4 * ((l >> 3) & 1)


def chunk2(l):
    return 2 * (l >> 4) + ((l >> 3) & 1)


def line_loads(chunk):
    """(row, chunk) each lane loads for X (rows 0-7) and Y (rows 8-15)."""
    X = [(l & 7, chunk(l)) for l in range(64)]
    Y = [(8 + (l & 7), chunk(l)) for l in range(64)]
    return X, Y


def test_loads_read_whole_lines():
    for chunk in (chunk4, chunk2):
        for half in line_loads(chunk):
            by_row = {}
            for row, c in half:
                by_row.setdefault(row, set()).add(c)
            assert len(by_row) == 8
            assert all(cs == set(range(8)) for cs in by_row.values())  # 8 lanes x 16 B = the row's 128 B


def test_chunk4_gives_operand_chunks_kq_and_4_plus_kq():
    a, b = lines_to_operands(*line_loads(chunk4))
    for l in range(64):
        kq, s = l >> 4, l & 15
        assert a[l] == (s, kq)
        assert b[l] == (s, 4 + kq)


def test_chunk2_gives_operand_chunks_2kq_and_2kq_plus_1():
    a, b = lines_to_operands(*line_loads(chunk2))
    for l in range(64):
        kq, s = l >> 4, l & 15
        assert a[l] == (s, 2 * kq)
        assert b[l] == (s, 2 * kq + 1)


def test_operands_form_the_same_product():
    """With operand a from the weights' line and the activation's in the same
    layout, the K index lane (kq, s) contributes is the same on both sides,
    so the two MFMAs sum every (row, column) product exactly once."""
    wa, wb = lines_to_operands(*line_loads(chunk4))
    xa, xb = lines_to_operands(*line_loads(chunk4))
    seen = set()
    for mf, (w, x) in enumerate(((wa, xa), (wb, xb))):
        for kq, s, t in itertools.product(range(4), range(16), range(16)):
            wrow, wch = w[16 * kq + s]   # A: lane (kq, s) holds row s
            trow, tch = x[16 * kq + t]   # B: lane (kq, t) holds token t
            assert wrow == s and trow == t and wch == tch
            for e in range(8):           # the chunk's 8 bf16 columns
                seen.add((s, t, 8 * wch + e))
    assert len(seen) == 16 * 16 * 64     # every row x token pair over all 64 columns, once
