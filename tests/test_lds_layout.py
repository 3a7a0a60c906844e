"""Host checks of the LDS tile layout that the direct-to-LDS kernels share (MomentKV alpha,
score round and pool score, the K-means assignment): rows of P 16-byte pieces, piece q of row
r stored at position q ^ f(r), with f(r) = r & 15 for P = 16 and (r >> 1) & 7 for P = 8.

The layout must be a permutation within every row (each piece stored once), and the operand
reads of 16 consecutive rows at one piece column must fall in 16 distinct 16-byte bank groups
(the LDS serves 64 four-byte banks, i.e. 16 such groups, per cycle), so that they meet no bank
conflicts.  The load side writes piece i*64 + lane of a tile for lane `lane` of load i, which
must cover every (row, piece) of the tile exactly once."""
import pytest


def swz(P, r):
    return (r & 15) if P == 16 else ((r >> 1) & 7)


@pytest.mark.parametrize("P", [8, 16])
def test_rows_are_permuted(P):
    for r in range(256):
        assert sorted(q ^ swz(P, r) for q in range(P)) == list(range(P))


@pytest.mark.parametrize("P", [8, 16])
def test_column_reads_are_conflict_free(P):
    for r0 in range(0, 256, 16):
        for piece in range(P):
            groups = [((r0 + i) * P + (piece ^ swz(P, r0 + i))) % 16 for i in range(16)]
            assert len(set(groups)) == 16, (P, r0, piece, groups)


@pytest.mark.parametrize("P,rows", [(16, 32), (8, 32), (16, 128), (8, 128), (8, 96)])
def test_loads_cover_the_tile_once(P, rows):
    seen = set()
    for i in range(rows * P // 64):          # 1 KB loads
        for lane in range(64):
            sl = i * 64 + lane
            r, q = sl // P, sl % P
            seen.add((r, q ^ swz(P, r)))      # the global piece this lane fetches
    assert seen == {(r, q) for r in range(rows) for q in range(P)}
