"""A plain-Python model of the device-side GEMM schedules, checked for
coverage on the CPU: the tile builder (build_tiles_kernel) with tail tiles
(and 320-row ext tiles) and with the K-split of the last round, and the
block maps of tile_kernel_tail and tile_kernel_ksplit.  The model restates the index
arithmetic of those kernels; the GPU parity tests run the kernels
themselves.  Invariants: every output tile (m-tile x n-tile, or its K parts)
is produced by exactly one block; every grid block index decodes in range;
rows are covered once; the combine's K-part count per row matches the
tiles that were split."""
import numpy as np
import pytest

BM, GM, TAIL = 256, 8, 128
EXT = 320


def _segments(counts, shared):
    """Expert segments, then the shared expert's slices: shared = (T, slices),
    each slice one segment of T rows."""
    T, slices = shared
    offs = np.concatenate([[0], np.cumsum(counts)])
    segs = [(int(offs[e]), int(offs[e + 1])) for e in range(len(counts))]
    base = int(offs[-1])
    for j in range(slices):
        segs.append((base + j * T, base + (j + 1) * T))
    return segs


def _max_m(counts, shared, E):
    T, slices = shared
    return -(-(sum(counts) + T * slices) // BM) + E + slices


def cover(rows, ext=True, tail_rows=TAIL):
    """(main m-tiles, tail tiles) of one segment: 256-row tiles, except that
    a remainder of at most EXT - 256 rows joins the last full tile (ext) or
    one of at most tail_rows rows goes to a tail tile."""
    rem = rows % BM
    merge = ext and rows > BM and 0 < rem <= EXT - BM
    tail = 1 if not merge and 0 < rem <= tail_rows else 0
    nmain = rows // BM + (1 if rem > 0 and not tail and not merge else 0)
    return nmain, tail


def build_tail(counts, shared, ext=True):
    """Tiles and unit table of the schedule with tail tiles."""
    tiles, units = [], []
    for r0, r1 in _segments(counts, shared):
        nmain, tail = cover(r1 - r0, ext)
        nt = nmain + tail
        start, ustart = len(tiles), len(units)
        ng = 0 if nt == 0 else (1 if nmain == 0 else -(-nmain // GM))
        tl = [None] * nt
        units.extend([None] * (2 * nmain + tail))
        for c in range(ng):
            first, last = c * nmain // ng, (c + 1) * nmain // ng
            ht = tail if c == ng - 1 else 0
            for j in range(first, last + ht):
                tl[j] = (r0 + j * BM, r0 + (j + 1) * BM if j + 1 < nt else r1)
            d = (start + first, last - first, ht, ustart + 2 * first)
            for u in range(2 * (last - first) + ht):
                units[ustart + 2 * first + u] = d
        tiles += tl
    return tiles, units


def run_tail(counts, shared, n_tiles_n, nparts, E, ext=True):
    tiles, units = build_tail(counts, shared, ext)
    assert all(u is not None for u in units)
    max_m = _max_m(counts, shared, E)
    assert len(tiles) <= max_m and len(units) <= 2 * max_m
    half = n_tiles_n * nparts // 2
    blocks = 8 * -(-(2 * max_m * half) // 8)
    total = len(units) * half
    per = -(-total // 8)
    seen = set()
    for b in range(blocks):
        xcd, local = b & 7, b >> 3
        t = xcd * per + local
        if local >= per or t >= total:
            continue
        first, cnt, tail, first_unit = units[t // half]
        w = t - first_unit * half
        pair, r = divmod(w, 2 * cnt + tail)
        if r < 2 * cnt:
            kpart, n = divmod(2 * pair + r // cnt, n_tiles_n)
            keys = [(first + r % cnt, kpart, n)]
            r0, r1 = tiles[first + r % cnt]
            assert 0 < r1 - r0 <= (EXT if ext else BM)  # > 256 rows: the 320-row body
        else:
            kpart = 2 * pair // n_tiles_n
            n512 = (2 * pair - kpart * n_tiles_n) // 2
            keys = [(first + cnt, kpart, 2 * n512), (first + cnt, kpart, 2 * n512 + 1)]
            r0, r1 = tiles[first + cnt]
            assert 0 < r1 - r0 <= TAIL
        for k in keys:
            assert k not in seen
            seen.add(k)
    assert len(seen) == len(tiles) * nparts * n_tiles_n
    rows = np.zeros(sum(counts) + shared[0] * shared[1], int)
    for r0, r1 in tiles:
        rows[r0:r1] += 1
    assert (rows == 1).all()


def build_split(counts, shared, nn, ext=True):
    """Tiles (row0, row1, group) and the split of the K-split schedule (no
    tail tiles; ext tiles as in the tail schedule)."""
    tiles = []
    for r0, r1 in _segments(counts, shared):
        nt, _ = cover(r1 - r0, ext, tail_rows=0)
        start = len(tiles)
        ng = -(-nt // GM) if nt else 0
        for j in range(nt):
            c = 0
            while j >= (c + 1) * nt // ng:
                c += 1
            first, last = c * nt // ng, (c + 1) * nt // ng
            tiles.append((r0 + j * BM, r0 + (j + 1) * BM if j + 1 < nt else r1,
                          (start + first) * 256 + last - first))
    nt = len(tiles)
    rem = (nt * nn) % 256
    first = nt
    if rem > 0:
        first = tiles[nt - (rem + nn - 1) // nn][2] >> 8
    return tiles, nt - first, (tiles[first][0] if first < nt else 2 ** 31 - 1)


def _tile_at(t, m0, nn, tiles):
    grp = tiles[m0 + t // nn][2]
    first, cnt = grp >> 8, grp & 255
    w = t - (first - m0) * nn
    assert w >= 0
    return first + w % cnt, w // cnt


def run_split(counts, shared, nn, parts, E, ext=True):
    tiles, ns, split_row = build_split(counts, shared, nn, ext)
    for r0, r1, _ in tiles:
        assert 0 < r1 - r0 <= (EXT if ext else BM)
    nt = len(tiles)
    max_m = _max_m(counts, shared, E)
    blocks = 8 * (-(-(max_m * nn) // 8) + -(-(max_m * nn * parts) // 8))
    pos_a, pos_b = (nt - ns) * nn, ns * nn * parts
    per_a, per_b = -(-pos_a // 8), -(-pos_b // 8)
    seen = set()
    for b in range(blocks):
        xcd, local = b & 7, b >> 3
        if local < per_a:
            t = xcd * per_a + local
            if t >= pos_a:
                continue
            m, n = _tile_at(t, 0, nn, tiles)
            assert m < nt - ns
            key = (m, n, 0)
        elif local < per_a + per_b:
            t = xcd * per_b + local - per_a
            if t >= pos_b:
                continue
            m, n2 = _tile_at(t, nt - ns, nn * parts, tiles)
            assert m >= nt - ns
            key = (m, n2 % nn, n2 // nn)
        else:
            continue
        assert key not in seen
        seen.add(key)
    assert len(seen) == (nt - ns) * nn + ns * nn * parts
    for m, (r0, r1, _) in enumerate(tiles):
        for r in (r0, r1 - 1):  # the combine sums `parts` parts exactly for split rows
            assert (r >= split_row) == (m >= nt - ns)
    if 0 < ns < nt:
        assert pos_a <= 256 * -(-(nt * nn) // 256)


_RNG = np.random.default_rng(2)
_Z = 1.0 / np.arange(1, 129) ** 1.2
CASES = [
    ("mixtral", _RNG.multinomial(8192, [1 / 8] * 8), (4096, 0), 8),
    ("dsv3", _RNG.multinomial(65536, [1 / 256] * 256), (8192, 1), 256),
    ("dsv3_shared_2I", _RNG.multinomial(65536, [1 / 256] * 256), (8192, 2), 256),
    ("qwen_zipf", _RNG.multinomial(131072, _Z / _Z.sum()), (16384, 0), 128),
    ("edges", np.array([0, 1, 128, 129, 255, 256, 257, 384, 385, 512, 2053, 2248, 4096, 2404]),
     (300, 3), 14),
    ("many_groups", np.array([3000, 10, 0, 2600]), (2000, 0), 4),
    ("one_small_expert", np.array([100]), (100, 0), 1),
    ("empty", np.array([0, 0, 0]), (0, 0), 3),
]


@pytest.mark.parametrize("name,counts,shared,E", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("n_tiles_n,nparts", [(2, 1), (16, 4), (28, 2), (112, 1)])
@pytest.mark.parametrize("ext", [True, False], ids=["ext", "no_ext"])
def test_tail_schedule_covers_every_tile_once(name, counts, shared, E, n_tiles_n, nparts, ext):
    run_tail(counts, shared, n_tiles_n, nparts, E, ext)


@pytest.mark.parametrize("name,counts,shared,E", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("nn,parts", [(1, 2), (2, 2), (16, 4), (28, 2)])
@pytest.mark.parametrize("ext", [True, False], ids=["ext", "no_ext"])
def test_ksplit_schedule_covers_every_tile_once(name, counts, shared, E, nn, parts, ext):
    run_split(counts, shared, nn, parts, E, ext)


def test_cover_tile_heights():
    """Every tile but the segment's last is a full 256-row tile; the last is
    a 1-256-row tile, a 257-320-row ext tile (a full tile plus a remainder
    of at most 64 rows) or a 1-128-row tail tile; never more
    tiles than 256-row tiles alone would need."""
    for rows in range(0, 3000):
        for ext in (True, False):
            nmain, tail = cover(rows, ext)
            nt = nmain + tail
            assert nt <= -(-rows // BM) and 2 * nmain + tail <= 2 * -(-rows // BM)
            if rows == 0:
                assert nt == 0
                continue
            last = rows - BM * (nt - 1)
            assert 0 < last
            if tail:
                assert last <= TAIL
            elif last > BM:
                assert ext and last <= EXT and (rows % BM) <= EXT - BM
