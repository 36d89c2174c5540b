"""The grouped matmuls' local group table, replayed on the host.

Every gmm / tgmm workgroup builds its table from the caller's group_sizes
(device data, unchecked): negative sizes count as 0, the row offsets are a
64-bit exclusive scan saturated at the row bound, and each group owns a
number of tiles.  This replays that arithmetic with the device's integer
widths (int32 table entries, 64-bit running sums) and checks that no row or
tile of any table leaves the buffer, whatever the sizes -- including sizes
whose sum passes 2^31, where a 32-bit running sum wraps."""

import numpy as np
import pytest

import moe_fp8_grouped_amd as m

I32 = np.iinfo(np.int32)


XROWS = 16     # rows an absorbing row block may carry past bm/2


def group_tiles(mr, bm, nt, mode):
    """mode 0 plain tiles, 1 wide tails, 2 every tile wide (bm/2 rows x two
    n-tiles), 3 every tile wide with absorbing row blocks (up to bm/2 + 16
    rows each)."""
    if nt <= 0:
        return 1
    if mode == 2:
        return -(-mr // (bm // 2)) * (nt // 2) + (nt & 1) * -(-mr // bm)
    if mode == 3:
        return -(-mr // (bm // 2 + XROWS)) * (nt // 2) + (nt & 1) * -(-mr // bm)
    full, rem = mr // bm, mr % bm
    if mode == 0 or rem == 0 or rem > bm // 2:
        return (full + (1 if rem else 0)) * nt
    return (nt // 2) * (2 * full + 1) + (nt & 1) * (full + 1)


def build_groups(sizes, max_rows, nt, bm, wide_tail):
    """The table as the device builds it: (rows_off, tiles_off, rows flag, size flag)."""
    v = np.asarray(sizes, np.int64)
    neg = bool((v < 0).any())
    v = np.maximum(v, 0)
    incl = np.cumsum(v)                                   # 64-bit: at most 1024 * 2^31
    rows_off = np.minimum(np.concatenate([[0], incl]), max_rows).astype(np.int32)
    over = bool(incl[-1] > max_rows) if v.size else False
    rows = np.diff(rows_off.astype(np.int64))
    tiles = np.array([group_tiles(int(r), bm, nt, wide_tail) for r in rows], np.int64)
    tiles_off = np.concatenate([[0], np.cumsum(tiles)])
    assert tiles_off[-1] <= I32.max, "the host bound keeps the tile count in int32"
    return rows_off, tiles_off.astype(np.int32), over, neg


def wrapping_rows_off(sizes):
    """A 32-bit running sum, for contrast: it wraps past 2^31."""
    v = np.maximum(np.asarray(sizes, np.int64), 0)
    s = np.concatenate([[0], np.cumsum(v)])
    return ((s + 2 ** 31) % 2 ** 32 - 2 ** 31).astype(np.int64)


CASES = [
    [1 << 30] * 3,
    [I32.max] * 1024,
    [5, -7, 2 ** 31 - 1, 3],
    [0] * 64,
    [300, 0, 1, 129, 256, 384],
    list(np.random.default_rng(0).integers(-10, 2 ** 31 - 1, 1024)),
]


@pytest.mark.parametrize("sizes", CASES)
@pytest.mark.parametrize("max_rows,nt,bm,wide", [(1000, 2, 256, 1), (8192, 32, 256, 1), (8192, 33, 256, 2),
                                                 (8192, 33, 256, 3), (1000, 4, 256, 3),
                                                 (40960, 1, 128, 0), (2 ** 31 - 2, 16, 256, 0)])
def test_table_stays_inside_the_buffer(sizes, max_rows, nt, bm, wide):
    if (max_rows // 128 + len(sizes) + 1) * nt > I32.max:
        pytest.skip("rejected by the host's tile-count bound")
    rows_off, tiles_off, over, neg = build_groups(sizes, max_rows, nt, bm, wide)
    assert rows_off[0] == 0 and (np.diff(rows_off) >= 0).all() and rows_off[-1] <= max_rows
    v = np.maximum(np.asarray(sizes, np.int64), 0)
    assert rows_off[-1] == min(int(v.sum()), max_rows)
    assert over == (int(v.sum()) > max_rows)
    assert neg == any(x < 0 for x in sizes)
    # every tile's rows lie inside [0, max_rows): a group's tiles cover its rows only
    for g in range(len(sizes)):
        r0, r1 = int(rows_off[g]), int(rows_off[g + 1])
        assert 0 <= r0 <= r1 <= max_rows
        assert tiles_off[g + 1] - tiles_off[g] == group_tiles(r1 - r0, bm, nt, wide)
    if wide >= 2 and len(sizes) <= 64:
        # the all-wide decode: tile -> (n-tile, first row, rows) covers every (row, n-tile) of each group once
        for g in range(len(sizes)):
            m_g = int(rows_off[g + 1] - rows_off[g])
            if m_g > 4096:
                continue
            check_wide_cover(m_g, nt, bm, wide, int(tiles_off[g + 1] - tiles_off[g]))


def wide_decode(local, m_g, nt, bm, mode):
    """(first row, rows, n-tiles) of tile `local` of a group, as the kernel decodes it."""
    half, npair = bm // 2, nt // 2
    mtw = -(-m_g // (half + XROWS)) if mode == 3 else -(-m_g // half)
    xr = max(m_g - half * mtw, 0) if mode == 3 else 0
    if local < npair * mtw:
        pr, mb = local // mtw, local % mtw
        roff = mb * half + min(XROWS * mb, xr)
        if mode == 3:
            nxt = (mb + 1) * half + min(XROWS * (mb + 1), xr) if mb + 1 < mtw else m_g
            rows = nxt - roff
        else:
            rows = min(half, m_g - roff)
        return roff, rows, (2 * pr, 2 * pr + 1)
    roff = (local - npair * mtw) * bm
    return roff, min(bm, m_g - roff), (nt - 1,)


def check_wide_cover(m_g, nt, bm, mode, ntiles):
    cover = np.zeros((max(m_g, 1), nt), np.int64)
    for local in range(ntiles):
        roff, rows, nts = wide_decode(local, m_g, nt, bm, mode)
        assert rows > 0 and roff + rows <= m_g
        limit = bm // 2 + (XROWS if mode == 3 else 0) if len(nts) == 2 else bm
        assert rows <= limit, (m_g, local, rows)
        for j in nts:
            cover[roff:roff + rows, j] += 1
    assert m_g == 0 or (cover == 1).all()


@pytest.mark.parametrize("nt", [2, 3, 32, 56])
def test_absorbing_blocks_cover_every_row_once(nt):
    """Every group size up to 1200 rows: the absorbing decode covers each
    (row, n-tile) once, no wide tile exceeds 144 rows, and it never needs more
    tiles than the plain all-wide decode (fewer when up to 16 rows per block
    spill past a multiple of 128)."""
    for m_g in range(0, 1201):
        t3, t2 = group_tiles(m_g, 256, nt, 3), group_tiles(m_g, 256, nt, 2)
        assert t3 <= t2
        check_wide_cover(m_g, nt, 256, 3, t3)
    # the expert-slice case: 257..288 rows take two row blocks, not three
    assert group_tiles(285, 256, 32, 3) == 2 * 16 and group_tiles(285, 256, 32, 2) == 3 * 16
    assert group_tiles(289, 256, 32, 3) == 3 * 16


def test_a_32_bit_running_sum_would_leave_the_buffer():
    """Why the scan is 64-bit and saturating: with [2^30] * 3 a 32-bit running
    sum makes group 2 start at -2^31 and ends the table below zero."""
    off = wrapping_rows_off([1 << 30] * 3)
    assert off[2] < 0 and off[3] < 0
    rows_off, _, over, _ = build_groups([1 << 30] * 3, 1000, 2, 256, 1)
    assert list(rows_off) == [0, 1000, 1000, 1000] and over


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmoefp8.so not built")
    return m.load_library()


def test_gmm_rejects_tile_tables_past_int32(lib):
    """The host bound that keeps the table's tile count in int32."""
    one = 1
    M, N, K = 2 ** 31 - 2, 128 * 1024, 128
    st = lib.moe_gmm_fp8(one, one, 0, one, one, 1, N, 1, one, 8, 0, 8, M, K, N, 0, one, one, 256, None)
    assert st == m.MOE_ERR_SHAPE


def absorb_decision(sizes, nt, workgroups=256, bm=256):
    """The kernel's per-launch choice: absorbing row blocks only when they
    take fewer rounds of tiles over an XCD's workgroups than plain wide tiles."""
    per_xcd = max(workgroups // 8, 1)
    rounds = lambda total: (-(-total // 8) + per_xcd - 1) // per_xcd
    t3 = sum(group_tiles(int(m), bm, nt, 3) for m in sizes)
    t2 = sum(group_tiles(int(m), bm, nt, 2) for m in sizes)
    return rounds(t3) < rounds(t2), t2, t3


def test_absorbing_decision_on_the_workload_routings():
    """The expert slice's routing (experts filled to ~250 rows, 11 of 32 past
    256) takes absorbing blocks on both of its launches (1200 -> 1024 and
    2100 -> 1792 tiles: one round and two rounds fewer); the skewed Zipf
    routing of the large up-projection keeps plain tiles (560 vs 544 tiles,
    three rounds either way)."""
    from workloads import CONFIGS, generate
    c4, c6 = CONFIGS[4], CONFIGS[6]
    ids4 = generate(c4, with_weights=False)["ids"]
    loc = np.bincount(ids4.ravel(), minlength=c4.E)[c4.group_offset:c4.group_offset + c4.E_loc]
    for n_cols, want in ((2 * c4.I, (1200, 1024)), (c4.H, (2100, 1792))):
        ok, t2, t3 = absorb_decision(loc, n_cols // 128)
        assert ok and (t2, t3) == want
    sizes6 = np.bincount(generate(c6, with_weights=False)["ids"].ravel(), minlength=c6.E)
    ok, t2, t3 = absorb_decision(sizes6, c6.I // 128)
    assert not ok and (t2, t3) == (560, 544)


def split_plan(total, grid, KT, nslots=None, per_xcd_max=128, min_steps=4):
    """The grouped matmul's work items, replayed: for each workgroup, its list
    of (tile, first K step, end K step, slot of a split part or None) and the
    counter each split tile uses."""
    nslots = grid if nslots is None else nslots
    items = {}
    for b in range(grid):
        x, xj = b % 8, b // 8
        step = (grid - x + 7) // 8
        lo, hi = total * x // 8, total * (x + 1) // 8
        first = lo + xj
        rounds = (hi - lo) // step
        lft = hi - lo - rounds * step
        lbase = lo + rounds * step
        s = 1
        if lft > 0 and grid <= nslots and lft <= per_xcd_max:
            s = max(min(step // lft, KT // min_steps), 1)
        n_full = rounds if s >= 2 else (len(range(first, hi, step)) if first < hi else 0)
        lst = [(first + i * step, 0, KT, None, None) for i in range(n_full)]
        if s >= 2 and lft > 0 and xj < lft * s:
            ul, up = xj % lft, xj // lft
            lst.append((lbase + ul, up * KT // s, (up + 1) * KT // s, b, (x * per_xcd_max + ul, s, lft)))
        items[b] = lst
    return items


@pytest.mark.parametrize("total,grid,KT", [(560, 256, 56), (24, 48, 16), (1024, 256, 56), (1200, 256, 56),
                                           (7, 256, 16), (300, 256, 4), (33, 40, 64), (2100, 256, 16), (9, 9, 8)])
def test_split_plan_covers_each_tile_once(total, grid, KT):
    """Whole tiles are computed once; a split tile's parts cover its K steps
    once, each part writes the slot of the workgroup that computes it, the
    counter is in range, and part p of a tile is workgroup l + p * lft of the
    XCD, as the last part's summation reads it."""
    items = split_plan(total, grid, KT)
    cover = {}
    for b, lst in items.items():
        for t, k0, k1, slot, ctr in lst:
            assert 0 <= t < total and 0 <= k0 < k1 <= KT
            cover.setdefault(t, []).append((k0, k1))
            if slot is not None:
                assert slot == b < grid
                ci, s, lft = ctr
                assert 0 <= ci < 8 * 128 and k1 - k0 >= 4
                x, ul = b % 8, ci % 128
                parts = [x + 8 * (ul + p * lft) for p in range(s)]
                assert b in parts and all(q < grid for q in parts)
    assert sorted(cover) == list(range(total))
    for t, ranges in cover.items():
        ranges.sort()
        assert ranges[0][0] == 0 and ranges[-1][1] == KT
        assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
    if (total, grid) == (560, 256):          # the skewed up-projection: its third round is split
        assert any(len(r) > 1 for r in cover.values())
