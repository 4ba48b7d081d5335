"""Host-only model of every global address the tiled GEMM kernels' DMAs form,
for every workgroup of the launch plans the library's own planner
(tf_gemm_plan) produces: 256 x 256 tiles (gemm256.hip), and 256 x 128,
256 x 64 and 128 x 128 tiles (gemm.hip), single launches, wide + narrow
launches and split K.

The kernels build each address as a 64-bit wave-uniform base plus 32-bit
lane offsets, with loads past the data clamped (x: to the row's last 16
bytes of the range; codes and records: to the last k-tile and the first
record).  The model repeats that arithmetic on numpy arrays and checks:
  - every byte read lies inside its buffer (x, the packed weights), and a
    block's codes and records inside that block;
  - every 32-bit lane offset stays below 2^32;
  - a load inside the data reads exactly the element the kernel's layout
    says it holds (x row and column, code tile, group record);
  - the workgroup-to-tile map is a bijection and each tile's loads cover
    every row and column of x and every code tile it needs.
A mismatch here is an out-of-bounds read or a wrong operand on the GPU, so
the model runs on the CPU before any shape reaches the device.  The
formulas follow the kernels' sources line by line in meaning: the
activation DMA (dma_a), the code DMA (dma_codes), the record DMA (dma_rec /
dma_meta) and the tile order at the top of each kernel.
"""

import numpy as np
import pytest

LANE = np.arange(64)


def _lib():
    import quantized_linear_layers_awq_amd as q

    q.load_library()
    return q


def layout(bits, K, N, G):
    RB = 40 if bits == 4 else 48
    TB = 1024 if bits == 4 else 2048
    ngroups, ktiles, nblocks = K // G, -(-K // 128), -(-N // 16)
    meta = (ngroups * RB + 15) // 16 * 16
    whole = G % 128 == 0 or G == K
    tpg = (ktiles if G == K else G // 128) if whole else 0
    return dict(RB=RB, TB=TB, ngroups=ngroups, ktiles=ktiles, nblocks=nblocks, meta=meta,
                block=meta + ktiles * TB, tpg=tpg, total=nblocks * (meta + ktiles * TB))


def tile_map(nwg, splits, m_tiles, band=2):
    """(split, row tile, column tile) of every workgroup: each XCD (bid % 8)
    takes a contiguous run of tiles, enumerated in bands of `band` row
    tiles, rows first within a band."""
    q8, rem = nwg >> 3, nwg & 7
    per_split = nwg // splits
    n_tiles = per_split // m_tiles
    band_rows = band if 0 < band < m_tiles else m_tiles
    out = []
    for bid in range(nwg):
        xcd, local = bid & 7, bid >> 3
        t_all = xcd * (q8 + 1) + local if xcd < rem else rem * (q8 + 1) + (xcd - rem) * q8 + local
        split, tile = t_all // per_split, t_all % per_split
        b = tile // (band_rows * n_tiles)
        ib = tile - b * band_rows * n_tiles
        rows_here = min(m_tiles - b * band_rows, band_rows)
        out.append((split, b * band_rows + ib % rows_here, ib // rows_here))
    want = [(s, a, c) for s in range(splits) for a in range(m_tiles) for c in range(n_tiles)]
    assert sorted(out) == want, (nwg, splits, m_tiles)
    return n_tiles


def split_range(L, G, K, split, split_tiles):
    """k_begin, k-tiles and K of a range; its first group; its first k-tile."""
    kt0 = split * split_tiles
    kt1 = min(kt0 + split_tiles, L["ktiles"])
    k_begin = kt0 * 128
    Kr = min(kt1 * 128, K) - k_begin
    g_begin = 0 if G == K else k_begin // G
    return k_begin, kt1 - kt0, Kr, g_begin, kt0


def check_x(M, K, k_begin, Kr, m0, R, AJ, wave, stages, x_bytes, cover):
    """Activation DMA of one wave: rows R w .. R w + R - 1 of the row tile, 8
    rows per instruction j; lane p: row 8 j + p / 8, swizzled unit c of its
    slot p % 8; offset clamped to the range's last 16 bytes of the row."""
    a_slot = LANE & 7
    a_c = [a_slot ^ ((LANE >> 4) & 7), a_slot ^ ((4 + (LANE >> 4)) & 7)]
    base_row = min(m0 + R * wave, M - 1)
    base = (base_row * K + k_begin) * 2
    a_last = 2 * Kr - 16
    for j in range(AJ):
        row = np.minimum(m0 + R * wave + 8 * j + (LANE >> 3), M - 1)
        voff = (row - base_row) * K * 2
        assert voff.min() >= 0 and voff.max() < 2**32
        col = np.minimum(stages[:, None] * 128 + 16 * a_c[j & 1][None, :], a_last)  # bytes into the range
        assert col.min() >= 0 and (voff[None, :] + col).max() < 2**32
        addr = base + voff[None, :] + col
        assert addr.min() >= 0 and addr.max() + 16 <= x_bytes
        # inside the data: exactly the element (row, k_begin + 64 s + 8 c)
        inside = stages[:, None] * 128 + 16 * a_c[j & 1][None, :] + 16 <= 2 * Kr
        want = (row[None, :] * K + k_begin + stages[:, None] * 64 + 8 * a_c[j & 1][None, :]) * 2
        assert np.array_equal(addr[inside], np.broadcast_to(want, addr.shape)[inside])
        rr = np.broadcast_to(row, addr.shape)[inside]
        kk = (np.broadcast_to(want, addr.shape)[inside] // 2) % K
        cover[rr - m0, kk // 8 - k_begin // 8] = True


def new_cover(M, m0, BM, Kr):
    """Which (row of the tile, 8-column unit of the range) the loads reach."""
    return np.zeros((min(m0 + BM, M) - m0, Kr // 8), dtype=bool)


def check_codes(L, blks, kt0, ts, halves):
    """Code DMA of blocks `blks` (array): 16 bytes per lane at soff = (the
    range's meta offset) + t * tile bytes (+ 1024 for a W8 half), from the
    block base moved by the range's first record; ts and halves: arrays of
    the k-tiles and halves fetched."""
    b = np.asarray(blks)[:, None, None]
    t = np.asarray(ts)[None, :, None]
    h = np.asarray(halves)[None, :, None]
    addr = L["block"] * b + L["meta"] + (kt0 + t) * L["TB"] + 1024 * h + 16 * LANE[None, None, :]
    assert np.all(addr >= L["block"] * b + L["meta"]) and np.all(addr + 16 <= L["block"] * (b + 1))
    assert addr.max() + 16 <= L["total"]


def check_records(L, blks, g_first, ngroups_range, g_begin, lane_off, want_first=None):
    """Record DMA (one dword per lane) of blocks `blks` for k-tiles whose
    first group in the range is g_first (array); lanes whose record lies past
    the range's groups re-read offset 0; the dwords stay inside the block's
    records, and the group read is the k-tile's (want_first)."""
    b = np.asarray(blks)[:, None, None]
    gf = np.asarray(g_first)[None, :, None]
    grp = (lane_off // L["RB"])[None, None, :]
    v = np.where(gf + grp < ngroups_range, gf * L["RB"] + lane_off[None, None, :], 0)
    addr = L["block"] * b + g_begin * L["RB"] + v
    assert np.all(addr >= L["block"] * b) and np.all(addr + 4 <= L["block"] * b + L["meta"])
    if want_first is not None:
        assert np.array_equal(g_begin + np.asarray(g_first), np.asarray(want_first))


def check_plan_256(q, bits, M, K, N, G, cus, route):
    m_tiles, wide, narrow, splits, split_tiles, gemv, rows, col_tile = q.tf_gemm_plan(bits, M, K, N, G, cus, route)
    assert gemv == 0 and rows == 256 and col_tile == 256 and narrow == 0
    L = layout(bits, K, N, G)
    nwg = m_tiles * wide * splits
    n_tiles = tile_map(nwg, splits, m_tiles)
    x_bytes, RB = M * K * 2, L["RB"]
    for split in range(splits):
        k_begin, kts, Kr, g_begin, kt0 = split_range(L, G, K, split, split_tiles)
        nstages = 2 * kts
        # x: stage 0 in the prologue, then stage s + 1 during stage s (the
        # last one past the range, clamped)
        stages = np.arange(0, nstages + 1)
        for mt in range(m_tiles):
            cover = new_cover(M, mt * 256, 256, Kr)
            for wave in range(8):
                check_x(M, K, k_begin, Kr, mt * 256, 32, 4, wave, stages, x_bytes, cover)
            assert cover.all()
        # codes: W4 k-tile 0 in the prologue, k-tile min(t + 1, last) during
        # k-tile t; W8 the halves of stages 0 and 1 in the prologue, stage
        # min(s + 2, last) during stage s.  Wave w fetches blocks 2 w and
        # 2 w + 1 of the tile (a block past N: block 0)
        b = np.arange(n_tiles * 16)
        blks = np.where(b < L["nblocks"], b, 0)
        if bits == 4:
            code_ts = np.array(sorted({0} | {min(t + 1, kts - 1) for t in range(kts)}))
            hs = np.zeros_like(code_ts)
        else:
            st = np.array(sorted({0, 1} | {min(s + 2, nstages - 1) for s in range(nstages)}))
            assert st.tolist() == list(range(nstages))
            code_ts, hs = st >> 1, st & 1
        assert sorted(set(code_ts.tolist())) == list(range(kts))
        check_codes(L, blks, kt0, code_ts, hs)
        ts = np.arange(kts)  # records: k-tile 0 in the prologue, min(t + 1, last) during k-tile t
        tpg = L["tpg"] if G != K else kts
        g_first = np.zeros_like(ts) if G == K else ts // tpg  # group_of(t), relative to the range
        ngroups_range = 1 if G == K else Kr // G
        lane_off = 4 * np.where(LANE < RB // 4, LANE, 0)
        # every lane of the record reads its own dword of the k-tile's group
        assert np.all(g_first + (lane_off // RB).max() < ngroups_range)
        check_records(L, blks, g_first, ngroups_range, g_begin, lane_off,
                      None if G == K else ((kt0 + ts) * 128) // G)
    return nwg


def check_plan_128(q, bits, M, K, N, G, cus, route):
    m_tiles, wide, narrow, splits, split_tiles, gemv, BM, col_tile = q.tf_gemm_plan(bits, M, K, N, G, cus, route)
    assert gemv == 0 and col_tile == 128 and BM in (128, 256)
    L = layout(bits, K, N, G)
    x_bytes, RB, TB = M * K * 2, L["RB"], L["TB"]
    assert wide * 128 + narrow * 64 >= N
    launches = [(2, wide, 0)] + ([(1, narrow, wide * 128)] if narrow else [])
    split_mode = G in (32, 64)
    gpt = 128 // G if split_mode else 1
    recs = 4 if split_mode else 1
    block_meta = recs * RB
    n_wg = 0
    for WN, ncols, col0 in launches:
        if ncols == 0:
            continue
        nwg = m_tiles * ncols * splits
        n_wg += nwg
        n_tiles = tile_map(nwg, splits, m_tiles)
        AJ, R = BM // 64, BM // 8
        for split in range(splits):
            k_begin, kts, Kr, g_begin, kt0 = split_range(L, G, K, split, split_tiles)
            nstages = 2 * kts
            # x: stages 0 and 1 in the prologue, min(s + 2, last) during s
            stages = np.array(sorted({0, 1} | {min(s + 2, nstages - 1) for s in range(nstages)}))
            for mt in range(m_tiles):
                cover = new_cover(M, mt * BM, BM, Kr)
                for wave in range(8):
                    check_x(M, K, k_begin, Kr, mt * BM, R, AJ, wave, stages, x_bytes, cover)
                assert cover.all()
            # codes: W4 k-tiles 0, min(1, last), then min(t + 2, last); W8
            # halves of stages 0, 1, 2, then min(s + 3, last)
            if bits == 4:
                ts = np.array(sorted({0, min(1, kts - 1)} | {min(t + 2, kts - 1) for t in range(kts)}))
                hs = np.zeros_like(ts)
            else:
                st = np.array(sorted({0, 1, min(2, nstages - 1)} | {min(s + 3, nstages - 1) for s in range(nstages)}))
                ts, hs = st >> 1, st & 1
            assert sorted(set(ts.tolist())) == list(range(kts))
            # records: k-tiles 0 and min(1, last) in the prologue, then
            # min(t + 2, last); the first group of k-tile t in the range
            meta_ts = np.array(sorted({0, min(1, kts - 1)} | {min(t + 2, kts - 1) for t in range(kts)}))
            if G == K:
                g_first = np.zeros_like(meta_ts)
            elif split_mode:
                g_first = meta_ts * gpt
            else:
                g_first = meta_ts // (G // 128)
            ngroups_range = 1 if G == K else Kr // G
            m_lane = np.where(LANE < block_meta // 4, LANE, 0)
            # the unpacking waves: one block each (a block past N: block 0)
            b = col0 // 16 + np.arange(n_tiles * 4 * WN)
            blks = np.where(b < L["nblocks"], b, 0)
            check_codes(L, blks, kt0, ts, hs)
            check_records(L, blks, g_first, ngroups_range, g_begin, 4 * m_lane,
                          None if G == K else ((kt0 + meta_ts) * 128) // G)
    return n_wg


# (bits, M, K, N, G): the prefill and large-dimension workloads, ragged
# rows, columns and K, every group rule, shapes that split K
SHAPES = [
    (4, 2048, 4096, 14336, 128), (4, 2048, 14336, 4096, 128), (4, 4096, 8192, 32768, 128),
    (4, 4096, 28672, 8192, 128), (8, 512, 8192, 8192, 8192), (4, 600, 2048, 1000, 128),
    (4, 260, 1024, 264, 256), (4, 513, 4128, 520, 4128), (4, 200, 8192, 512, 512), (4, 129, 1024, 8, 128),
    (4, 300, 128, 264, 128), (4, 1024, 4096, 2048, 128), (4, 300, 32, 64, 32), (4, 100, 2592, 128, 32),
    (8, 140, 32, 40, 32), (4, 96, 4096, 256, 512), (8, 64, 3072, 128, 3072), (4, 40, 2080, 128, 32),
    (8, 520, 1024, 456, 128), (8, 384, 2048, 264, 2048), (4, 700, 512, 1000, 64), (8, 513, 1024, 392, 32),
    (4, 129, 4096, 28672, 128), (4, 256, 14336, 4096, 128), (8, 1000, 224, 40, 224),
    # W8 on 256 x 256 tiles: the prefill shape, per channel with a ragged
    # last k-tile, groups of two k-tiles split over K, a partial column tile
    (8, 2048, 4096, 14336, 128), (8, 300, 4128, 520, 4128), (8, 200, 8192, 264, 256),
]


@pytest.mark.parametrize("cus", [1, 7, 256, 4096])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_dma_addresses_stay_in_bounds(shape, cus):
    q = _lib()
    bits, M, K, N, G = shape
    checked = 0
    # AUTO: the product's plan (the GEMV kernels up to 64 rows, not modelled
    # here); TILED: the tiled GEMM at any M, 256 x 256 tiles wherever they
    # apply; TILED128: 256 x 128 / 256 x 64 / 128 x 128 tiles
    for route in (q.TF_ROUTE_AUTO, q.TF_ROUTE_TILED, q.TF_ROUTE_TILED128):
        plan = q.tf_gemm_plan(bits, M, K, N, G, cus, route)
        if plan[5]:
            continue
        if plan[7] == 256:
            checked += check_plan_256(q, bits, M, K, N, G, cus, route)
        else:
            checked += check_plan_128(q, bits, M, K, N, G, cus, route)
    assert checked > 0


def test_model_covers_both_tile_heights_splits_and_narrow_tiles():
    """The shape list reaches every plan kind the model checks."""
    q = _lib()
    kinds = set()
    for bits, M, K, N, G in SHAPES:
        for cus in (1, 7, 256, 4096):
            for route in (q.TF_ROUTE_TILED, q.TF_ROUTE_TILED128):
                mt, wide, narrow, splits, _, _, rows, cols = q.tf_gemm_plan(bits, M, K, N, G, cus, route)
                kinds.add((rows, cols, narrow > 0, splits > 1))
    for want in ((256, 256, False, False), (256, 256, False, True), (256, 128, False, False),
                 (256, 128, True, False), (256, 128, False, True), (128, 128, False, False),
                 (128, 128, False, True)):
        assert want in kinds, (want, sorted(kinds))
