"""Address bounds of the ping-pong grouped GEMM's direct-to-LDS loads, and the
tile walk of the persistent weight-streaming launches (CPU only).

The eight-wave 128 / 256 / 320 x 256 tiles load each K step through two buffer
descriptors without range checks: the weight descriptor starts at the tile's
first weight row, the activation descriptor at row 0 of the activation matrix.
This replays the kernel's per-lane offset formulas for every wave, lane and
chunk of a tile and checks that every 16-byte read of every K step stays inside
its matrix, for the tile shapes the layer plan picks, including tiles taller
than the whole batch (the 320-row tile of a 150-token top-2 layer)."""
import pytest

from mixture_experts_transformer_moe_amd import binding as B


def pp_offsets(BM, K, esz, m0, r1, a_rows=None):
    """(descriptor, byte offset) of every chunk load of every lane, as the kernel
    computes them: chunks i < 4 are weight rows, the rest activation rows
    (clamped into the segment)."""
    HB = BM // 2
    NCG = 16 + HB // 8
    NCH = NCG // 4
    assert NCH * 4 == NCG
    out = []
    for wave in range(8):
        wave_n, g = wave % 4, wave // 4
        for lane in range(64):
            col = ((lane & 7) ^ (lane >> 3)) * 16
            voff = []
            for i in range(NCH):
                c = wave_n + 4 * i
                if i < 4:
                    row = g * 128 + c * 8 + (lane >> 3)
                    voff.append(("w", row * K * esz + col))
                else:
                    r = min(m0 + g * HB + (c - 16) * 8 + (lane >> 3), r1 - 1)
                    arow = a_rows[r] if a_rows is not None else r
                    voff.append(("a", arow * K * esz + col))
            out.extend(voff)
    return out


def pp2_offsets(BM, K, esz, m0, r1, a_rows=None):
    """The same for the 256 x 256 / 320 x 256 tiles: each group (waves 0-3, 4-7)
    loads 128 weight rows and its BM / 2 activation rows per stage, (16 + BM /
    16) / 4 8-row chunks per wave (chunk c = wave % 4 + 4 i: c < 16 weight rows
    128 g + 8 c, else activation rows BM / 2 g + 8 (c - 16), clamped into the
    segment)."""
    HB = BM // 2
    NCH = (16 + HB // 8) // 4
    out = []
    for wave in range(8):
        g, wl = wave // 4, wave % 4
        for lane in range(64):
            col = ((lane & 7) ^ (lane >> 3)) * 16
            for i in range(NCH):
                c = wl + 4 * i
                if i < 4:
                    row = g * 128 + c * 8 + (lane >> 3)
                    out.append(("w", row * K * esz + col))
                else:
                    r = min(m0 + g * HB + (c - 16) * 8 + (lane >> 3), r1 - 1)
                    arow = a_rows[r] if a_rows is not None else r
                    out.append(("a", arow * K * esz + col))
    return out


def pp2_lds_rows(BM):
    """LDS rows each wave's chunks land in (weights 0-255, activations 256 ..):
    every row of a stage exactly once."""
    HB = BM // 2
    NCH = (16 + HB // 8) // 4
    rows = []
    for wave in range(8):
        g, wl = wave // 4, wave % 4
        for i in range(NCH):
            c = wl + 4 * i
            base = g * 128 + c * 8 if i < 4 else 256 + g * HB + (c - 16) * 8
            rows.extend(range(base, base + 8))
    return rows


def check_tile(BM, K, esz, m0, r1, a_total_rows, a_rows=None):
    nk = K * esz // 128
    last = (nk - 1) * 128 + 16          # the last step's 16 bytes past the base offset
    offs = pp2_offsets(BM, K, esz, m0, r1, a_rows) if BM in (256, 320) else pp_offsets(BM, K, esz, m0, r1, a_rows)
    for kind, off in offs:
        assert off >= 0
        if kind == "w":
            assert off + last <= 256 * K * esz, (BM, kind, off)
        else:
            assert off + last <= a_total_rows * K * esz, (BM, kind, off, a_total_rows)


@pytest.mark.parametrize("BM", [128, 256, 320])
def test_expert_tiles_stay_inside_operands(BM):
    # first GEMM: A = x [T, H] read through slot_token; second GEMM: A = h [R_max, F]
    for T, H, seg in [(150, 256, 150), (1024, 512, 300), (20, 512, 17), (129, 256, 129)]:
        for r0 in (0, T - seg):
            r1 = r0 + seg
            a_rows = [min(r, T - 1) for r in range(r1)]         # any token index < T
            for mt in range((seg + BM - 1) // BM):
                check_tile(BM, H, 2, r0 + mt * BM, r1, T, a_rows)
                check_tile(BM, H, 2, r0 + mt * BM, r1, r1)       # h rows


@pytest.mark.parametrize("BM", [128, 256, 320])
def test_dense_mlp_tiles_stay_inside_x(BM):
    for T in (1, 100, 150, 160, 300):
        for mt in range((T + BM - 1) // BM):
            check_tile(BM, 512, 2, mt * BM, T, T)


@pytest.mark.parametrize("BM", [256, 320])
def test_pp2_stage_rows_each_loaded_once(BM):
    rows = pp2_lds_rows(BM)
    assert sorted(rows) == list(range(256 + BM))


def test_plan_picks_320_rows_for_short_batches():
    """The layer plan does send a 150-token top-2 layer to 320-row tiles (one
    tile per 300-row segment), so the bound above is what keeps its loads
    inside x."""
    plan = B.moe_layer_plan(B.make_desc(150, 256, 512, 2, 2, 2.0, "f16"))
    assert plan["tile"] == (320, 256, 256)


def persistent_walk(total, grid):
    """Tiles each work-group of a persistent weight-streaming launch takes, as the
    kernel computes them: work-group b runs on XCD x = b % 8 and takes tiles
    start_x + b // 8, + grid // 8, ... below end_x, where [start_x, end_x) is XCD
    x's contiguous share of the list (the split one tile per work-group gives)."""
    g8 = grid // 8
    q, rr = total // 8, total % 8
    walks = []
    for b in range(grid):
        x, j = b % 8, b // 8
        start = x * q + min(x, rr)
        end = start + q + (1 if x < rr else 0)
        walks.append(list(range(start + j, end, g8)))
    return walks


def xcd_remap(i, total):
    q, r = total // 8, total % 8
    x, slot = i % 8, i // 8
    return x * q + min(x, r) + slot


@pytest.mark.parametrize("grid", [8, 512, 768, 1024])
def test_persistent_walk_covers_every_tile_once(grid):
    """Every tile of the list is taken by exactly one work-group, by one on the
    XCD that the one-tile-per-work-group launch would give it."""
    for total in list(range(0, 80)) + [527, 528, 1055, 1056, 2112, 6144, 65535]:
        walks = persistent_walk(total, grid)
        taken = sorted(t for w in walks for t in w)
        assert taken == list(range(total)), (total, grid)
        one_per_wg = {xcd_remap(i, total): i % 8 for i in range(total)}
        for b, w in enumerate(walks):
            assert all(one_per_wg[t] == b % 8 for t in w), (total, grid, b)
