"""Where the fused decode step (pkv_decode_step) may store the new token.

The range that ends at a sequence's new token (position L - 1) stores that
token's K/V row from inside the attention launch, without a barrier.  That
is only correct when, for every 16-byte piece of the row, the one lane whose
load of the piece feeds the scores is the lane that stores it, and its load
comes after the store in that lane's program order.  Loads whose data is
thrown away (rows past the range end, a repeated block, the spare tile of a
wave without tiles) may read the piece at any time.

This models the load schedules of decode_partial_vec (decode.hip) and
decode_partial_mfma (decode_mfma.hip) lane by lane, for every range length up
to several full strides, and checks the store placement the kernels use: the
storing lane is chosen by the kernels' own rule (wave, row group and piece of
the token), and the store sits before the wave's first tile load when the
wave has one tile, else right after it.  The schedule constants restate the
kernels' shapes; a change of either kernel's load order must change this
model with it."""
import numpy as np
import pytest

WAVES = 4            # waves per workgroup in both kernels
LANES = np.arange(64)


# ---------------------------------------------------------------- vector path
def vec_shape(kvb: int, d: int):
    epl = 16 // kvb                    # elements per 16-byte piece
    r = d // epl                       # lanes (pieces) per token row
    rw = 64 // r                       # rows per wave load
    u = min(16 // rw, 4)               # loads per lane per tile
    return r, rw, u, u * rw            # ..., tokens per wave tile


def vec_loads(n: int, kvb: int, d: int):
    """Every (wave, lane, load index, row, piece, used) of one range of n tokens."""
    r, rw, u_n, tok = vec_shape(kvb, d)
    stride = WAVES * tok
    rg, col = LANES // r, LANES % r
    out = []
    for w in range(WAVES):
        tw0 = w * tok
        nt = (n - tw0 + stride - 1) // stride if tw0 < n else 0
        tiles = [tw0 + k * stride for k in range(nt)] if nt else [(n - 1) & ~(tok - 1)]
        for li, t in enumerate(tiles):
            for u in range(u_n):
                rows = t + u * rw + rg
                used = (nt > 0) & (rows < n)
                out.append((w, li, rows, col, used))
    return out


def vec_store(n: int, kvb: int, d: int):
    """Storing lanes per wave (the kernel's rule) and the load index the store precedes."""
    r, rw, _, tok = vec_shape(kvb, d)
    stride = WAVES * tok
    o = n - 1
    lanes = {}
    for w in range(WAVES):
        tw0 = w * tok
        nt = (n - tw0 + stride - 1) // stride if tw0 < n else 0
        sel = (w == (o // tok) % WAVES) & ((LANES // r) == (o % tok) % rw)
        lanes[w] = (sel, 0 if nt == 1 else 1)
    return lanes, LANES % r


# ----------------------------------------------------------- matrix-core path
MF_TILE = 32


def mf_shape(kvb: int, d: int):
    rowb = d * kvb
    r = rowb // 16
    rpi = 64 // r
    lpb = (MF_TILE * rowb) // (64 * 16) // 2      # loads per lane per 16-token block
    return r, rpi, lpb


def mf_loads(n: int, kvb: int, d: int):
    r, rpi, lpb = mf_shape(kvb, d)
    stride = WAVES * MF_TILE
    out = []
    for w in range(WAVES):
        tw0 = w * MF_TILE
        nt = (n - tw0 + stride - 1) // stride if tw0 < n else 0
        tiles = [tw0 + k * stride for k in range(nt)] if nt else [(n - 1) & ~15]
        for li, t0 in enumerate(tiles):
            for blk in range(2):
                tb = t0 if (blk == 1 and t0 + 16 >= n) else t0 + 16 * blk
                for i in range(lpb):
                    rows = tb + LANES // r + rpi * i
                    tok = 16 * blk + LANES // r + rpi * i          # the row the data is scored as
                    used = (nt > 0) & (t0 + tok < n)
                    out.append((w, li, rows, LANES % r, used))
    return out


def mf_store(n: int, kvb: int, d: int):
    r, rpi, _ = mf_shape(kvb, d)
    stride = WAVES * MF_TILE
    o = n - 1
    lanes = {}
    for w in range(WAVES):
        tw0 = w * MF_TILE
        nt = (n - tw0 + stride - 1) // stride if tw0 < n else 0
        sel = (w == (o // MF_TILE) % WAVES) & ((LANES // r) == (o & 15) % rpi)
        lanes[w] = (sel, 0 if nt == 1 else 1)
    return lanes, LANES % r


def check_range(n, loads, store, pieces):
    o = n - 1
    lanes, piece_of_lane = store
    # one storing lane per piece in the workgroup
    stored = {}
    for w, (sel, _) in lanes.items():
        for lane in np.nonzero(sel)[0]:
            p = int(piece_of_lane[lane])
            assert p not in stored, f"n={n}: piece {p} stored twice"
            stored[p] = (w, int(lane))
    assert sorted(stored) == list(range(pieces)), f"n={n}: pieces stored {sorted(stored)}"
    # the used loads of each piece of row o
    used = {p: [] for p in range(pieces)}
    for w, li, rows, cols, ok in loads:
        hit = (rows == o) & ok
        for lane in np.nonzero(hit)[0]:
            used[int(cols[lane])].append((w, int(lane), li))
    for p in range(pieces):
        assert len(used[p]) == 1, f"n={n}: piece {p} used by {used[p]}"
        w, lane, li = used[p][0]
        assert stored[p] == (w, lane), f"n={n}: piece {p} stored by {stored[p]}, used by {(w, lane)}"
        assert li >= lanes[w][1], f"n={n}: piece {p} loaded (load {li}) before its store"


VEC_SHAPES = [(4, 64), (4, 128), (2, 64), (2, 128), (1, 64), (1, 128)]   # (KV bytes, head_dim)
MF_SHAPES = [(2, 64), (2, 128), (1, 64), (1, 128)]


@pytest.mark.parametrize("kvb,d", VEC_SHAPES)
def test_vector_decode_stores_from_the_lane_that_uses_the_piece(kvb, d):
    r, _, _, tok = vec_shape(kvb, d)
    for n in range(1, 3 * WAVES * tok + 2 * tok + 2):
        check_range(n, vec_loads(n, kvb, d), vec_store(n, kvb, d), r)


@pytest.mark.parametrize("kvb,d", MF_SHAPES)
def test_matrix_core_decode_stores_from_the_lane_that_uses_the_piece(kvb, d):
    r, _, _ = mf_shape(kvb, d)
    for n in range(1, 3 * WAVES * MF_TILE + 2 * MF_TILE + 2):
        check_range(n, mf_loads(n, kvb, d), mf_store(n, kvb, d), r)


def test_model_catches_a_wrong_store_rule():
    """The check is not vacuous: choosing the token's row group from the
    wrong token offset (o + 1) fails it."""
    kvb, d = 2, 128
    r, rw, _, tok = vec_shape(kvb, d)
    n = 2 * WAVES * tok + 5
    lanes, piece = vec_store(n, kvb, d)
    o = n                                            # the mistake
    bad = {w: (((w == (o // tok) % WAVES) & ((LANES // r) == (o % tok) % rw)), s)
           for w, (_, s) in lanes.items()}
    with pytest.raises(AssertionError):
        check_range(n, vec_loads(n, kvb, d), (bad, piece), r)
