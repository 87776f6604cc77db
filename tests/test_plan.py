"""Production orders, tile numbering, task and wait tables (host only)."""
import itertools
import json
import os

import pytest

import tile_overlapped_gemm_amd as tog
from libentwine import ensure_built

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ORDERS = [tog.ORDER_ROW_MAJOR, tog.ORDER_PARTITION_MAJOR, tog.ORDER_INTERLEAVED, tog.ORDER_COL_MAJOR]
# (M, N, P, bm, bn, tm, tn): multi-block, ragged partitions (125 rows), N
# not a multiple of the block, wide and tall blocks.
SHAPES = [
    (512, 768, 4, 128, 256, 128, 128),
    (1000, 1536, 8, 128, 128, 128, 128),
    (1000, 1408, 8, 256, 256, 128, 128),
    (256, 256, 4, 128, 128, 64, 64),
    (2048, 640, 2, 256, 128, 128, 64),
    (96, 136, 3, 128, 128, 64, 128),
    (1000, 1160, 8, 128, 384, 128, 128),   # three tiles per block, a ragged last column
]


@pytest.fixture(scope="module", autouse=True)
def lib():
    return ensure_built()


def test_figure4b_worked_example():
    with open(os.path.join(GOLDEN, "fig4b_interleaved_schedule.json")) as f:
        fx = json.load(f)
    s = fx["shape"]
    P = s["P"]
    M = P * s["rows_per_partition"]
    geo = (s["block_m"], s["block_n"], s["tile_m"], s["tile_n"])
    nb, bd, q = tog.entwine_plan_shape(M, s["N"], P, *geo)
    assert (bd, q) == (3, 6)
    tiles_of_block = {}
    for t, (tr, tc) in enumerate(tog.entwine_plan_tiles(M, s["N"], P, *geo)):
        tiles_of_block.setdefault((tr, tc // 2), []).append(t)
    for rank in range(P):  # the same on every rank
        blocks = tog.entwine_plan_blocks(M, s["N"], P, rank, tog.ORDER_INTERLEAVED, *geo)
        for p, want in fx["visits"]:
            d, br, bc, first = blocks[p]
            assert d == fx["partition"]
            assert tiles_of_block[(br, bc)] == want
            assert first == want[0]
    for j, want in fx["consumers"].items():
        assert tog.entwine_plan_tasks(q, fx["budget"], int(j)) == want


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("order", ORDERS)
def test_every_block_produced_once(shape, order):
    M, N, P, bm, bn, tm, tn = shape
    nb, bd, q = tog.entwine_plan_shape(*shape)
    R = M // P
    assert bd == -(-R // bm) * -(-N // bn) and nb == P * bd
    for rank in range(P):
        blocks = tog.entwine_plan_blocks(M, N, P, rank, order, bm, bn, tm, tn)
        seen = {(d, br, bc) for d, br, bc, _ in blocks}
        assert len(seen) == nb
        assert seen == {(d, br, bc) for d in range(P) for br in range(-(-R // bm))
                        for bc in range(-(-N // bn))}


@pytest.mark.parametrize("shape", SHAPES)
def test_order_definitions(shape):
    M, N, P, bm, bn, tm, tn = shape
    nb, bd, q = tog.entwine_plan_shape(*shape)
    cb = -(-N // bn)
    rb = -(-(M // P) // bm)
    for rank in range(P):
        inter = tog.entwine_plan_blocks(M, N, P, rank, tog.ORDER_INTERLEAVED, bm, bn, tm, tn)
        assert [b[0] for b in inter] == [p % P for p in range(nb)]
        # block i within partition is N-major: (i // cb, i % cb), i = p // P
        assert [(b[1], b[2]) for b in inter] == [((p // P) // cb, (p // P) % cb) for p in range(nb)]
        row = tog.entwine_plan_blocks(M, N, P, rank, tog.ORDER_ROW_MAJOR, bm, bn, tm, tn)
        assert [b[0] for b in row] == [p // bd for p in range(nb)]
        part = tog.entwine_plan_blocks(M, N, P, rank, tog.ORDER_PARTITION_MAJOR, bm, bn, tm, tn)
        runs = [part[k * bd][0] for k in range(P)]
        assert runs == [(rank + 1 + k) % P for k in range(P)] and runs[-1] == rank
        for k in range(P):
            assert {b[0] for b in part[k * bd:(k + 1) * bd]} == {runs[k]}
        col = tog.entwine_plan_blocks(M, N, P, rank, tog.ORDER_COL_MAJOR, bm, bn, tm, tn)
        assert [b[2] for b in col] == sorted(b[2] for b in col)
        assert [(b[0] * rb + b[1]) for b in col[:P * rb]] == list(range(P * rb))


@pytest.mark.parametrize("shape", SHAPES)
def test_tile_numbering(shape):
    M, N, P, bm, bn, tm, tn = shape
    nb, bd, q = tog.entwine_plan_shape(*shape)
    R = M // P
    tiles = tog.entwine_plan_tiles(*shape)
    rt, ct = -(-R // tm), -(-N // tn)
    assert q == rt * ct and sorted(tiles) == sorted(itertools.product(range(rt), range(ct)))
    # numbered block by block in N-major block order, row-major inside a block
    keys = [((tr * tm // bm) * -(-N // bn) + tc * tn // bn, tr, tc) for tr, tc in tiles]
    assert keys == sorted(keys)
    # a block's first-tile field points at its first tile
    blocks = tog.entwine_plan_blocks(M, N, P, 0, tog.ORDER_ROW_MAJOR, bm, bn, tm, tn)
    for d, br, bc, first in blocks:
        assert tiles[first] == (br * bm // tm, bc * bn // tn)


@pytest.mark.parametrize("shape", SHAPES)
def test_wait_tables(shape):
    M, N, P, bm, bn, tm, tn = shape
    nb, bd, q = tog.entwine_plan_shape(*shape)
    for rank in range(P):
        for order in ORDERS:
            pre = tog.entwine_plan_waits(M, N, P, rank, order, bm, bn, tm, tn, tog.PEERS_PRESEEDED)
            assert pre == [[rank * q + t if r == rank else -1 for r in range(P)] + [-1] for t in range(q)]
        for order in (tog.ORDER_INTERLEAVED, tog.ORDER_ROW_MAJOR, tog.ORDER_COL_MAJOR):
            sym = tog.entwine_plan_waits(M, N, P, rank, order, bm, bn, tm, tn, tog.PEERS_SYMMETRIC)
            assert sym == [[rank * q + t] * P + [-1] for t in range(q)]
        # Partition-major: peer r reaches partition `rank` after (rank-r-1) mod P runs;
        # this GPU is then in partition (rank+1+k) mod P = (2*rank - r) mod P.
        sym = tog.entwine_plan_waits(M, N, P, rank, tog.ORDER_PARTITION_MAJOR, bm, bn, tm, tn,
                                     tog.PEERS_SYMMETRIC)
        assert sym == [[((2 * rank - r) % P) * q + t for r in range(P)] + [-1] for t in range(q)]


def test_release_groups():
    M, N, P, bm, bn, tm, tn = 512, 768, 4, 128, 256, 128, 128
    nb, bd, q = tog.entwine_plan_shape(M, N, P, bm, bn, tm, tn)
    rank = 2
    blocks = tog.entwine_plan_blocks(M, N, P, rank, tog.ORDER_INTERLEAVED, bm, bn, tm, tn)
    part = tog.entwine_plan_waits(M, N, P, rank, tog.ORDER_INTERLEAVED, bm, bn, tm, tn,
                                  tog.PEERS_PRESEEDED, tog.RELEASE_PARTITION)
    last = max(p for p in range(nb) if blocks[p][0] == rank)
    # any flag of the closing block will do: a block publishes all of its
    # tiles' flags together, after all of its stores
    closing = {rank * q + blocks[last][3], rank * q + blocks[last][3] + 1}
    assert {w[P] for w in part} <= closing
    assert [w[rank] for w in part] == [rank * q + t for t in range(q)]
    out = tog.entwine_plan_waits(M, N, P, rank, tog.ORDER_INTERLEAVED, bm, bn, tm, tn,
                                 tog.PEERS_PRESEEDED, tog.RELEASE_OUTPUT)
    d, _, _, first = blocks[nb - 1]
    assert {w[P] for w in out} <= {d * q + first, d * q + first + 1}
    g2 = tog.entwine_plan_waits(M, N, P, rank, tog.ORDER_INTERLEAVED, bm, bn, tm, tn,
                                tog.PEERS_PRESEEDED, 4)
    # groups {0..3} and {4,5}: closed by the blocks holding tiles {2,3} and {4,5}
    assert [w[P] - rank * q for w in g2] == [2, 2, 2, 3, 4, 5]


@pytest.mark.parametrize("q,x", [(6, 2), (128, 32), (96, 1), (5, 9), (1, 1)])
def test_tasks_partition_the_tiles(q, x):
    seqs = [tog.entwine_plan_tasks(q, x, j) for j in range(x + 2)]
    flat = sorted(t for s in seqs for t in s)
    assert flat == list(range(q))
    for j, s in enumerate(seqs):
        assert s == list(range(j, q, min(x, q))) if j < min(x, q) else s == []


def _panels(blocks, positions, Rb):
    rows = {blocks[p][0] * Rb + blocks[p][1] for p in positions}
    cols = {blocks[p][2] for p in positions}
    return len(rows) + len(cols)


@pytest.mark.parametrize("shape,window", [
    ((4096, 4096, 8, 256, 256, 128, 128), 256),     # one window: the whole grid
    ((8192, 8192, 8, 256, 256, 128, 128), 256),     # four windows
    ((16384, 5120, 4, 256, 256, 128, 128), 256),    # five windows
    ((1000, 12288, 8, 128, 128, 128, 128), 512),    # two blocks per CU
    ((1000, 12288, 8, 128, 384, 128, 128), 256),    # one window of 128 x 384 blocks
    ((1000, 1536, 8, 128, 128, 128, 128), 40),      # a partial last window
])
def test_dispatch_is_windowed_permutation(shape, window):
    """Workgroup b computes logical position dispatch[b]: a permutation that
    keeps every window of consecutive positions on the same window of
    workgroups (production order is kept across windows) and gives every XCD
    (workgroups b with equal b % 8) a compact set of blocks."""
    M, N, P, bm, bn, tm, tn = shape
    nb, bd, q = tog.entwine_plan_shape(*shape)
    for order in ORDERS:
        disp = tog.entwine_plan_dispatch(M, N, P, 0, order, bm, bn, tm, tn, window)
        assert sorted(disp) == list(range(nb))
        w = window - window % 8
        for b, p in enumerate(disp):
            assert b // w == p // w
        assert tog.entwine_plan_dispatch(M, N, P, 0, order, bm, bn, tm, tn, 0) == list(range(nb))
        # the busiest XCD of each window touches no more panels than with the
        # identity dispatch
        blocks = tog.entwine_plan_blocks(M, N, P, 0, order, bm, bn, tm, tn)
        Rb = -(-(M // P) // bm)
        for w0 in range(0, nb, w):
            span = range(w0, min(nb, w0 + w))
            mine = max(_panels(blocks, [disp[b] for b in span if b % 8 == x], Rb) for x in range(8))
            ident = max(_panels(blocks, [b for b in span if b % 8 == x], Rb) for x in range(8))
            assert mine <= ident


def test_dispatch_panel_counts_mlp():
    """MLP slice, 256x256 blocks, one window of 256: interleaved order gives XCD
    x the 32 blocks of partition x (2 row panels + 16 column panels); the
    XCD-aware deal gives each XCD a 4 x 8 rectangle (12 panels)."""
    M, N, P, bm, bn, tm, tn = 4096, 4096, 8, 256, 256, 128, 128
    blocks = tog.entwine_plan_blocks(M, N, P, 0, tog.ORDER_INTERLEAVED, bm, bn, tm, tn)
    disp = tog.entwine_plan_dispatch(M, N, P, 0, tog.ORDER_INTERLEAVED, bm, bn, tm, tn, 256)
    for x in range(8):
        assert _panels(blocks, [b for b in range(256) if b % 8 == x], 2) == 18
        assert _panels(blocks, [disp[b] for b in range(256) if b % 8 == x], 2) == 12


@pytest.mark.parametrize("shape", SHAPES[:3] + [(4096, 4096, 8, 256, 256, 128, 128)])
@pytest.mark.parametrize("mode,group", [(tog.PEERS_PRESEEDED, tog.RELEASE_TILE),
                                        (tog.PEERS_SYMMETRIC, tog.RELEASE_TILE),
                                        (tog.PEERS_PRESEEDED, 3),
                                        (tog.PEERS_SYMMETRIC, tog.RELEASE_PARTITION)])
def test_fused_task_order_follows_production(shape, mode, group):
    """The fused kernel's tasks: a permutation of tile x slab, each tile's
    slabs together and in order, tiles sorted by the dispatch index of the
    last block that their wait slots depend on (ties by tile number)."""
    M, N, P, bm, bn, tm, tn = shape
    nb, _, q = tog.entwine_plan_shape(M, N, P, bm, bn, tm, tn)
    rank = P - 1
    window = 16
    for order in ORDERS:
        blocks = tog.entwine_plan_blocks(M, N, P, rank, order, bm, bn, tm, tn)
        dispatch = tog.entwine_plan_dispatch(M, N, P, rank, order, bm, bn, tm, tn, window)
        at = {p: b for b, p in enumerate(dispatch)}
        pos = {tuple(blocks[p][:3]): p for p in range(nb)}
        tiles = tog.entwine_plan_tiles(M, N, P, bm, bn, tm, tn)
        waits = tog.entwine_plan_waits(M, N, P, rank, order, bm, bn, tm, tn, mode, group)

        def ready(t):
            last = -1
            for f in waits[t]:
                if f >= 0:
                    d, tt = divmod(f, q)
                    tr, tc = tiles[tt]
                    last = max(last, at[pos[(d, tr // (bm // tm), tc // (bn // tn))]])
            return last

        for slabs in (1, 4):
            got = tog.entwine_plan_task_order(M, N, P, rank, order, bm, bn, tm, tn, mode, group,
                                              window, slabs)
            assert sorted(got) == list(range(q * slabs))
            seq = [got[k] // slabs for k in range(0, len(got), slabs)]
            for k, t in enumerate(seq):
                assert got[k * slabs:(k + 1) * slabs] == [t * slabs + s for s in range(slabs)]
            keys = [(ready(t), t) for t in seq]
            assert keys == sorted(keys)


def test_fused_task_order_errors():
    with pytest.raises(tog.EntwineError):
        tog.entwine_plan_task_order(512, 768, 4, 0, tog.ORDER_INTERLEAVED, 128, 256, 128, 128,
                                    task_slabs=3)
    with pytest.raises(tog.EntwineError):
        tog.entwine_plan_task_order(512, 768, 4, 0, tog.ORDER_INTERLEAVED, 128, 256, 128, 128,
                                    window=-1)
