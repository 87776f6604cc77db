"""The offline sweep's selection rule and table format (host only)."""
import pytest

import tile_overlapped_gemm_amd as tog
import workloads as wl
from libentwine import ensure_built
from tile_overlapped_gemm_amd import sweep


def C(us, budget=4, threads=256, order=2, slabs=1, schedule=1, bm=128, bn=128, variant=0):
    return sweep.Candidate(bm, bn, order, budget, threads, slabs, schedule, variant=variant, us=us)


def test_pick_lowest_latency():
    assert sweep.pick([C(10.0, budget=8), C(12.0, budget=1), C(None, budget=0)]).budget == 8


def test_pick_ties_go_to_smaller_budget_threads_order():
    # within 1 %: equal latency; smaller budget wins, then threads, then order
    assert sweep.pick([C(100.0, budget=8), C(100.5, budget=2), C(99.8, budget=4)]).budget == 2
    assert sweep.pick([C(100.0, threads=512), C(100.2, threads=128)]).threads == 128
    assert sweep.pick([C(100.0, order=3), C(100.3, order=0)]).order == 0
    assert sweep.pick([C(100.0, variant=4), C(100.4, variant=0)]).variant == 0
    assert sweep.pick([C(97.0, variant=4), C(100.0, variant=0)]).variant == 4
    # outside the tie band the faster one wins even with a larger budget
    assert sweep.pick([C(100.0, budget=64), C(110.0, budget=0)]).budget == 64
    with pytest.raises(ValueError):
        sweep.pick([C(None)])


def test_pipelines_per_block_shape():
    assert sweep.pipelines_for(256, 256) == [0, 4]
    assert sweep.pipelines_for(128, 384) == [0]
    assert sweep.pipelines_for(256, 256, wkn=True) == [0]


def test_budget_list():
    assert sweep.budgets_for(4, 256) == [0, 1, 2, 4]
    b = sweep.budgets_for(1280, 256)
    assert b[0] == 0 and max(b) == 255 and b == sorted(set(b))
    assert max(sweep.budgets_for(1280, 128)) < 128


def test_table_line_is_loadable(tmp_path):
    ensure_built()
    w = wl.BY_NAME["mlp"]
    line = sweep.table_line(w, C(50.0, budget=255, slabs=4, schedule=tog.SCHEDULE_FUSED, bm=256,
                                 bn=256, variant=4))
    assert line == "4096 4096 1792 8 2 255 256 256 256 4 2 4"
    p = tmp_path / "t.txt"
    p.write_text("# header\n" + line + "\n")
    tog.entwine_load_tuning(str(p))
    tog.entwine_load_tuning(tog.__file__.replace("__init__.py", "tuning.txt"))
