"""The step/layer schedule of "RainFusion Attention" (vLLM-Omni user guide),
Configuration: start_step early steps and end_step final steps stay dense, so
do the DiT blocks that skip_layers names. Pure host logic."""
import pytest

from block_sparse_video_rf_amd import DenseSchedule, parse_layers, route


def test_selector_of_the_configuration_table():
    # the page's example selector "0-3,38"
    assert parse_layers("0-3,38") == frozenset({0, 1, 2, 3, 38})
    assert parse_layers("0-1") == frozenset({0, 1})
    assert parse_layers(" 5 , 2-2,7-9 ") == frozenset({2, 5, 7, 8, 9})
    assert parse_layers("") == frozenset()
    assert parse_layers(None) == frozenset()
    assert parse_layers([3, 1]) == frozenset({1, 3})


@pytest.mark.parametrize("bad", ["3-1", "a", "1-", "-2", "1,,x", "1.5", "0-3-5"])
def test_bad_selectors_raise(bad):
    with pytest.raises(ValueError):
        parse_layers(bad)


@pytest.mark.parametrize("bad", [[-1], [1.0], [True]])
def test_bad_index_lists_raise(bad):
    with pytest.raises(ValueError):
        parse_layers(bad)


def test_default_schedule_is_sparse_everywhere():
    s = DenseSchedule()
    assert all(s.sparse(t, 50, layer) for t in range(50) for layer in range(40))


def test_page_example_configuration():
    # BlockSparseSpec(sparsity=0.8, start_step=0, skip_layers="0-1")
    s = DenseSchedule(start_step=0, skip_layers="0-1")
    assert not s.sparse(0, 40, 0) and not s.sparse(7, 40, 1)
    assert s.sparse(0, 40, 2) and s.sparse(39, 40, 39)


def test_start_and_end_steps_stay_dense():
    s = DenseSchedule(start_step=2, end_step=3, skip_layers="38")
    got = [s.sparse(t, 10, 5) for t in range(10)]
    assert got == [False, False, True, True, True, True, True, False, False, False]
    assert not s.sparse(4, 10, 38)
    # windows that cover every step leave nothing sparse
    s = DenseSchedule(start_step=6, end_step=6)
    assert not any(s.sparse(t, 10, 0) for t in range(10))


@pytest.mark.parametrize("kw", [dict(start_step=-1), dict(end_step=-2), dict(start_step=1.5),
                                dict(end_step=True), dict(skip_layers="2-1")])
def test_invalid_schedules_raise(kw):
    with pytest.raises(ValueError):
        DenseSchedule(**kw)


def test_out_of_range_queries_raise():
    s = DenseSchedule()
    with pytest.raises(ValueError):
        s.sparse(10, 10, 0)
    with pytest.raises(ValueError):
        s.sparse(-1, 10, 0)
    with pytest.raises(ValueError):
        s.sparse(0, 10, -1)


def test_route_keeps_the_configured_precision_on_both_paths():
    # The page shares the precision between the dense and sparse paths.
    sched = DenseSchedule(start_step=2, end_step=1, skip_layers="5")
    assert route(sched, "fp8", 0, 10, 1) == ("dense", "fp8")     # warm-up step
    assert route(sched, "fp8", 9, 10, 1) == ("dense", "fp8")     # final step
    assert route(sched, "mix", 4, 10, 5) == ("dense", "mix")     # excluded layer
    assert route(sched, "fp8", 4, 10, 1) == ("sparse", "fp8")
    assert route(sched, "bf16", 3, 10, 7) == ("sparse", "bf16")
