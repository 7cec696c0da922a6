"""Host-side logic of bench.py (no GPU): the round statistics reported beside
the mean step time, and the source hash that keeps committed HBM counters tied
to the kernel they were taken on."""
import os

import numpy as np
import pytest

import bench

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "sampling_sparse_attention_amd", "csrc")


def test_round_stats_median_and_interval():
    rounds = [25.1e-6, 25.3e-6, 25.2e-6, 26.0e-6, 25.4e-6, 25.2e-6, 25.25e-6]
    r = bench.round_stats(rounds)
    assert r["rounds"] == len(rounds)
    assert r["median_us"] == pytest.approx(np.median(rounds) * 1e6)
    lo, hi = r["ci95_us"]
    assert min(rounds) * 1e6 <= lo <= r["median_us"] <= hi <= max(rounds) * 1e6
    assert r["min_us"] == pytest.approx(25.1) and r["max_us"] == pytest.approx(26.0)


def test_round_stats_constant_rounds_have_a_point_interval():
    r = bench.round_stats([20e-6] * 10)
    assert r["ci95_us"][0] == pytest.approx(20.0) and r["ci95_us"][1] == pytest.approx(20.0)


def test_round_stats_empty():
    assert bench.round_stats([]) is None


def test_strip_comments_keeps_code_only():
    src = "int a; // trailing\n/* block\n   comment */ int b;\n\n   // whole line\nint c; /* x */\n"
    assert bench.strip_comments(src) == "int a;\n int b;\nint c;"


def _sources():
    out = {}
    for name in bench.KERNEL_SOURCES:
        with open(os.path.join(CSRC, name)) as f:
            out[name] = f.read()
    return out


def test_source_hash_ignores_comments_but_not_code():
    src = _sources()
    base = bench.kernel_source_hash(lambda n: src[n])
    assert base == bench.kernel_source_hash()
    first = bench.KERNEL_SOURCES[0]
    commented = dict(src)
    commented[first] = "// an added comment line\n" + src[first].replace("\n", "  /* note */\n", 1)
    assert bench.kernel_source_hash(lambda n: commented[n]) == base
    changed = dict(src)
    changed[first] = src[first] + "\nstatic int added_symbol = 1;\n"
    assert bench.kernel_source_hash(lambda n: changed[n]) != base


@pytest.mark.parametrize("steps", [1, 7, 10, 20, 97, 200, 400, 2000, 4000])
@pytest.mark.parametrize("ncopies", [1, 3, 8])
def test_graph_plan_times_exactly_the_requested_calls(steps, ncopies):
    L, P, replays, rounds = bench.graph_plan(steps, ncopies)
    assert L * replays == steps                         # exactly --steps calls
    assert 1 <= L <= bench.MAX_GRAPH_CALLS
    assert rounds <= replays
    assert rounds >= min(10, steps)                     # the driver's --steps 20 still has 10 rounds
    # graph j replays calls j*L .. j*L+L-1; P graphs bring the KV copy back to where graph 0 starts
    assert (P * L) % ncopies == 0 and all((j * L) % ncopies != 0 for j in range(1, P))


def test_graph_plan_uses_full_graphs_for_long_runs():
    L, P, replays, rounds = bench.graph_plan(4000, 8)
    assert (L, rounds) == (32, 20) and replays == 125
    assert bench.graph_plan(20, 8)[:1] == (2,)


def test_gpus_above_one_exit_with_a_message(capsys):
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
