"""Host-side arithmetic of bench.py: the graph blocks cover exactly the
warm-up and timed steps for any step counts (the driver runs
``bench.py --gpus 1 --steps 20 --warmup 5``), the one-GPU guard, and the
CPU baseline's process pool on the tiny workload.  No GPU is touched."""
import itertools
import subprocess
import sys

import pytest

import bench


def _cover(blocks):
    steps = []
    for i0, n in blocks:
        assert n >= 1
        steps.extend(range(i0, i0 + n))
    return steps


@pytest.mark.parametrize("steps,warmup", [(20, 5), (1, 0), (7, 3), (1000, 50), (25, 25), (26, 24), (3, 100)])
@pytest.mark.parametrize("per_graph", [1, 5, 25, 64])
def test_graph_blocks_cover_exactly(steps, warmup, per_graph):
    wb = bench.graph_blocks(0, warmup, per_graph)
    tb = bench.graph_blocks(warmup, steps, per_graph)
    assert _cover(wb) == list(range(warmup))
    assert _cover(tb) == list(range(warmup, warmup + steps))
    for _, n in wb + tb:
        assert n <= per_graph
    # whole blocks first, at most one shorter block at the end of each phase
    for blocks in (wb, tb):
        assert all(n == per_graph for _, n in blocks[:-1])


def test_driver_arguments_parse():
    a = bench.parse(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (a.gpus, a.steps, a.warmup) == (1, 20, 5)
    assert a.workload == bench.HEADLINE
    tb = bench.graph_blocks(a.warmup, a.steps, bench.steps_per_graph(1.3e-3, a.steps_per_graph))
    assert sum(n for _, n in tb) == 20


def test_steps_per_graph_bounds():
    for est, cap in itertools.product([1e-7, 7e-6, 2.4e-5, 1.3e-3, 1.0], [1, 25]):
        s = bench.steps_per_graph(est, cap)
        assert 1 <= s <= cap


def test_percentiles():
    p = bench.percentiles([5.0, 1.0, 3.0, 2.0, 4.0])
    assert p["p50"] == 3.0 and p["p10"] == pytest.approx(1.4) and p["p90"] == pytest.approx(4.6)
    assert bench.percentiles([2.5]) == dict(p10=2.5, p50=2.5, p90=2.5)


def test_headline_bound_is_the_matrix_cores():
    import synth
    assert bench.attention_bound(synth.workload_by_name(bench.HEADLINE)) == "mfma"
    for i in (0, 1, 2, 4):
        assert bench.attention_bound(synth.WORKLOADS[i]) == "hbm"


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_pool_on_tiny_workload():
    import synth
    x = synth.make_inputs(synth.WORKLOADS[0])
    r = bench.cpu_baseline(x, 0.5, 2)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s" and r["value"] > 0
    assert r["cores"] == 1            # one request: one worker
    assert r["host_cpus"] >= 1
