"""The algorithmic work bench.py divides by measured kernel time, checked on the CPU
against a closed form of the inverse sweep."""
import importlib.util
import os

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TB = 128


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def sweep_update_flops(n):
    """Step k of the sweep (block width b_k) subtracts a rank-b_k product from every
    entry on or above the diagonal outside block row and column k: the upper triangle
    of an order n - b_k matrix, 2 flops per multiply-add. An order 128m + 1 takes m
    block steps (its last column is a bordered step of the finish)."""
    nb = -(-n // TB)
    steps = n // TB if (n > TB and n % TB == 1) else nb
    total = 0
    for k in range(steps):
        b = min(TB, n - k * TB)
        r = n - b
        total += 2 * b * r * (r + 1) // 2
    return total


@pytest.mark.parametrize("group", [1, 2, 3, 4, 5, 6])
def test_grouping_only_moves_work(bench, group):
    """Grouped steps split the sweep's updates between the update launches and the row
    updates; together they are the whole sweep for every group size."""
    sizes = [1, 2, 64, 65, 127, 128, 129, 130, 256, 257, 300, 577, 1000, 1153, 2305]
    upd, row = bench.inverse_update_flops(sizes, group)
    assert upd + row == sum(sweep_update_flops(n) for n in sizes)
    if group == 1:
        assert row == 0


def test_resnet50_update_share(bench):
    layers = synth.conv_layers(32)
    n_all = [l.d_a for l in layers] + [l.d_g for l in layers]
    total = sum(sweep_update_flops(n) for n in n_all)
    upd, row = bench.inverse_update_flops(n_all, 4)
    assert upd + row == total
    # the updates are most of the method's sum of n^3 (the rest is pivots and panels)
    assert 0.85 < total / sum(n ** 3 for n in n_all) < 0.95


def test_measured_traffic_keyed_to_source_and_group(bench):
    """A measured byte count is reported only for the kernel, stream mode and group size
    it was measured with, and only while the kernel's source hashes to the recorded value."""
    for (name, side), (value, sha) in bench.MEASURED_TRAFFIC.items():
        group = next(g for g in range(1, 9) if bench.kernel_source_sha(name, g) == sha)
        assert bench.measured_traffic(name, side, group) == value
        assert bench.measured_traffic(name, not side, group) is None
        for other in range(1, 9):
            if other != group:
                assert bench.measured_traffic(name, side, other) is None
    assert bench.kernel_source_sha("gemm_tn_kernel", 6) is None
