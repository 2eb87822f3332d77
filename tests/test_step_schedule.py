"""Host logic of KfacStep's two-stream schedule (no GPU): which inverses go to the
second stream."""
import synth
from fac_second_order_amd.step import side_split


def test_resnet50_long_sweeps_are_the_three_4609_factors():
    layers = synth.conv_layers(32)
    n_all = [l.c_in * l.kh * l.kw + (1 if l.bias else 0) for l in layers] + [l.c_out for l in layers]
    side = side_split(n_all)
    assert [n_all[i] for i in side] == [4609, 4609, 4609]
    assert all(2 * n <= 4609 + 2 for i, n in enumerate(n_all) if i not in side)


def test_no_second_stream_for_short_or_uniform_batches():
    assert side_split([64, 16]) == []            # a small layer
    assert side_split([577, 64]) == []           # longest sweep under 8 block steps
    assert side_split([2048, 2048, 2049]) == []  # every matrix long: nothing left to overlap
    assert side_split([]) == []


def test_half_the_largest_order_is_the_cut():
    assert side_split([2048, 1025, 1024]) == [0]   # 2 * 1025 = 2050 is not above 2048 + 2
    assert side_split([2048, 1026, 1024]) == [0, 1]
