"""Host logic of KfacStep's two-stream schedule (no GPU): which inverses go to the
second stream, and the groups of layers of the caller's stream's calls."""
import synth
from fac_second_order_amd.step import KfacStep, side_split


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


def test_main_stream_call_groups():
    """The caller's stream splits its factor, preconditioning and BN calls into groups of
    layers: every group non-empty, in order, together exactly the input, at most the
    asked count, and no group above the even share by more than one layer's cost."""
    layers = synth.conv_layers(32)
    bns = synth.bn_layers(32)
    d_a = [l.c_in * l.kh * l.kw + (1 if l.bias else 0) for l in layers]
    for parts in (1, 2, 4, 7):
        for idx, cost in ((list(range(len(layers))), lambda l: d_a[l] ** 2 * layers[l].rows),
                          (list(range(len(bns))), lambda b: bns[b].hw * bns[b].c),
                          ([3], lambda i: 1.0), ([], lambda i: 1.0)):
            groups = KfacStep._groups(idx, cost, parts)
            assert [i for g in groups for i in g] == idx
            assert all(groups) and len(groups) <= parts
            if idx:
                share = sum(cost(i) for i in idx) / parts
                assert all(sum(cost(i) for i in g) <= share + max(cost(i) for i in g) for g in groups)
    assert len(KfacStep._groups(list(range(10)), lambda i: 1.0, 4)) == 4
