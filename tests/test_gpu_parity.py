"""GPU parity of every C-ABI entry point against the fp64 oracle on identical seeded
inputs, at sizes the oracle finishes in seconds that span several tiles and ragged
edges, plus the edge cases (order 1, ragged blocks, breakdown, NaN, in place, EMA,
determinism).

Tolerances (relative Frobenius error, fp64):
  factors from fp16 inputs 1e-2, preconditioned gradients 2e-2, fp32 inverses at
  condition number <= 1e4: 1e-4 (the stated bars); packing and integer-input factors
  bit-exact; BatchNorm vectors 1e-4 (fp32 sums of at most ~1.5e3 terms per
  accumulator: n*u = 1.5e3 * 6e-8 = 9e-5).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import S_GAMMA, host, relF, say, to_dev

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# symmetric packing (bit-exact)
# ---------------------------------------------------------------------------

PACK_SIZES = [1, 2, 3, 63, 64, 65, 127, 128, 129, 577, 1000]


def test_pack_unpack_bitexact(kfac_gpu):
    rng = synth.layer_rng(1000, 0)
    mats = [rng.standard_normal((n, n)).astype(np.float32) for n in PACK_SIZES]
    full = [to_dev(m) for m in mats]
    packed = [torch.full((n * (n + 1) // 2,), np.nan, device=full[0].device) for n in PACK_SIZES]
    say("kfac_pack_sym direction 0, sizes", PACK_SIZES)
    kfac_gpu.kfac_pack_sym(PACK_SIZES, full, packed, 0)
    for n, m, p in zip(PACK_SIZES, mats, packed):
        assert np.array_equal(host(p), oracle.pack_upper(m)), n
    out = [torch.full((n, n), np.nan, device=full[0].device) for n in PACK_SIZES]
    say("kfac_pack_sym direction 1")
    kfac_gpu.kfac_pack_sym(PACK_SIZES, out, packed, 1)
    for n, m, o in zip(PACK_SIZES, mats, out):
        assert np.array_equal(host(o), oracle.unpack_upper(oracle.pack_upper(m), n)), n
    # direction 2: upper triangle only, the strict lower triangle keeps its contents
    base = [rng.standard_normal((n, n)).astype(np.float32) for n in PACK_SIZES]
    out = [to_dev(b) for b in base]
    say("kfac_pack_sym direction 2")
    kfac_gpu.kfac_pack_sym(PACK_SIZES, out, packed, 2)
    for n, m, b, o in zip(PACK_SIZES, mats, base, out):
        want = np.where(np.triu(np.ones((n, n), dtype=bool)),
                        oracle.unpack_upper(oracle.pack_upper(m), n), b)
        assert np.array_equal(host(o), want), n
    # direction 2 from packed buffers that are only 4-byte aligned (element loads)
    sizes = [3, 129, 577]
    src = [oracle.pack_upper(m) for m in mats if m.shape[0] in sizes]
    store = [torch.zeros(p.size + 1, device="cuda") for p in src]
    views = []
    for st_, p in zip(store, src):
        st_[1:] = to_dev(p)
        views.append(st_[1:])
    base = [rng.standard_normal((n, n)).astype(np.float32) for n in sizes]
    out = [to_dev(b) for b in base]
    say("kfac_pack_sym direction 2, unaligned packed", sizes)
    kfac_gpu.kfac_pack_sym(sizes, out, views, 2)
    for n, p, b, o in zip(sizes, src, base, out):
        want = np.where(np.triu(np.ones((n, n), dtype=bool)), oracle.unpack_upper(p, n), b)
        assert np.array_equal(host(o), want), n
    # direction 2 into full matrices that are only 4-byte aligned, at an order whose packed
    # array spans several 16,384-float slices (row segments cross slice boundaries)
    sizes = [577, 1000, 2049]
    mats2 = [rng.standard_normal((n, n)).astype(np.float32) for n in sizes]
    src = [oracle.pack_upper(m) for m in mats2]
    base = [rng.standard_normal((n, n)).astype(np.float32) for n in sizes]
    fstore = [torch.zeros(n * n + 1, device="cuda") for n in sizes]
    fviews = []
    for st_, b in zip(fstore, base):
        st_[1:] = to_dev(b).reshape(-1)
        fviews.append(st_[1:].view(b.shape))
        assert fviews[-1].data_ptr() % 16 == 4
    say("kfac_pack_sym direction 2, unaligned full", sizes)
    kfac_gpu.kfac_pack_sym(sizes, fviews, [to_dev(p) for p in src], 2)
    for n, p, b, o in zip(sizes, src, base, fviews):
        want = np.where(np.triu(np.ones((n, n), dtype=bool)), oracle.unpack_upper(p, n), b)
        assert np.array_equal(host(o), want), n


# ---------------------------------------------------------------------------
# BatchNorm diagonal Fisher
# ---------------------------------------------------------------------------

BN_CASES = [synth.BNLayer("a", 3, 7, 5), synth.BNLayer("b", 2, 49, 64),
            synth.BNLayer("c", 4, 300, 24), synth.BNLayer("d", 2, 3, 2050),
            synth.BNLayer("e", 1, 1, 1), synth.BNLayer("f", 5, 1000, 8)]


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_bn_diag(kfac_gpu, dtype):
    rng = synth.layer_rng(1001, 0)
    xs = [rng.standard_normal(b.shape).astype(dtype) for b in BN_CASES]
    gs = [(rng.standard_normal(b.shape) * 0.1).astype(dtype) for b in BN_CASES]
    F = [torch.zeros(2, b.c, device="cuda") for b in BN_CASES]
    P = [torch.zeros(2, b.c, device="cuda") for b in BN_CASES]
    say("kfac_bn_diag", dtype.__name__, [b.shape for b in BN_CASES])
    kfac_gpu.kfac_bn_diag(BN_CASES, [to_dev(x) for x in xs], [to_dev(g) for g in gs], F, P, 0.0, 1e-3)
    refs = []
    for i, b in enumerate(BN_CASES):
        ref = oracle.bn_diag_fisher(xs[i], gs[i], 1e-3)
        refs.append(ref)
        assert relF(host(F[i]), ref["fisher"]) <= 1e-4, b
        assert relF(host(P[i]), ref["precond"]) <= 1e-4, b
    # moving average with the stored Fisher, and decay 1 (stale Fisher, fresh gradient)
    xs2 = [rng.standard_normal(b.shape).astype(dtype) for b in BN_CASES]
    say("kfac_bn_diag ema 0.95")
    kfac_gpu.kfac_bn_diag(BN_CASES, [to_dev(x) for x in xs2], [to_dev(g) for g in gs], F, P, 0.95, 1e-3)
    for i, b in enumerate(BN_CASES):
        ref = oracle.bn_diag_fisher(xs2[i], gs[i], 1e-3, 0.95, refs[i]["fisher"])
        assert relF(host(F[i]), ref["fisher"]) <= 1e-4, b
        assert relF(host(P[i]), ref["precond"]) <= 1e-4, b
        refs[i] = ref
    say("kfac_bn_diag stale (decay 1)")
    F_before = [host(f) for f in F]
    kfac_gpu.kfac_bn_diag(BN_CASES, [to_dev(x) for x in xs], [to_dev(g) for g in gs], F, P, 1.0, 1e-3)
    for i, b in enumerate(BN_CASES):
        fresh = oracle.bn_diag_fisher(xs[i], gs[i], 1e-3)
        assert np.array_equal(host(F[i]), F_before[i]), b
        assert relF(host(P[i]), fresh["grad"] / (F_before[i].astype(np.float64) + 1e-3)) <= 1e-4, b


# ---------------------------------------------------------------------------
# factors
# ---------------------------------------------------------------------------

FACTOR_LAYERS = [
    synth.Layer("c3x3p1", 2, 9, 7, 16, 9, 7, 24, 3, 3, 1, 1, 1, 1, 1),
    synth.Layer("c3x3s2", 3, 10, 10, 8, 5, 5, 8, 3, 3, 2, 2, 1, 1, 1),
    synth.Layer("conv1like", 2, 15, 15, 3, 8, 8, 16, 7, 7, 2, 2, 3, 3, 1),
    synth.Layer("c1x1", 2, 6, 6, 136, 6, 6, 200, 1, 1, 1, 1, 0, 0, 1),
    synth.Layer("c1x1s2", 2, 7, 7, 40, 4, 4, 12, 1, 1, 2, 2, 0, 0, 1),
    synth.Layer("fc_nobias", 5, 1, 1, 130, 1, 1, 3, 1, 1, 1, 1, 0, 0, 0),
    synth.Layer("c3x3big", 2, 12, 12, 32, 12, 12, 64, 3, 3, 1, 1, 1, 1, 1),   # d_A = 289
]


def _oracle_factors(layer, act, gout):
    return oracle.conv_factors(act, gout, layer.kh, layer.kw, layer.sh, layer.sw,
                               layer.ph, layer.pw, layer.bias)


def _run_factors(kfac, layers, act, gout, ema=0.0, A=None, G=None):
    if A is None:
        A = [torch.full((l.d_a * (l.d_a + 1) // 2,), np.nan, device="cuda") for l in layers]
        G = [torch.full((l.d_g * (l.d_g + 1) // 2,), np.nan, device="cuda") for l in layers]
    kfac.kfac_factors(layers, [to_dev(a) for a in act], [to_dev(g) for g in gout], A, G, ema)
    return A, G


def test_factors_fp16_geometries(kfac_gpu):
    rng = synth.layer_rng(1002, 0)
    act = [synth.relu_normal_f16(rng, l.act_shape) for l in FACTOR_LAYERS]
    gout = [synth.normal_f16(rng, l.gout_shape, 0.1) for l in FACTOR_LAYERS]
    say("kfac_factors fp16", [l.name for l in FACTOR_LAYERS])
    A, G = _run_factors(kfac_gpu, FACTOR_LAYERS, act, gout)
    for l, layer in enumerate(FACTOR_LAYERS):
        Ar, Gr = _oracle_factors(layer, act[l], gout[l])
        ea = relF(host(A[l]), oracle.pack_upper(Ar))
        eg = relF(host(G[l]), oracle.pack_upper(Gr))
        say(f"  {layer.name}: A relF {ea:.2e}  G relF {eg:.2e}")
        assert ea <= 1e-2 and eg <= 1e-2, layer.name


def test_factors_element_gathers(kfac_gpu):
    """Activation tensors whose base is not 16-byte aligned take the per-element
    gathers of the patch matrix (2-byte loads with bounds checks per tap), in the
    gather form (3x3, strided 1x1) and the row form (1x1 stride 1, G factors)."""
    layers = [synth.Layer("c3x3", 3, 9, 7, 16, 9, 7, 24, 3, 3, 1, 1, 1, 1, 1),
              synth.Layer("c1x1s2", 2, 9, 9, 24, 5, 5, 16, 1, 1, 2, 2, 0, 0, 1),
              synth.Layer("c1x1", 2, 6, 6, 32, 6, 6, 8, 1, 1, 1, 1, 0, 0, 0),
              # shaped for 256x256 tiles, which need 16-byte gathers: 128x128 tiles instead
              synth.Layer("c1x1_256", 2, 6, 6, 256, 6, 6, 264, 1, 1, 1, 1, 0, 0, 1)]
    rng = synth.layer_rng(1012, 0)
    act = [synth.relu_normal_f16(rng, l.act_shape) for l in layers]
    gout = [synth.normal_f16(rng, l.gout_shape, 0.1) for l in layers]

    def offset_by_one(a):      # same values at a base 2 bytes past a 16-byte boundary
        buf = torch.empty(a.size + 8, dtype=torch.float16, device="cuda")
        view = buf[1:1 + a.size].view(a.shape)
        view.copy_(torch.from_numpy(a))
        assert view.data_ptr() % 16 == 2
        return view

    A = [torch.full((l.d_a * (l.d_a + 1) // 2,), np.nan, device="cuda") for l in layers]
    G = [torch.full((l.d_g * (l.d_g + 1) // 2,), np.nan, device="cuda") for l in layers]
    say("kfac_factors with misaligned inputs (element gathers)")
    kfac_gpu.kfac_factors(layers, [offset_by_one(a) for a in act], [offset_by_one(g) for g in gout], A, G)
    for l, layer in enumerate(layers):
        Ar, Gr = _oracle_factors(layer, act[l], gout[l])
        ea, eg = relF(host(A[l]), oracle.pack_upper(Ar)), relF(host(G[l]), oracle.pack_upper(Gr))
        say(f"  {layer.name}: A relF {ea:.2e}  G relF {eg:.2e}")
        assert ea <= 1e-2 and eg <= 1e-2, layer.name


def test_factors_integer_inputs_bitexact(kfac_gpu):
    """Inputs in {-2..2}: fp32 sums are exact integers, so each output is the single
    fp32 product fp32(sum) * fp32(1/R)."""
    rng = synth.layer_rng(1003, 0)
    act = [rng.integers(-2, 3, size=l.act_shape).astype(np.float16) for l in FACTOR_LAYERS]
    gout = [rng.integers(-2, 3, size=l.gout_shape).astype(np.float16) for l in FACTOR_LAYERS]
    say("kfac_factors integer inputs")
    A, G = _run_factors(kfac_gpu, FACTOR_LAYERS, act, gout)
    for l, layer in enumerate(FACTOR_LAYERS):
        X = oracle.im2col_nhwc(act[l], layer.kh, layer.kw, layer.sh, layer.sw, layer.ph, layer.pw,
                               layer.bias)
        Gam = gout[l].astype(np.float64).reshape(-1, layer.c_out)
        inv_r = np.float32(1.0) / np.float32(X.shape[0])
        for got, S in ((A[l], oracle.gram(X)), (G[l], oracle.gram(Gam))):
            expect = oracle.pack_upper(S).astype(np.float32) * inv_r
            assert np.array_equal(host(got), expect), layer.name


SHIFT_EDGE_LAYERS = [   # 3x3, stride 1, padding 1: factors formed from shift products
    synth.Layer("row_image", 2, 1, 5, 8, 1, 5, 8, 3, 3, 1, 1, 1, 1, 0),
    synth.Layer("column_image", 1, 4, 1, 24, 4, 1, 16, 3, 3, 1, 1, 1, 1, 1),
    synth.Layer("two_row_blocks", 3, 2, 3, 136, 2, 3, 8, 3, 3, 1, 1, 1, 1, 1),
    synth.Layer("single_pixel", 4, 1, 1, 16, 1, 1, 8, 3, 3, 1, 1, 1, 1, 1),
]


def test_factors_shift_products_edge_cases(kfac_gpu):
    """[OTUNYM] eq. (5) for 3x3 stride-1 convolutions on images of one row, one
    column, one pixel and with more than 128 channels, integer inputs: bit-exact, as
    every sum (the shift products, their border strips and corners) is an exact integer."""
    rng = synth.layer_rng(1013, 0)
    act = [rng.integers(-2, 3, size=l.act_shape).astype(np.float16) for l in SHIFT_EDGE_LAYERS]
    gout = [rng.integers(-2, 3, size=l.gout_shape).astype(np.float16) for l in SHIFT_EDGE_LAYERS]
    say("kfac_factors shift-product edge cases")
    A, G = _run_factors(kfac_gpu, SHIFT_EDGE_LAYERS, act, gout)
    for l, layer in enumerate(SHIFT_EDGE_LAYERS):
        X = oracle.im2col_nhwc(act[l], 3, 3, 1, 1, 1, 1, layer.bias)
        inv_r = np.float32(1.0) / np.float32(X.shape[0])
        expect = oracle.pack_upper(oracle.gram(X)).astype(np.float32) * inv_r
        assert np.array_equal(host(A[l]), expect), layer.name


# Factors of order >= 1024 and the shift products of 3x3 layers with >= 256 channels run
# on 256x256 tiles: direct and split-reduced results, the bias column, rows and columns
# that end inside a tile (264, 1032, 1040 channels), both gather forms (rows, strided 1x1
# gathers) and tiles off the diagonal. Orders 256-512 next to them take 128x128 tiles.
BIG_TILE_LAYERS = [
    synth.Layer("c3x3_256", 2, 8, 8, 256, 8, 8, 256, 3, 3, 1, 1, 1, 1, 1),           # A 2305, G 256
    synth.Layer("c3x3_264_split", 40, 8, 8, 264, 8, 8, 24, 3, 3, 1, 1, 1, 1, 1),     # R = 2560
    synth.Layer("c1x1_1032_split", 48, 8, 8, 1032, 8, 8, 1040, 1, 1, 1, 1, 0, 0, 1),  # R = 3072
    synth.Layer("c1x1s2_1024", 2, 10, 10, 1024, 5, 5, 1024, 1, 1, 2, 2, 0, 0, 1),
    synth.Layer("fc_1024", 64, 1, 1, 1024, 1, 1, 1000, 1, 1, 1, 1, 0, 0, 0),
    synth.Layer("c1x1_296_split", 48, 8, 8, 296, 8, 8, 320, 1, 1, 1, 1, 0, 0, 1),
    synth.Layer("fc_512", 64, 1, 1, 512, 1, 1, 264, 1, 1, 1, 1, 0, 0, 0),
]


def test_factors_big_tiles_integer_bitexact(kfac_gpu):
    """[OTUNYM] eq. (5) through the 256x256-tile path (and 128x128 tiles for the orders
    below 1024) with inputs in {-2..2}: every sum
    is an exact integer, so each output is fp32(sum) * fp32(1/R), bit for bit."""
    rng = synth.layer_rng(1014, 0)
    act = [rng.integers(-2, 3, size=l.act_shape).astype(np.float16) for l in BIG_TILE_LAYERS]
    gout = [rng.integers(-2, 3, size=l.gout_shape).astype(np.float16) for l in BIG_TILE_LAYERS]
    say("kfac_factors 256x256 tiles, integer inputs", [l.name for l in BIG_TILE_LAYERS])
    A, G = _run_factors(kfac_gpu, BIG_TILE_LAYERS, act, gout)
    for l, layer in enumerate(BIG_TILE_LAYERS):
        X = oracle.im2col_nhwc(act[l], layer.kh, layer.kw, layer.sh, layer.sw, layer.ph, layer.pw,
                               layer.bias)
        Gam = gout[l].astype(np.float64).reshape(-1, layer.c_out)
        inv_r = np.float32(1.0) / np.float32(X.shape[0])
        for which, got, S in (("A", A[l], oracle.gram(X)), ("G", G[l], oracle.gram(Gam))):
            expect = oracle.pack_upper(S).astype(np.float32) * inv_r
            g = host(got)
            bad = int(np.count_nonzero(g != expect))
            say(f"  {layer.name} {which}: {bad} of {g.size} entries differ")
            assert bad == 0, (layer.name, which)


def test_factors_big_tiles_fp16(kfac_gpu):
    """The same layers with fp16 ReLU activations and Gaussian output gradients: relF
    against the fp64 oracle, and bitwise identical results from a second call."""
    rng = synth.layer_rng(1015, 0)
    act = [synth.relu_normal_f16(rng, l.act_shape) for l in BIG_TILE_LAYERS]
    gout = [synth.normal_f16(rng, l.gout_shape, 0.1) for l in BIG_TILE_LAYERS]
    say("kfac_factors 256x256 tiles, fp16")
    A, G = _run_factors(kfac_gpu, BIG_TILE_LAYERS, act, gout)
    A2, G2 = _run_factors(kfac_gpu, BIG_TILE_LAYERS, act, gout)
    for x, y in zip(A + G, A2 + G2):
        assert torch.equal(x, y)
    for l, layer in enumerate(BIG_TILE_LAYERS):
        Ar, Gr = _oracle_factors(layer, act[l], gout[l])
        ea = relF(host(A[l]), oracle.pack_upper(Ar))
        eg = relF(host(G[l]), oracle.pack_upper(Gr))
        say(f"  {layer.name}: A relF {ea:.2e}  G relF {eg:.2e}")
        # fp16 products are exact in fp32; fp32 sums of R <= 3072 terms, typically
        # ~sqrt(R) u = 3e-6 relative: well inside the stated 1e-2 bar
        assert ea <= 1e-4 and eg <= 1e-4, layer.name


def _upper_bits(full):
    d = full.shape[0]
    iu = torch.triu_indices(d, d, device=full.device)
    return full[iu[0], iu[1]].view(torch.int32), full[iu[1], iu[0]][iu[0] != iu[1]]


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_factors_full_matches_packed(kfac_gpu, dtype):
    """kfac_factors_full: each full matrix's upper triangle holds the packed factor's
    bits (what direction 2 of kfac_pack_sym writes) and its strict lower triangle is
    left alone, through every kernel path (256x256 and 128x128 tiles, direct and split,
    shift products and their assembly, conv1's patch rows, fp32 inputs), with and
    without the EMA blend; the packed factors equal those of kfac_factors."""
    layers = FACTOR_LAYERS + (BIG_TILE_LAYERS if dtype == torch.float16 else [])
    rng = synth.layer_rng(1016, 0)
    np_dt = np.float16 if dtype == torch.float16 else np.float32
    inputs = []
    for _ in range(2):
        inputs.append(([to_dev(synth.relu_normal_f16(rng, l.act_shape).astype(np_dt)) for l in layers],
                       [to_dev(synth.normal_f16(rng, l.gout_shape, 0.1).astype(np_dt)) for l in layers]))
    sentinel = -7.25
    A = [torch.full((l.d_a * (l.d_a + 1) // 2,), np.nan, device="cuda") for l in layers]
    G = [torch.full((l.d_g * (l.d_g + 1) // 2,), np.nan, device="cuda") for l in layers]
    Af = [torch.full((l.d_a, l.d_a), sentinel, device="cuda") for l in layers]
    Gf = [torch.full((l.d_g, l.d_g), sentinel, device="cuda") for l in layers]
    A_ref = [torch.full_like(x, np.nan) for x in A]
    G_ref = [torch.full_like(x, np.nan) for x in G]
    for step, ema in enumerate((0.0, 0.75)):
        act, gout = inputs[step]
        say(f"kfac_factors_full {dtype} ema {ema}", [l.name for l in layers])
        kfac_gpu.kfac_factors_full(layers, act, gout, A, G, Af, Gf, ema)
        kfac_gpu.kfac_factors(layers, act, gout, A_ref, G_ref, ema)
        torch.cuda.synchronize()
        for l, layer in enumerate(layers):
            for packed, ref, full in ((A[l], A_ref[l], Af[l]), (G[l], G_ref[l], Gf[l])):
                up, low = _upper_bits(full)
                assert torch.equal(packed.view(torch.int32), ref.view(torch.int32)), layer.name
                assert torch.equal(up, packed.view(torch.int32)), layer.name
                assert bool((low == sentinel).all()), layer.name
    # a NULL entry leaves that full matrix alone
    keep = Af[0].clone()
    kfac_gpu.kfac_factors_full(layers, inputs[0][0], inputs[0][1], A, G, [None] + Af[1:], Gf, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(Af[0], keep)


def test_factors_fp32_fc_and_kronecker(kfac_gpu):
    """The fc workload in fp32 (a[32x64], g[32x16], no bias): factors, damped inverses
    and G^-1 dW A^-1 through the library, checked against the oracle and against the
    explicit 1024x1024 Kronecker solve."""
    seed = synth.config_seed("fc")
    a = synth.normal_f32(synth.layer_rng(seed, 0), (32, 64))
    g = synth.normal_f32(synth.layer_rng(seed, 1), (32, 16))
    dW = (g.astype(np.float64).T @ a.astype(np.float64)) / 32.0
    layer = synth.Layer("fc", 32, 1, 1, 64, 1, 1, 16, 1, 1, 1, 1, 0, 0, 0)
    st = kfac_gpu.KfacStep([layer], [], "cuda", in_dtype=torch.float32)
    say("fc fp32 chain")
    st.factors([to_dev(a.reshape(32, 1, 1, 64))], [to_dev(g.reshape(32, 1, 1, 16))])
    st.invert()
    st.precondition([to_dev(dW.astype(np.float32))])
    A, G = oracle.conv_factors(a.reshape(32, 1, 1, 64), g.reshape(32, 1, 1, 16), 1, 1, 1, 1, 0, 0, 0)
    assert relF(host(st.A_packed[0]), oracle.pack_upper(A)) <= 1e-5
    assert relF(host(st.G_packed[0]), oracle.pack_upper(G)) <= 1e-5
    Ai, _ = oracle.damped_inverse(A, S_GAMMA)
    Gi, _ = oracle.damped_inverse(G, S_GAMMA)
    assert relF(host(st.A_inv[0]), Ai) <= 1e-4
    assert relF(host(st.G_inv[0]), Gi) <= 1e-4
    K = np.kron(G + S_GAMMA * np.eye(16), A + S_GAMMA * np.eye(64))
    ref = np.linalg.solve(K, dW.reshape(-1)).reshape(16, 64)
    e = relF(host(st.out[0]), ref)
    say(f"  P vs Kronecker solve relF {e:.2e}")
    assert e <= 2e-2
    assert int(host(st.info).sum()) == 0


def test_factors_ema_and_determinism(kfac_gpu):
    rng = synth.layer_rng(1004, 0)
    layers = FACTOR_LAYERS[:4]
    act = [synth.relu_normal_f16(rng, l.act_shape) for l in layers]
    gout = [synth.normal_f16(rng, l.gout_shape, 0.1) for l in layers]
    act2 = [synth.relu_normal_f16(rng, l.act_shape) for l in layers]
    say("kfac_factors determinism + ema")
    A1, G1 = _run_factors(kfac_gpu, layers, act, gout)
    A2, G2 = _run_factors(kfac_gpu, layers, act, gout)
    for x, y in zip(A1 + G1, A2 + G2):
        assert torch.equal(x, y)
    _run_factors(kfac_gpu, layers, act2, gout, ema=0.95, A=A1, G=G1)
    for l, layer in enumerate(layers):
        Ar, Gr = _oracle_factors(layer, act[l], gout[l])
        Ar2, Gr2 = _oracle_factors(layer, act2[l], gout[l])
        assert relF(host(A1[l]), oracle.pack_upper(oracle.ema_update(Ar, Ar2, 0.95))) <= 1e-2
        assert relF(host(G1[l]), oracle.pack_upper(oracle.ema_update(Gr, Gr2, 0.95))) <= 1e-2


def test_factors_skip_null(kfac_gpu):
    """A NULL activation skips that A factor and leaves its buffer untouched."""
    layer = FACTOR_LAYERS[0]
    rng = synth.layer_rng(1005, 0)
    act = synth.relu_normal_f16(rng, layer.act_shape)
    gout = synth.normal_f16(rng, layer.gout_shape, 0.1)
    A = [torch.full((layer.d_a * (layer.d_a + 1) // 2,), 7.0, device="cuda")]
    G = [torch.zeros(layer.d_g * (layer.d_g + 1) // 2, device="cuda")]
    kfac_gpu.kfac_factors([layer], [None], [to_dev(gout)], A, G)
    assert bool((A[0] == 7.0).all())
    _, Gr = _oracle_factors(layer, act, gout)
    assert relF(host(G[0]), oracle.pack_upper(Gr)) <= 1e-2


# ---------------------------------------------------------------------------
# damped inverses
# ---------------------------------------------------------------------------

INV_SIZES = [1, 2, 3, 31, 64, 65, 127, 128, 129, 200, 257, 300, 513]


def spd_factor(rng, n, kappa):
    """Symmetric factor F (fp32) with cond(F + 1e-3 I) <= kappa: Gram of a
    log-scaled Gaussian matrix with 4n rows, rescaled by its largest eigenvalue."""
    sig = np.logspace(0, -3, n)
    X = rng.standard_normal((4 * n, n)) * sig
    F = X.T @ X / (4 * n)
    lam = np.linalg.eigvalsh(F)[-1]
    F *= (kappa - 1) * 1e-3 / lam
    return F.astype(np.float32)


def test_invert_sizes_and_chol(kfac_gpu):
    rng = synth.layer_rng(1006, 0)
    Fs = [spd_factor(rng, n, 1e4) for n in INV_SIZES]
    mat = [to_dev(F) for F in Fs]
    inv = [torch.full((n, n), np.nan, device="cuda") for n in INV_SIZES]
    chol = [torch.zeros(n, n, device="cuda") for n in INV_SIZES]
    info = torch.full((len(INV_SIZES),), -7, dtype=torch.int32, device="cuda")
    say("kfac_invert sizes", INV_SIZES)
    kfac_gpu.kfac_invert(INV_SIZES, mat, inv, [1e-3] * len(INV_SIZES), info, chol)
    assert host(info).tolist() == [0] * len(INV_SIZES)
    for n, F, X, U in zip(INV_SIZES, Fs, inv, chol):
        M = F.astype(np.float64) + 1e-3 * np.eye(n)
        ref, _ = oracle.damped_inverse(F, 1e-3)
        x = host(X)
        e = relF(x, ref)
        Uref, _ = oracle.cholesky_upper(M)
        eu = relF(np.triu(host(U)), Uref)
        say(f"  n={n}: inverse relF {e:.2e}  chol relF {eu:.2e}  cond {np.linalg.cond(M):.1e}")
        assert np.array_equal(x, x.T), n
        assert e <= 1e-4, n
        assert eu <= 1e-4, n


def test_invert_in_place_matches(kfac_gpu):
    rng = synth.layer_rng(1007, 0)
    sizes = [129, 300]
    Fs = [spd_factor(rng, n, 1e3) for n in sizes]
    a = [to_dev(F) for F in Fs]
    b = [to_dev(F) for F in Fs]
    out = [torch.empty(n, n, device="cuda") for n in sizes]
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    kfac_gpu.kfac_invert(sizes, a, out, [1e-3, 1e-3], info)
    kfac_gpu.kfac_invert(sizes, b, b, [1e-3, 1e-3], info)
    for x, y in zip(out, b):
        assert torch.equal(x, y)


def _device_factors(sizes, seed):
    """Damped-Gram SPD factors drawn and formed on the device (inputs only)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    out = []
    for n in sizes:
        X = torch.randn(4 * n, n, device="cuda", generator=g) * torch.logspace(0, -3, n, device="cuda")
        out.append((X.t().contiguous() @ X) / (4 * n))
    return out


@pytest.mark.timeout(300)
def test_invert_concurrent_streams_bitexact(kfac_gpu):
    """Two inversion calls running at the same time on two streams, with a matrix
    product competing for the compute units, give bit-for-bit the results of the same
    calls run alone. Regression test for the panel step, whose two blocks per tile
    once read the whole tile and wrote their halves of it back in place: a block
    delayed behind other work could then read rows its partner had overwritten."""
    big, small = [2049, 2049, 1153], [1025, 577, 513, 257, 129, 65, 64]
    Fb, Fs = _device_factors(big, 71), _device_factors(small, 72)
    ref_b = [torch.empty_like(F) for F in Fb]
    ref_s = [torch.empty_like(F) for F in Fs]
    info_b = torch.zeros(len(big), dtype=torch.int32, device="cuda")
    info_s = torch.zeros(len(small), dtype=torch.int32, device="cuda")
    kfac_gpu.kfac_invert(big, Fb, ref_b, [1e-3] * len(big), info_b)
    kfac_gpu.kfac_invert(small, Fs, ref_s, [1e-3] * len(small), info_s)
    assert host(info_b).tolist() == [0] * len(big) and host(info_s).tolist() == [0] * len(small)
    ws_b = torch.empty(kfac_gpu.kfac_invert_workspace(big) + 256, dtype=torch.uint8, device="cuda")
    ws_s = torch.empty(kfac_gpu.kfac_invert_workspace(small) + 256, dtype=torch.uint8, device="cuda")
    busy = torch.randn(3072, 3072, device="cuda")
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(4):
        out_b = [torch.full_like(F, float("nan")) for F in Fb]
        out_s = [torch.full_like(F, float("nan")) for F in Fs]
        torch.cuda.synchronize()
        say(f"concurrent inversion, repetition {rep}: {big} on one stream, {small} and a 3072^2 product on another")
        with torch.cuda.stream(s0):
            busy2 = busy @ busy
            kfac_gpu.kfac_invert(small, Fs, out_s, [1e-3] * len(small), info_s, workspace=ws_s, stream=s0)
        kfac_gpu.kfac_invert(big, Fb, out_b, [1e-3] * len(big), info_b, workspace=ws_b, stream=s1)
        with torch.cuda.stream(s0):
            busy2 = busy2 @ busy
        torch.cuda.synchronize()
        assert host(info_b).tolist() == [0] * len(big) and host(info_s).tolist() == [0] * len(small)
        for x, r in zip(out_b + out_s, ref_b + ref_s):
            assert torch.equal(x, r), x.shape
    del busy2


def test_invert_breakdown_info(kfac_gpu):
    """Non-positive pivots report the 1-based column (LAPACK potrf convention),
    including in a later 128-block, at the bordered last column of an order
    128m + 1, and for NaN input."""
    n = 300
    cases = []
    F1 = np.eye(n, dtype=np.float32) * 2
    cases.append((F1, -3.0))                         # first pivot negative
    F2 = np.eye(n, dtype=np.float32) * 2
    F2[199, 199] = 0.5
    cases.append((F2, -1.0))                         # pivot 200 (second block) negative
    F3 = np.eye(n, dtype=np.float32)
    F3[5, 7] = np.nan
    cases.append((F3, 0.1))                          # NaN reaches pivot 8
    F4 = np.eye(4, dtype=np.float32)
    F4[2, 2] = 0.0
    cases.append((F4, 0.0))                          # exact zero pivot 3
    # orders 128m + 1 end with a bordered column (taken after the block sweep)
    F5 = np.eye(257, dtype=np.float32) * 2
    F5[256, 256] = 0.5
    cases.append((F5, -1.0))                         # last pivot (257) negative
    F6 = np.eye(129, dtype=np.float32)
    F6[5, 128] = np.nan
    cases.append((F6, 0.1))                          # NaN reaches the last pivot 129
    F7 = np.eye(129, dtype=np.float32) * 2
    F7[3, 3] = 0.5
    F7[128, 128] = 0.5
    cases.append((F7, -1.0))                         # pivot 4 fails first, the last one too
    sizes = [F.shape[0] for F, _ in cases]
    expect = []
    for F, s in cases:
        M = np.triu(F.astype(np.float64)) + np.triu(F.astype(np.float64), 1).T + s * np.eye(F.shape[0])
        expect.append(oracle.cholesky_upper(M)[1])
    assert expect == [1, 200, 8, 3, 257, 129, 4]
    mats = [to_dev(F) for F, _ in cases]
    info = torch.zeros(len(cases), dtype=torch.int32, device="cuda")
    say("kfac_invert breakdown cases")
    kfac_gpu.kfac_invert(sizes, mats, mats, [s for _, s in cases], info)
    assert host(info).tolist() == expect


# ---------------------------------------------------------------------------
# preconditioning
# ---------------------------------------------------------------------------

PRE_DIMS = [(16, 64), (64, 577), (100, 257), (3, 5), (129, 130), (1, 1)]


@pytest.mark.parametrize("gdtype", [np.float32, np.float16])
def test_precondition(kfac_gpu, gdtype):
    rng = synth.layer_rng(1008, 0)
    Gi = [rng.standard_normal((g, g)).astype(np.float32) for g, _ in PRE_DIMS]
    Ai = [rng.standard_normal((a, a)).astype(np.float32) for _, a in PRE_DIMS]
    Gi = [(x + x.T) / 2 for x in Gi]
    Ai = [(x + x.T) / 2 for x in Ai]
    grads = [(rng.standard_normal((g, a)) * 0.1).astype(gdtype) for g, a in PRE_DIMS]
    out = [torch.full((g, a), np.nan, device="cuda") for g, a in PRE_DIMS]
    say("kfac_precondition", gdtype.__name__, PRE_DIMS)
    kfac_gpu.kfac_precondition([g for g, _ in PRE_DIMS], [a for _, a in PRE_DIMS],
                               [to_dev(x) for x in Gi], [to_dev(x) for x in Ai],
                               [to_dev(x) for x in grads], out)
    for (g, a), G_, A_, dW, o in zip(PRE_DIMS, Gi, Ai, grads, out):
        e = relF(host(o), oracle.precondition(G_, dW, A_))
        assert e <= 2e-2, (g, a, e)
        assert e <= 1e-5, (g, a, e)   # fp32 products of exactly widened inputs


# ---------------------------------------------------------------------------
# parameter update of eq. (8), fused into the preconditioning and BN kernels
# ---------------------------------------------------------------------------

def test_precondition_update(kfac_gpu):
    """w <- w - lr * G^-1 dW A^-1 in the GEMM epilogue: the step equals -lr times the
    oracle's preconditioned gradient, the new weights equal the oracle's update, and
    storing P or not leaves the weights bit-identical."""
    rng = synth.layer_rng(1010, 0)
    lr = 0.37
    Gi = [rng.standard_normal((g, g)).astype(np.float32) for g, _ in PRE_DIMS]
    Ai = [rng.standard_normal((a, a)).astype(np.float32) for _, a in PRE_DIMS]
    Gi = [(x + x.T) / 2 for x in Gi]
    Ai = [(x + x.T) / 2 for x in Ai]
    grads = [(rng.standard_normal((g, a)) * 0.1).astype(np.float32) for g, a in PRE_DIMS]
    w0 = [rng.standard_normal((g, a)).astype(np.float32) for g, a in PRE_DIMS]
    dg, da = [g for g, _ in PRE_DIMS], [a for _, a in PRE_DIMS]
    args = ([to_dev(x) for x in Gi], [to_dev(x) for x in Ai], [to_dev(x) for x in grads])
    out = [torch.full((g, a), np.nan, device="cuda") for g, a in PRE_DIMS]
    w = [to_dev(x) for x in w0]
    say("kfac_precondition_update", PRE_DIMS)
    kfac_gpu.kfac_precondition_update(dg, da, *args, out, w, lr)
    for (g, a), G_, A_, dW, o, wn, wo in zip(PRE_DIMS, Gi, Ai, grads, out, w, w0):
        P = oracle.precondition(G_, dW, A_)
        assert relF(host(o), P) <= 1e-5, (g, a)
        step = host(wn).astype(np.float64) - wo
        assert relF(step, -lr * P) <= 2e-2, (g, a)
        assert relF(host(wn), oracle.sgd_update(wo, P, lr)) <= 1e-5, (g, a)
    say("kfac_precondition_update out=None")
    w2 = [to_dev(x) for x in w0]
    kfac_gpu.kfac_precondition_update(dg, da, *args, None, w2, lr)
    for a_, b_ in zip(w, w2):
        assert torch.equal(a_, b_)
    say("kfac_precondition_update lr=0")
    w3 = [to_dev(x) for x in w0]
    kfac_gpu.kfac_precondition_update(dg, da, *args, None, w3, 0.0)
    for a_, b_ in zip(w3, w0):
        assert np.array_equal(host(a_), b_)


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_bn_update(kfac_gpu, dtype):
    """gamma/beta <- gamma/beta - lr * precond in the BN finish kernel; fisher and
    precond as from kfac_bn_diag."""
    rng = synth.layer_rng(1011, 0)
    lr = 0.25
    xs = [rng.standard_normal(b.shape).astype(dtype) for b in BN_CASES]
    gs = [(rng.standard_normal(b.shape) * 0.1).astype(dtype) for b in BN_CASES]
    p0 = [rng.standard_normal((2, b.c)).astype(np.float32) for b in BN_CASES]
    F = [torch.zeros(2, b.c, device="cuda") for b in BN_CASES]
    P = [torch.zeros(2, b.c, device="cuda") for b in BN_CASES]
    prm = [to_dev(x) for x in p0]
    say("kfac_bn_update", dtype.__name__, [b.shape for b in BN_CASES])
    kfac_gpu.kfac_bn_update(BN_CASES, [to_dev(x) for x in xs], [to_dev(g) for g in gs], F, P, prm, lr,
                            0.0, 1e-3)
    for i, b in enumerate(BN_CASES):
        ref = oracle.bn_diag_fisher(xs[i], gs[i], 1e-3)
        assert relF(host(F[i]), ref["fisher"]) <= 1e-4, b
        assert relF(host(P[i]), ref["precond"]) <= 1e-4, b
        step = host(prm[i]).astype(np.float64) - p0[i]
        assert relF(step, -lr * ref["precond"]) <= 1e-4, b
        assert relF(host(prm[i]), oracle.sgd_update(p0[i], ref["precond"], lr)) <= 1e-4, b
        # the kernel's own update of its own precond is exact up to one fma rounding
        own = p0[i].astype(np.float64) - lr * host(P[i]).astype(np.float64)
        assert np.allclose(host(prm[i]), own, rtol=1e-6, atol=1e-6 * np.abs(own).max()), b


# ---------------------------------------------------------------------------
# preconditioning with fp64 accumulation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gdtype", [np.float32, np.float16])
def test_precondition_f64_accumulation(kfac_gpu, gdtype):
    """kfac_precondition_ex with KFAC_F64 on generic inputs: exact products summed in
    fp64, so only the fp32 intermediate and the output rounding remain."""
    rng = synth.layer_rng(1012, 0)
    Gi = [rng.standard_normal((g, g)).astype(np.float32) for g, _ in PRE_DIMS]
    Ai = [rng.standard_normal((a, a)).astype(np.float32) for _, a in PRE_DIMS]
    Gi = [(x + x.T) / 2 for x in Gi]
    Ai = [(x + x.T) / 2 for x in Ai]
    grads = [(rng.standard_normal((g, a)) * 0.1).astype(gdtype) for g, a in PRE_DIMS]
    w0 = [rng.standard_normal((g, a)).astype(np.float32) for g, a in PRE_DIMS]
    dg, da = [g for g, _ in PRE_DIMS], [a for _, a in PRE_DIMS]
    out = [torch.full((g, a), np.nan, device="cuda") for g, a in PRE_DIMS]
    w = [to_dev(x) for x in w0]
    lr = 0.25
    say("kfac_precondition_ex f64", gdtype.__name__, PRE_DIMS)
    kfac_gpu.kfac_precondition_ex(dg, da, [to_dev(x) for x in Gi], [to_dev(x) for x in Ai],
                                  [to_dev(x) for x in grads], out, w, lr, kfac_gpu.KFAC_F64)
    for (g, a), G_, A_, dW, o, wn, wo in zip(PRE_DIMS, Gi, Ai, grads, out, w, w0):
        P = oracle.precondition(G_, dW, A_)
        assert relF(host(o), P) <= 1e-6, (g, a)
        assert relF(host(wn), oracle.sgd_update(wo, P, lr)) <= 1e-6, (g, a)
    say("kfac_precondition_ex f64 without update")
    out2 = [torch.full((g, a), np.nan, device="cuda") for g, a in PRE_DIMS]
    kfac_gpu.kfac_precondition_ex(dg, da, [to_dev(x) for x in Gi], [to_dev(x) for x in Ai],
                                  [to_dev(x) for x in grads], out2, None, 0.0, kfac_gpu.KFAC_F64)
    for a_, b_ in zip(out, out2):
        assert torch.equal(a_, b_)


def test_precondition_cancellation(kfac_gpu):
    """A gradient in the range of rank-deficient factors (dW = Gamma^T X / R, factors
    from the same 8 rows, damping 1e-3): the products cancel by a factor rho, the fp32
    sums lose about rho*u, the fp64 sums do not. Inputs are the oracle's inverses
    rounded to fp32; the reference is their exact product."""
    rng = synth.layer_rng(1013, 0)
    R, dg, da = 8, 96, 1025
    X = np.maximum(rng.standard_normal((R, da)), 0.0)
    X[:, -1] = 1.0
    Gam = rng.standard_normal((R, dg))
    s = S_GAMMA
    Ai, _ = oracle.damped_inverse(X.T @ X / R, s)
    Gi, _ = oracle.damped_inverse(Gam.T @ Gam / R, s)
    Ai32, Gi32 = Ai.astype(np.float32), Gi.astype(np.float32)
    dW = (Gam.T @ X / R).astype(np.float32)
    P = oracle.precondition(Gi32.astype(np.float64), dW, Ai32.astype(np.float64))
    rho = np.linalg.norm(np.abs(Gi32) @ np.abs(dW) @ np.abs(Ai32)) / np.linalg.norm(P)
    errs = {}
    for name, accum in (("f32", kfac_gpu.KFAC_F32), ("f64", kfac_gpu.KFAC_F64)):
        out = [torch.full((dg, da), np.nan, device="cuda")]
        say("kfac_precondition_ex cancellation", name)
        kfac_gpu.kfac_precondition_ex([dg], [da], [to_dev(Gi32)], [to_dev(Ai32)], [to_dev(dW)], out, None, 0.0,
                                      accum)
        errs[name] = relF(host(out[0]), P)
    say(f"cancellation rho {rho:.2e}: relF f32 {errs['f32']:.2e}, f64 {errs['f64']:.2e}")
    assert rho > 1e3                                # the case is what it claims to be
    assert errs["f64"] <= 4 * 6e-8 * rho            # fp32 rounding of the intermediate only
    assert errs["f64"] <= 2e-2
    assert errs["f64"] < errs["f32"]


def _stress_factor(n, kappa, seed):
    """Exactly symmetric fp32 factor with cond(F + 1e-3 I) <= kappa, built as the stress
    set is (damped Gram of a log-scaled Gaussian matrix with 4n rows)."""
    from test_gpu_fullsize import resnet_factor
    F = resnet_factor(n, kappa, seed)
    return np.triu(F) + np.triu(F, 1).T


@pytest.mark.timeout(300)
def test_invert_refine(kfac_gpu):
    """One refinement step with the residual summed in fp64 takes fp32 inverses of damped
    factors at cond 1e4 from their fp32 error (up to ~1e-5 at n = 4609) to close to
    the rounding of the fp64 inverse: for every n >= 65 the refined error is at most a
    quarter of the unrefined one and at most 1e-6; the output stays exactly symmetric."""
    sizes = [1, 65, 129, 257, 300, 513, 1025, 2049, 4609]
    Fs = [_stress_factor(n, 1e4, 40 + i) for i, n in enumerate(sizes)]
    full = [to_dev(F) for F in Fs]
    inv = [torch.empty(n, n, device="cuda") for n in sizes]
    info = torch.zeros(len(sizes), dtype=torch.int32, device="cuda")
    say("kfac_invert + kfac_invert_refine sizes", sizes)
    kfac_gpu.kfac_invert(sizes, full, inv, [1e-3] * len(sizes), info)
    assert host(info).tolist() == [0] * len(sizes)
    before = [host(x).copy() for x in inv]
    kfac_gpu.kfac_invert_refine(sizes, full, [1e-3] * len(sizes), inv)
    for n, F, x0, X in zip(sizes, Fs, before, inv):
        ref, _ = oracle.damped_inverse(F, 1e-3)
        x = host(X)
        e0, e1 = relF(x0, ref), relF(x, ref)
        say(f"  n={n}: relF {e0:.2e} -> {e1:.2e}")
        assert np.array_equal(x, x.T), n
        assert e1 <= 1e-6, n
        if n >= 65:
            assert e1 <= e0 / 4, (n, e0, e1)


def test_invert_refine_rejects_overlap(kfac_gpu):
    """An inv buffer may overlap no mat and no other inv buffer (any byte); mat buffers
    may overlap each other (they are only read)."""
    buf = torch.zeros(200, device="cuda")

    def m(lo):          # a 4 x 4 matrix starting at float lo of buf
        return buf[lo:lo + 16].view(4, 4)

    cases = [
        ([4], [m(0)], [m(0)]),                        # the same buffer
        ([4, 4], [m(0), m(32)], [m(64), m(8)]),       # inv[1] partly over mat[0]
        ([4, 4], [m(0), m(32)], [m(32), m(64)]),      # inv[0] is mat[1]
        ([4, 4], [m(100), m(120)], [m(0), m(8)]),     # two inv buffers share bytes
    ]
    for n, mat, inv in cases:
        with pytest.raises(kfac_gpu.KfacError):
            kfac_gpu.kfac_invert_refine(n, mat, [0.0] * len(n), inv)
    kfac_gpu.kfac_invert_refine([4, 4], [m(100), m(108)], [0.0, 0.0], [m(0), m(16)])
    assert bool((buf == 0).all())     # zero matrices and zero inverses stay zero
