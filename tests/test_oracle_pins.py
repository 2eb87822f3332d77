"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin fixes the oracle by a closed form, an exact rational brute force written
independently here, a library routine in a special case, or an invariant. The
mutation tests at the end plant plausible mistakes in copies of oracle functions and
check that some pin fails, so the pins are known to bite.

Equation numbers refer to Osawa et al., "Large-scale distributed second-order
optimization using Kronecker-factored approximate curvature for deep convolutional
neural networks" (Sections 3.1-3.2).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
S_GAMMA = float(np.float32(np.sqrt(1e-3)))      # per-factor damping sqrt(gamma), gamma = 1e-3


def relF(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(x - ref) / np.linalg.norm(ref)


# ---------------------------------------------------------------------------
# helpers written independently of the oracle (plain Python, exact arithmetic)
# ---------------------------------------------------------------------------

def brute_patches(x, kh, kw, sh, sw, ph, pw, bias):
    """Patch rows by explicit loops over Python objects (ints or Fractions)."""
    n, h, w, c = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    ho = (h + 2 * ph - kh) // sh + 1
    wo = (w + 2 * pw - kw) // sw + 1
    rows = []
    for b in range(n):
        for oh in range(ho):
            for ow in range(wo):
                row = []
                for i in range(kh):
                    for j in range(kw):
                        for ci in range(c):
                            y, z = oh * sh + i - ph, ow * sw + j - pw
                            row.append(x[b][y][z][ci] if 0 <= y < h and 0 <= z < w else 0)
                if bias:
                    row.append(1)
                rows.append(row)
    return rows


def brute_gram(rows):
    d = len(rows[0])
    return [[sum(r[i] * r[j] for r in rows) for j in range(d)] for i in range(d)]


def frac_inverse(M):
    """Exact inverse of a rational matrix by Gauss-Jordan with row pivoting."""
    n = len(M)
    a = [[Fraction(v) for v in row] + [Fraction(int(i == j)) for j in range(n)]
         for i, row in enumerate(M)]
    for c in range(n):
        p = next(r for r in range(c, n) if a[r][c] != 0)
        a[c], a[p] = a[p], a[c]
        pv = a[c][c]
        a[c] = [v / pv for v in a[c]]
        for r in range(n):
            if r != c and a[r][c] != 0:
                f = a[r][c]
                a[r] = [vr - f * vc for vr, vc in zip(a[r], a[c])]
    return [row[n:] for row in a]


def frac_det(M):
    n = len(M)
    a = [[Fraction(v) for v in row] for row in M]
    det = Fraction(1)
    for c in range(n):
        p = next((r for r in range(c, n) if a[r][c] != 0), None)
        if p is None:
            return Fraction(0)
        if p != c:
            a[c], a[p] = a[p], a[c]
            det = -det
        det *= a[c][c]
        for r in range(c + 1, n):
            f = a[r][c] / a[c][c]
            a[r] = [vr - f * vc for vr, vc in zip(a[r], a[c])]
    return det


def frac_matmul(A, B):
    return [[sum(A[i][k] * B[k][j] for k in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def c1_inputs():
    """The fc workload: a[32x64], g[32x16] fp32 N(0,1), dW = g^T a / 32, no bias."""
    seed = synth.config_seed("fc")
    a = synth.normal_f32(synth.layer_rng(seed, 0), (32, 64))
    g = synth.normal_f32(synth.layer_rng(seed, 1), (32, 16))
    dW = (g.astype(np.float64).T @ a.astype(np.float64)) / 32.0
    return a, g, dW


# ---------------------------------------------------------------------------
# pin checks (functions so that the mutation tests can rerun them)
# ---------------------------------------------------------------------------

def check_kronecker_bruteforce(factors=oracle.conv_factors, inv=oracle.damped_inverse,
                               pre=oracle.precondition):
    """eq. (5)-(7): solve with the explicit 1024x1024 Kronecker product."""
    a, g, dW = c1_inputs()
    A, G = factors(a.reshape(32, 1, 1, 64), g.reshape(32, 1, 1, 16), 1, 1, 1, 1, 0, 0, 0)
    s = S_GAMMA
    K = np.kron(G + s * np.eye(16), A + s * np.eye(64))
    ref = np.linalg.solve(K, dW.reshape(-1)).reshape(16, 64)
    Ai, _ = inv(A, s)
    Gi, _ = inv(G, s)
    return relF(pre(Gi, dW, Ai), ref)


def check_single_sample_fisher(factors=oracle.conv_factors):
    """eq. (3) vs eq. (5): for one sample the empirical Fisher of a fully connected
    layer is vec(g a^T) vec(g a^T)^T = (g g^T) (x) (a a^T) exactly."""
    rng = np.random.default_rng(7)
    a = rng.standard_normal(5)
    g = rng.standard_normal(3)
    v = np.outer(g, a).reshape(-1)
    fisher = np.outer(v, v)
    A, G = factors(a.reshape(1, 1, 1, 5), g.reshape(1, 1, 1, 3), 1, 1, 1, 1, 0, 0, 0)
    return np.abs(np.kron(G, A) - fisher).max()


GEOMS = [  # (n, h, w, c, kh, kw, sh, sw, ph, pw, bias)
    (2, 5, 5, 3, 3, 3, 1, 1, 1, 1, 1),
    (2, 6, 5, 2, 3, 3, 2, 2, 1, 1, 1),
    (1, 7, 7, 3, 7, 7, 2, 2, 3, 3, 1),
    (3, 4, 4, 4, 1, 1, 2, 2, 0, 0, 0),
    (2, 3, 3, 5, 1, 1, 1, 1, 0, 0, 1),
]


def check_im2col_integer(factors_gram=None):
    """Integer inputs: the Gram of the patch matrix, computed with exact Python
    integers by explicit loops, must equal the oracle's fp64 Gram bit for bit."""
    worst = 0.0
    rng = np.random.default_rng(11)
    for (n, h, w, c, kh, kw, sh, sw, ph, pw, bias) in GEOMS:
        x = rng.integers(-2, 3, size=(n, h, w, c))
        rows = brute_patches(x.tolist(), kh, kw, sh, sw, ph, pw, bias)
        ref = np.array(brute_gram(rows), dtype=np.float64)
        X = oracle.im2col_nhwc(x, kh, kw, sh, sw, ph, pw, bias)
        got = (factors_gram or oracle.gram)(X)
        if got.shape != ref.shape:
            return np.inf
        worst = max(worst, np.abs(got - ref).max())
    return worst


def check_ema(ema=oracle.ema_update):
    """Fixed point and two-batch closed form of the moving average."""
    S1 = np.array([[2.0, 1.0], [1.0, 3.0]])
    S2 = np.array([[4.0, 0.0], [0.0, 1.0]])
    S = ema(None, S1, 0.0)
    for _ in range(5):
        S = ema(S, S1, 0.95)
    e1 = np.abs(S - S1).max()
    e2 = np.abs(ema(S1, S2, 0.95) - (0.95 * S1 + 0.05 * S2)).max()
    return max(e1, e2)


def check_bn_bruteforce(bn=oracle.bn_diag_fisher):
    """Empirical Fisher of eq. (3) over BN's (gamma, beta) built from explicit
    per-sample gradients; its diagonal, the mean gradient and grad/(F+shift) must
    match."""
    rng = np.random.default_rng(5)
    N, HW, C = 4, 6, 3
    x = rng.standard_normal((N, HW, C))
    g = rng.standard_normal((N, HW, C))
    per_sample = []
    for n in range(N):
        dg = [sum(g[n, p, c] * x[n, p, c] for p in range(HW)) for c in range(C)]
        db = [sum(g[n, p, c] for p in range(HW)) for c in range(C)]
        per_sample.append(np.array(dg + db))
    full = sum(np.outer(v, v) for v in per_sample) / N
    mean = sum(per_sample) / N
    out = bn(x, g, 0.25)
    F = np.concatenate([out["fisher"][0], out["fisher"][1]])
    grd = np.concatenate([out["grad"][0], out["grad"][1]])
    pre = np.concatenate([out["precond"][0], out["precond"][1]])
    return max(np.abs(F - np.diag(full)).max(), np.abs(grd - mean).max(),
               np.abs(pre - mean / (np.diag(full) + 0.25)).max())


def check_pack(pack=oracle.pack_upper, unpack=oracle.unpack_upper):
    """LAPACK's lower column-packed storage of a symmetric matrix is the same
    sequence as the upper triangle row by row."""
    worst = 0.0
    for n in (1, 2, 5, 17):
        rng = np.random.default_rng(n)
        M = rng.standard_normal((n, n))
        M = M + M.T
        ref, info = scipy.linalg.lapack.dtrttp(M, uplo='L')
        assert info == 0
        p = pack(M)
        worst = max(worst, np.abs(p - ref).max(), np.abs(unpack(p, n) - M).max())
    return worst


def check_cholesky_vs_lapack(chol=oracle.cholesky_upper, triinv=oracle.upper_triangular_inverse):
    worst = 0.0
    for n in (1, 2, 3, 17, 64, 65):
        rng = np.random.default_rng(100 + n)
        X = rng.standard_normal((2 * n + 3, n))
        M = X.T @ X / (2 * n + 3) + 0.1 * np.eye(n)
        U, info = chol(M)
        assert info == 0
        Ur = scipy.linalg.cholesky(M, lower=False)
        Uir = scipy.linalg.solve_triangular(Ur, np.eye(n), lower=False)
        worst = max(worst, relF(U, Ur), relF(triinv(U), Uir))
    return worst


# ---------------------------------------------------------------------------
# the pins
# ---------------------------------------------------------------------------

def test_kronecker_bruteforce_fc():
    """Pin P1 (eq. 5-7): the fc workload against the explicit Kronecker solve."""
    assert check_kronecker_bruteforce() < 1e-11


def test_single_sample_fisher_is_kronecker():
    """Pin P3 (eq. 3 vs eq. 5): one sample's Fisher equals G (x) A exactly."""
    assert check_single_sample_fisher() < 1e-12


def test_kronecker_order_pages_vs_north_star():
    """(G (x) A)^-1 vec_row(dW) = vec_row(G^-1 dW A^-1) and (A (x) G)^-1 vec_col(dW)
    = vec_col(same): the two Kronecker orders agree once vec matches."""
    a, g, dW = c1_inputs()
    A, G = oracle.conv_factors(a.reshape(32, 1, 1, 64), g.reshape(32, 1, 1, 16),
                               1, 1, 1, 1, 0, 0, 0)
    s = S_GAMMA
    P = oracle.precondition(oracle.damped_inverse(G, s)[0], dW, oracle.damped_inverse(A, s)[0])
    K2 = np.kron(A + s * np.eye(64), G + s * np.eye(16))
    col = np.linalg.solve(K2, dW.reshape(-1, order="F"))
    assert relF(col.reshape(16, 64, order="F"), P) < 1e-11


def test_sherman_morrison():
    """Pin P2: (x x^T + s I)^-1 = (I - x x^T / (s + x^T x)) / s."""
    rng = np.random.default_rng(3)
    for n, s in [(1, 0.5), (7, 1e-3), (65, S_GAMMA)]:
        x = rng.standard_normal(n)
        ref = (np.eye(n) - np.outer(x, x) / (s + x @ x)) / s
        got, info = oracle.damped_inverse(np.outer(x, x), s)
        assert info == 0
        assert relF(got, ref) < 1e-12


def test_exact_rational_chain():
    """Exact rational brute force of the whole fc chain: integer a, g; shift 1/4
    (exact in binary); factors, inverses and G^-1 dW A^-1 in Fractions."""
    rng = np.random.default_rng(21)
    R, da, dg = 3, 3, 2
    a = rng.integers(-3, 4, size=(R, da))
    g = rng.integers(-3, 4, size=(R, dg))
    dW = rng.integers(-5, 6, size=(dg, da))
    s = Fraction(1, 4)
    A = [[Fraction(sum(int(a[r, i]) * int(a[r, j]) for r in range(R)), R) + (s if i == j else 0)
          for j in range(da)] for i in range(da)]
    G = [[Fraction(sum(int(g[r, i]) * int(g[r, j]) for r in range(R)), R) + (s if i == j else 0)
          for j in range(dg)] for i in range(dg)]
    Ai, Gi = frac_inverse(A), frac_inverse(G)
    P = frac_matmul(frac_matmul(Gi, [[Fraction(int(v)) for v in row] for row in dW]), Ai)
    oA, oG = oracle.conv_factors(a.reshape(R, 1, 1, da), g.reshape(R, 1, 1, dg),
                                 1, 1, 1, 1, 0, 0, 0)
    oAi, _ = oracle.damped_inverse(oA, 0.25)
    oGi, _ = oracle.damped_inverse(oG, 0.25)
    oP = oracle.precondition(oGi, dW, oAi)
    assert relF(oAi, np.array(Ai, dtype=float)) < 1e-14
    assert relF(oGi, np.array(Gi, dtype=float)) < 1e-14
    assert relF(oP, np.array(P, dtype=float)) < 1e-13


def test_im2col_integer_bruteforce():
    """Pins P4/P5: exact integer Gram of explicit patch loops (stride, padding,
    C_in = 3 with a 7x7 kernel, bias on and off)."""
    assert check_im2col_integer() == 0.0


def test_im2col_impulse():
    """Pin P5: a single non-zero pixel v at (y, z, ci) reaches exactly the (tap,
    output) pairs that cover it; A's non-zero pattern is predicted by hand."""
    x = np.zeros((1, 4, 4, 2))
    x[0, 1, 2, 1] = 3.0
    X = oracle.im2col_nhwc(x, 3, 3, 1, 1, 1, 1, 1)
    A = oracle.gram(X)
    # taps (i, j) with 0 <= 1 - i + 1 < 4 and 0 <= 2 - j + 1 < 4: all 9 taps; each
    # touches one output position, so column (i*3+j)*2+1 holds a single 3.
    cols = [(i * 3 + j) * 2 + 1 for i in range(3) for j in range(3)]
    nz = {(p, q) for p, q in zip(*np.nonzero(A))}
    expect = {(p, q) for p in cols for q in cols if p == q} | {(p, 18) for p in cols} \
        | {(18, p) for p in cols} | {(18, 18)}
    assert nz == expect
    assert all(A[p, p] == 9.0 for p in cols) and A[18, 18] == 16.0
    assert all(A[p, 18] == 3.0 for p in cols)


def test_im2col_vs_unfold():
    """Pin P6: an independent im2col (torch.nn.functional.unfold, channel-major)
    permuted to the (kh, kw, c_in) column order."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    for (n, h, w, c, kh, kw, sh, sw, ph, pw, _) in GEOMS:
        x = rng.standard_normal((n, h, w, c))
        X = oracle.im2col_nhwc(x, kh, kw, sh, sw, ph, pw, 0)
        t = torch.from_numpy(x).permute(0, 3, 1, 2)                   # NCHW
        U = torch.nn.functional.unfold(t, (kh, kw), padding=(ph, pw), stride=(sh, sw))
        L = U.shape[-1]                                               # [N, C*kh*kw, L]
        U = U.reshape(n, c, kh, kw, L).permute(0, 4, 2, 3, 1).reshape(n * L, kh * kw * c)
        assert np.abs(U.numpy() - X).max() == 0.0


def test_packed_storage_vs_lapack():
    """Pin P7: packed order equals LAPACK dtrttp(lower); round trip exact."""
    assert check_pack() == 0.0
    n = 9
    idx = [(i, j) for i in range(n) for j in range(i, n)]
    assert [oracle.packed_offset(i, j, n) for i, j in idx] == list(range(len(idx)))


def test_cholesky_and_triangular_inverse_vs_lapack():
    """Pin P8 (library special case): potrf and trtri of LAPACK via SciPy."""
    assert check_cholesky_vs_lapack() < 1e-12


@pytest.mark.parametrize("n", [1, 2, 63, 65, 129, 300])
def test_inverse_invariants(n):
    """Pin P8: M M^-1 = I, exact symmetry, positive definiteness and agreement with
    numpy.linalg.inv, on ReLU factors like the network's (rank-deficient at small R)."""
    rng = np.random.default_rng(n)
    R = max(2, n // 3)
    X = np.maximum(rng.standard_normal((R, n)), 0)
    F = X.T @ X / R
    Minv, info = oracle.damped_inverse(F, S_GAMMA)
    assert info == 0
    M = F + S_GAMMA * np.eye(n)
    cond = np.linalg.cond(M)
    assert np.abs(Minv - Minv.T).max() == 0.0
    assert np.linalg.norm(M @ Minv - np.eye(n)) < 1e-13 * cond * n
    assert np.linalg.eigvalsh(Minv).min() > 0
    assert relF(Minv, np.linalg.inv(M)) < 1e-14 * cond * n


def test_cholesky_info_sylvester():
    """Breakdown index = first leading principal minor that is not positive
    (Sylvester's criterion), computed with exact rational determinants."""
    rng = np.random.default_rng(9)
    seen = set()
    for _ in range(200):
        n = int(rng.integers(1, 6))
        B = rng.integers(-3, 4, size=(n, n))
        M = (B + B.T) // 2 + np.diag(rng.integers(0, 4, size=n))
        minors = [frac_det(M[:k, :k].tolist()) for k in range(1, n + 1)]
        expect = next((k for k, m in enumerate(minors, 1) if m <= 0), 0)
        _, info = oracle.cholesky_upper(M.astype(float))
        # a minor that is exactly 0 can round to a tiny positive pivot; skip those
        if expect and minors[expect - 1] == 0:
            continue
        assert info == expect, (M, minors)
        seen.add(expect)
    assert 0 in seen and len(seen) >= 3
    A = np.eye(3)
    A[1, 2] = np.nan
    assert oracle.cholesky_upper(A)[1] == 3


def test_precondition_special_cases():
    """Pin P9: identity and diagonal factors."""
    rng = np.random.default_rng(4)
    dW = rng.standard_normal((5, 7))
    s = S_GAMMA
    Ai, _ = oracle.damped_inverse(np.eye(7), s)
    Gi, _ = oracle.damped_inverse(np.eye(5), s)
    assert relF(oracle.precondition(Gi, dW, Ai), dW / (1 + s) ** 2) < 1e-14
    a = rng.uniform(0.5, 2, 7)
    g = rng.uniform(0.5, 2, 5)
    Ai, _ = oracle.damped_inverse(np.diag(a), s)
    Gi, _ = oracle.damped_inverse(np.diag(g), s)
    ref = dW / np.outer(g + s, a + s)
    assert relF(oracle.precondition(Gi, dW, Ai), ref) < 1e-14


def test_bn_bruteforce_fisher():
    """Pin P10: diagonal of the eq. (3) Fisher over per-sample (gamma, beta)
    gradients, and a constant-input closed form."""
    assert check_bn_bruteforce() < 1e-12
    N, HW, C, c = 3, 5, 2, 0.5
    out = oracle.bn_diag_fisher(np.ones((N, HW, C)), np.full((N, HW, C), c), 1.0)
    assert np.allclose(out["fisher"], (HW * c) ** 2, rtol=0, atol=1e-15)
    assert np.allclose(out["precond"], HW * c / ((HW * c) ** 2 + 1.0), rtol=0, atol=1e-15)


def check_update_rule(update=None):
    """Pin P12: eq. (8) applied to the eq. (7) gradient of a tiny layer equals
    w - lr * (G (x) A)^-1 vec(dW), the Kronecker system solved densely."""
    update = update or oracle.sgd_update
    rng = np.random.default_rng(12)
    dg, da, lr = 3, 4, 0.37
    G = rng.standard_normal((dg, dg)); G = G @ G.T + np.eye(dg)
    A = rng.standard_normal((da, da)); A = A @ A.T + np.eye(da)
    dW = rng.standard_normal((dg, da))
    w = rng.standard_normal((dg, da))
    P = oracle.precondition(np.linalg.inv(G), dW, np.linalg.inv(A))
    ref = w - lr * np.linalg.solve(np.kron(G, A), dW.reshape(-1)).reshape(dg, da)
    return relF(update(w, P, lr), ref)


def test_update_rule():
    assert check_update_rule() < 1e-12
    w = np.arange(6.0).reshape(2, 3)
    assert np.array_equal(oracle.sgd_update(w, np.ones_like(w), 0.0), w)
    assert np.array_equal(oracle.sgd_update(np.zeros(3), np.array([1.0, -2.0, 4.0]), 0.5),
                          np.array([-0.5, 1.0, -2.0]))


def test_bn_ema():
    rng = np.random.default_rng(6)
    x, g = rng.standard_normal((2, 2, 3, 4))
    F0 = rng.uniform(1, 2, (2, 4))
    out = oracle.bn_diag_fisher(x, g, 0.1, ema_decay=0.95, fisher_prev=F0)
    fresh = oracle.bn_diag_fisher(x, g, 0.1)
    assert np.allclose(out["fisher"], 0.95 * F0 + 0.05 * fresh["fisher"], rtol=1e-15)
    assert np.allclose(out["precond"], fresh["grad"] / (out["fisher"] + 0.1), rtol=1e-15)


def test_ema_closed_form():
    """Pin P11: fixed point of identical batches; two-batch closed form."""
    assert check_ema() < 1e-15


def test_fc_golden_regression():
    """Stored oracle outputs for the fc workload (written by
    tests/golden/make_fc_golden.py, which calls only the oracle)."""
    with open(os.path.join(GOLDEN, "fc_oracle.json")) as f:
        gold = json.load(f)
    a, g, dW = c1_inputs()
    A, G = oracle.conv_factors(a.reshape(32, 1, 1, 64), g.reshape(32, 1, 1, 16),
                               1, 1, 1, 1, 0, 0, 0)
    Ai, _ = oracle.damped_inverse(A, S_GAMMA)
    Gi, _ = oracle.damped_inverse(G, S_GAMMA)
    P = oracle.precondition(Gi, dW, Ai)
    for name, v in (("A", A), ("G", G), ("A_inv", Ai), ("G_inv", Gi), ("P", P)):
        ref = gold[name]
        assert abs(np.linalg.norm(v) - ref["fro"]) <= 1e-12 * ref["fro"]
        for (i, j), val in zip(ref["idx"], ref["val"]):
            assert abs(v[i, j] - val) <= 1e-12 * max(1.0, abs(val))


def test_resnet50_shapes_golden():
    """The ResNet-50 layer geometry (He et al. 2016, the network of Section 1 and
    Table 1) against a hand-typed fixture of its factor sizes, rows and BN classes."""
    from collections import Counter
    with open(os.path.join(GOLDEN, "resnet50_batch32.json")) as f:
        gold = json.load(f)
    L = synth.conv_layers(32)
    assert len(L) == gold["n_kfac_layers"]
    dims = Counter([l.d_a for l in L] + [l.d_g for l in L])
    assert {str(k): v for k, v in dims.items()} == gold["factor_dims"]
    rows = Counter(l.rows for l in L)
    assert {str(k): v for k, v in rows.items()} == gold["rows_by_count"]
    bn = Counter((b.c, b.hw) for b in synth.bn_layers(32))
    assert sorted([c, hw, k] for (c, hw), k in bn.items()) == sorted(gold["bn_classes"])
    assert sum(b.c for b in synth.bn_layers(32)) == gold["bn_channels"]


# ---------------------------------------------------------------------------
# mutation checks: a planted mistake in a copy of an oracle step must fail a pin
# ---------------------------------------------------------------------------

def _mut_factors_transposed(act, gout, *geo):
    A, G = oracle.conv_factors(act, gout, *geo)
    return G, A                                     # swapped factors


def _mut_factors_centred(act, gout, *geo):
    X = oracle.im2col_nhwc(act, *geo)
    X = X - X.mean(axis=0)
    Gm = np.asarray(gout, dtype=float).reshape(-1, np.shape(gout)[-1])
    return X.T @ X / X.shape[0], Gm.T @ Gm / Gm.shape[0]


def _mut_pre_transposed(Gi, dW, Ai):
    return Gi @ dW @ Ai.T @ np.diag(np.linspace(1, 1.01, Ai.shape[0]))


def _mut_inv_no_damping(F, s):
    return oracle.damped_inverse(F, 0.0 if s < 0.1 else s)


def _mut_gram_scaled(X):
    return X.T @ X / X.shape[0]


def _mut_bn_sum_not_mean(x, g, shift, **kw):
    out = oracle.bn_diag_fisher(x, g, shift, **kw)
    out["fisher"] = out["fisher"] * np.shape(x)[0]
    return out


def _mut_ema_swapped(old, batch, decay):
    if decay == 0.0:
        return np.asarray(batch, dtype=float)
    return (1 - decay) * np.asarray(old) + decay * np.asarray(batch)


def _mut_pack_lower(M):
    M = np.asarray(M)
    return np.concatenate([M[i, :i + 1] for i in range(M.shape[0])])   # lower, row by row


def _mut_chol_sign(M):
    U, info = oracle.cholesky_upper(M)
    U[0, 1:] = -U[0, 1:]
    return U, info


@pytest.mark.parametrize("check,kwargs,limit", [
    (check_kronecker_bruteforce, {"factors": _mut_factors_transposed}, 1e-11),
    (check_kronecker_bruteforce, {"pre": _mut_pre_transposed}, 1e-11),
    (check_kronecker_bruteforce, {"inv": _mut_inv_no_damping}, 1e-11),
    (check_single_sample_fisher, {"factors": _mut_factors_centred}, 1e-12),
    (check_im2col_integer, {"factors_gram": _mut_gram_scaled}, 1e-9),
    (check_bn_bruteforce, {"bn": _mut_bn_sum_not_mean}, 1e-12),
    (check_ema, {"ema": _mut_ema_swapped}, 1e-15),
    (check_pack, {"pack": _mut_pack_lower}, 1e-15),
    (check_cholesky_vs_lapack, {"chol": _mut_chol_sign}, 1e-12),
    (check_update_rule, {"update": lambda w, g, lr: np.asarray(w) + lr * np.asarray(g)}, 1e-12),
])
def test_planted_mistake_is_caught(check, kwargs, limit):
    try:
        err = check(**kwargs)
    except (ValueError, IndexError, np.linalg.LinAlgError):
        return                                   # the pin refuses the mutant outright
    assert not (err < limit)


def test_planted_im2col_order_is_caught():
    """Channel-major column order (c_in, kh, kw) instead of (kh, kw, c_in)."""
    real = oracle.im2col_nhwc

    def wrong(x, kh, kw, sh, sw, ph, pw, bias):
        X = real(x, kh, kw, sh, sw, ph, pw, 0)
        c = np.shape(x)[-1]
        X = X.reshape(X.shape[0], kh * kw, c).transpose(0, 2, 1).reshape(X.shape[0], -1)
        if bias:
            X = np.concatenate([X, np.ones((X.shape[0], 1))], axis=1)
        return X

    oracle.im2col_nhwc = wrong
    try:
        assert check_im2col_integer() > 0
    finally:
        oracle.im2col_nhwc = real
