"""Host-side checks of the network capture (no GPU): the weight layout matches the
patch columns of the K-FAC activation factor, and the hooks record every layer with
the geometry the library expects."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

cap_mod = pytest.importorskip("fac_second_order_amd.capture")


@pytest.mark.parametrize("k,s,p,bias", [(3, 2, 1, False), (1, 1, 0, True), (7, 2, 3, False)])
def test_weight_matrix_matches_patch_columns(k, s, p, bias):
    """conv2d(x, W) equals X W_mat^T with X the oracle's im2col patches: the matrix
    layout the capture gives the library is the one its factor A is built on."""
    torch.manual_seed(0)
    conv = torch.nn.Conv2d(5, 4, k, s, p, bias=bias).double()
    x = torch.randn(2, 5, 9, 9, dtype=torch.float64)
    y = conv(x).permute(0, 2, 3, 1).reshape(-1, 4).detach().numpy()
    X = oracle.im2col_nhwc(x.permute(0, 2, 3, 1).numpy(), k, k, s, s, p, p, bias)
    W = cap_mod.KfacCapture._to_matrix(conv).double().numpy()
    assert np.allclose(X @ W.T, y, rtol=1e-12, atol=1e-12)


def test_matrix_round_trip():
    torch.manual_seed(1)
    for m in (torch.nn.Conv2d(3, 6, 3, 1, 1, bias=False), torch.nn.Linear(7, 5)):
        before = [t.detach().clone() for t in m.parameters()]
        mat = cap_mod.KfacCapture._to_matrix(m)
        for t in m.parameters():
            t.data.zero_()
        cap_mod.KfacCapture._from_matrix(m, mat)
        for b, t in zip(before, m.parameters()):
            assert torch.equal(b, t.data)


def test_hooks_record_every_layer():
    torch.manual_seed(2)
    model = cap_mod.ResNet50(classes=10)
    cap = cap_mod.KfacCapture(model)
    x = torch.randn(2, 3, 32, 32)
    loss = F.cross_entropy(model(x), torch.tensor([1, 7]))
    loss.backward()
    layers, bns = cap._geometry()
    assert len(layers) == 54 and len(bns) == 53
    for L, a, g in zip(layers, cap.act, cap.gout):
        assert (L.h + 2 * L.ph - L.kh) // L.sh + 1 == L.h_out
        assert a.dtype == torch.float16 and a.is_contiguous() and a.shape == (L.n, L.h, L.w, L.c_in) or \
            a.shape == (L.n, L.c_in)
        assert g.dtype == torch.float16 and g.is_contiguous()
    assert layers[0].c_in == 3 and layers[0].kh == 7 and layers[-1].c_out == 10 and layers[-1].bias == 1
    assert sum(L.kh == 3 for L in layers) == 16 and sum(L.sh == 2 for L in layers) == 7
    for B, xh, gb in zip(bns, cap.xhat, cap.bgout):
        assert xh.shape == (B.n, B.hw, B.c) == gb.shape and xh.is_contiguous() and gb.is_contiguous()
    # the classifier's captured output gradient is n times the batch-mean gradient
    logits = model(x)
    p = torch.softmax(logits.detach(), 1)
    p[[0, 1], [1, 7]] -= 1
    assert torch.allclose(cap.gout[-1].float(), p.half().float(), atol=2e-3)
    cap.remove()
