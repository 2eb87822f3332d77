"""The BatchNorm entry point that allocates nothing (kfac_bn_diag_noalloc, for callers
that cannot allocate device memory) against the workspace entry points it stands in
for: bit-identical Fisher, preconditioned gradients and updated parameters, on two
calls in a row, the first large enough to run in several passes over the static
scratch, the second smaller and blending into the first call's Fisher."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(bns, seed):
    rng = synth.layer_rng(seed, 0)
    return ([to_dev(synth.normal_f16(rng, b.shape)) for b in bns],
            [to_dev(synth.normal_f16(rng, b.shape)) for b in bns])


def _fresh(bns, fill):
    return [torch.full((2, b.c), fill, device="cuda") for b in bns]


def test_bn_noalloc_matches_workspace_calls(kfac_gpu):
    big = synth.bn_layers(32)                       # needs more than the 16 MiB scratch
    small = [synth.BNLayer("a", 3, 49, 64), synth.BNLayer("b", 2, 25, 40), synth.BNLayer("c", 4, 9, 24)]
    assert kfac_gpu.kfac_bn_diag_workspace(big) > kfac_gpu._lib.KFAC_BN_NOALLOC_SCRATCH_BYTES
    say("noalloc call 1: ResNet-50 BN layers at batch 32 (several passes)")
    x, g = _inputs(big, 2001)
    f_ref, p_ref = _fresh(big, 0.0), _fresh(big, 0.0)
    f_new, p_new = _fresh(big, 5.0), _fresh(big, 5.0)
    kfac_gpu.kfac_bn_diag(big, x, g, f_ref, p_ref, 0.0, 1e-3)
    kfac_gpu.kfac_bn_diag_noalloc(big, x, g, f_new, p_new, None, 0.0, 0.0, 1e-3)
    torch.cuda.synchronize()
    for a, b in zip(f_ref + p_ref, f_new + p_new):
        assert torch.equal(a, b)
    say("noalloc call 2: three small layers, EMA 0.95 and the update")
    x, g = _inputs(small, 2002)
    rng = np.random.default_rng(7)
    f0 = [to_dev(np.abs(rng.standard_normal((2, b.c))).astype(np.float32)) for b in small]
    w0 = [to_dev(rng.standard_normal((2, b.c)).astype(np.float32)) for b in small]
    f_ref, f_new = [t.clone() for t in f0], [t.clone() for t in f0]
    w_ref, w_new = [t.clone() for t in w0], [t.clone() for t in w0]
    p_ref, p_new = _fresh(small, 0.0), _fresh(small, 9.0)
    kfac_gpu.kfac_bn_update(small, x, g, f_ref, p_ref, w_ref, 0.05, 0.95, 1e-3)
    kfac_gpu.kfac_bn_diag_noalloc(small, x, g, f_new, p_new, w_new, 0.05, 0.95, 1e-3)
    torch.cuda.synchronize()
    for a, b in zip(f_ref + p_ref + w_ref, f_new + p_new + w_new):
        assert torch.equal(a, b)
    assert not torch.equal(w_new[0], w0[0])


def test_bn_noalloc_rejects_a_layer_larger_than_its_scratch(kfac_gpu):
    """A single layer whose partial sums exceed the static scratch is refused before
    any work is enqueued (kfac_bn_diag with a workspace has no such limit)."""
    huge = [synth.BNLayer("huge", 2048, 112 * 112, 64)]
    p = torch.zeros(1, device="cuda")
    with pytest.raises(kfac_gpu.KfacError, match="static buffer"):
        kfac_gpu.kfac_bn_diag_noalloc(huge, [p], [p], [p], [p])
