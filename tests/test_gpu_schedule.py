"""Stale-curvature schedule on the GPU against the oracle running the same schedule.

Factors (and the BN Fisher) are refreshed every 10 steps with an exponential moving
average of decay 0.95 (the first refresh overwrites); the damped inverses are
recomputed at refreshes only; every step preconditions fresh fp16 gradients
N(0, 1e-2) with the stored inverses. Two activation/gradient sets alternate across
refreshes. Layers: three ResNet-50 shapes at batch 128 (a 3x3 stage-4 convolution,
a strided 1x1 and the classifier) and two BN layers.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import host, relF, say, to_dev

pytestmark = pytest.mark.gpu

REFRESH = 10
DECAY = 0.95
STEPS = 21


def _layers():
    L = {l.name: l for l in synth.conv_layers(128)}
    B = {b.name: b for b in synth.bn_layers(128)}
    return [L["s4b1.c2"], L["s5b0.c1"], L["fc"]], [B["bn_s4b1.c2"], B["bn_s5b0.c3"]]


@pytest.mark.timeout(600)
def test_stale_schedule_matches_oracle(kfac_gpu):
    layers, bns = _layers()
    seed = synth.config_seed("stale")
    sets = []
    for s in range(2):  # two input sets, alternated across refreshes
        acts, gouts = [], []
        for i, l in enumerate(layers):
            rng = synth.layer_rng(seed, 100 * s + i)
            acts.append(synth.relu_normal_f16(rng, l.act_shape))
            gouts.append(synth.normal_f16(rng, l.gout_shape, 0.1))
        xh, bg = [], []
        for i, b in enumerate(bns):
            rng = synth.layer_rng(seed, 100 * s + 50 + i)
            xh.append(synth.normal_f16(rng, b.shape))
            bg.append(synth.normal_f16(rng, b.shape, 0.1))
        sets.append((acts, gouts, xh, bg))
    grads = [[synth.normal_f16(synth.layer_rng(seed, 1000 + 10 * t + i), (l.d_g, l.d_a), 0.1)
              for i, l in enumerate(layers)] for t in range(STEPS)]
    dev_sets = [tuple([to_dev(a) for a in part] for part in st) for st in sets]
    dev_grads = [[to_dev(g) for g in gs] for gs in grads]

    st = kfac_gpu.KfacStep(layers, bns, "cuda")
    # oracle state
    A = [None] * len(layers)
    G = [None] * len(layers)
    Ai = [None] * len(layers)
    Gi = [None] * len(layers)
    F = [None] * len(bns)
    nref = 0
    for t in range(STEPS):
        refresh = t % REFRESH == 0
        s = nref % 2 if refresh else (nref - 1) % 2
        acts, gouts, xh, bg = sets[s]
        dacts, dgouts, dxh, dbg = dev_sets[s]
        decay = 0.0 if (refresh and nref == 0) else DECAY
        say(f"step {t} refresh={refresh} set={s}")
        st.step(dacts, dgouts, dev_grads[t], dxh, dbg, ema_decay=decay, refresh=refresh)
        if refresh:
            for i, l in enumerate(layers):
                a, g = oracle.conv_factors(acts[i], gouts[i], l.kh, l.kw, l.sh, l.sw, l.ph, l.pw,
                                           l.bias)
                A[i] = oracle.ema_update(A[i], a, decay)
                G[i] = oracle.ema_update(G[i], g, decay)
                Ai[i], _ = oracle.damped_inverse(A[i], st.shift)
                Gi[i], _ = oracle.damped_inverse(G[i], st.shift)
            nref += 1
        bn_out = []
        for i, b in enumerate(bns):
            out = oracle.bn_diag_fisher(xh[i], bg[i], st.bn_shift,
                                        ema_decay=(decay if refresh else 1.0), fisher_prev=F[i])
            F[i] = out["fisher"]
            bn_out.append(out)
        if t % 5 == 0 or t == STEPS - 1:
            for i, l in enumerate(layers):
                P = oracle.precondition(Gi[i], grads[t][i], Ai[i])
                e = relF(host(st.out[i]), P)
                ea = relF(host(st.A_packed[i]), oracle.pack_upper(A[i]))
                say(f"  t={t} {l.name}: P relF {e:.2e}  A relF {ea:.2e}")
                assert e <= 2e-2 and ea <= 1e-2, (t, l.name, e, ea)
            for i, b in enumerate(bns):
                assert relF(host(st.fisher[i]), bn_out[i]["fisher"]) <= 1e-4, (t, b.name)
                assert relF(host(st.bn_pre[i]), bn_out[i]["precond"]) <= 1e-4, (t, b.name)
    assert int(host(st.info).sum()) == 0
