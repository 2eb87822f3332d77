"""One K-FAC step over a fixed set of layers: device buffers plus the sequence of
library calls (factors -> unpack -> damped inverses -> preconditioning, and the
BatchNorm diagonal). Python only allocates and sequences; every number is computed
by libkfac's HIP kernels.

Step order follows Osawa et al. (CVPR 2019): stage 1-2 of their Figure 1 (factors
from the forward activations and backward gradients), eq. (6) (inverses of the
damped factors), eq. (7) (preconditioned gradients) and, when parameters are
given, eq. (8) (the update with learning rate lr); BatchNorm uses the diagonal
Fisher (Section 1, contributions)."""
import math

import torch

from . import _lib as K


class KfacStep:
    """Buffers for `layers` (objects with the kfac_layer fields) and `bn_layers`
    (objects with n, hw, c). Tikhonov damping gamma puts sqrt(gamma) on each
    Kronecker factor (float32-rounded) and gamma on the BN diagonal. precond_accum
    "f64" sums the preconditioning products in fp64 (kfac_precondition_ex).
    refine_inverse applies one fp64-residual refinement step to every inverse
    (kfac_invert_refine), which keeps a full symmetric copy of each factor."""

    def __init__(self, layers, bn_layers=(), device="cuda", damping=1e-3, bn_shift=None,
                 in_dtype=torch.float16, precond_accum="f32", refine_inverse=False):
        self.layers = list(layers)
        self.bn_layers = list(bn_layers)
        self.device = torch.device(device)
        if precond_accum not in ("f32", "f64"):
            raise ValueError("precond_accum must be 'f32' or 'f64'")
        self.accum = K.KFAC_F64 if precond_accum == "f64" else K.KFAC_F32
        self.shift = float(torch.tensor(math.sqrt(damping), dtype=torch.float32))
        self.bn_shift = float(damping if bn_shift is None else bn_shift)
        self.d_a = [l.c_in * l.kh * l.kw + (1 if l.bias else 0) for l in self.layers]
        self.d_g = [l.c_out for l in self.layers]
        dev = self.device
        f32 = torch.float32
        self.A_packed = [torch.empty(d * (d + 1) // 2, dtype=f32, device=dev) for d in self.d_a]
        self.G_packed = [torch.empty(d * (d + 1) // 2, dtype=f32, device=dev) for d in self.d_g]
        # factor k of the inverse batch: A of every layer, then G of every layer
        self.n_all = self.d_a + self.d_g
        self.full = [torch.empty(d, d, dtype=f32, device=dev) for d in self.n_all]
        self.packed_all = self.A_packed + self.G_packed
        self.info = torch.zeros(len(self.n_all), dtype=torch.int32, device=dev)
        self.out = [torch.empty(g, a, dtype=f32, device=dev) for g, a in zip(self.d_g, self.d_a)]
        self.refine = bool(refine_inverse)
        self.factor_full = [torch.empty(d, d, dtype=f32, device=dev) for d in self.n_all] if self.refine else []
        self.fisher = [torch.zeros(2, b.c, dtype=f32, device=dev) for b in self.bn_layers]
        self.bn_pre = [torch.empty(2, b.c, dtype=f32, device=dev) for b in self.bn_layers]
        code = K.KFAC_F16 if in_dtype == torch.float16 else K.KFAC_F32
        sizes = [K.kfac_factors_workspace(self.layers, code),
                 K.kfac_pack_sym_workspace(self.n_all),
                 K.kfac_invert_workspace(self.n_all),
                 K.kfac_precondition_workspace(self.d_g, self.d_a)]
        if self.refine:
            sizes.append(K.kfac_invert_refine_workspace(self.n_all))
        if self.bn_layers:
            sizes.append(K.kfac_bn_diag_workspace(self.bn_layers))
        # one workspace serves every call: they run one after another on one stream
        self.workspace = torch.empty(max(sizes) + 256, dtype=torch.uint8, device=dev)

    @property
    def A_inv(self):
        return self.full[:len(self.layers)]

    @property
    def G_inv(self):
        return self.full[len(self.layers):]

    def factors(self, act, gout, ema_decay=0.0, stream=None):
        K.kfac_factors(self.layers, act, gout, self.A_packed, self.G_packed, ema_decay,
                       self.workspace, stream)

    def invert(self, stream=None):
        # kfac_invert reads only the upper triangle: unpack that half
        K.kfac_pack_sym(self.n_all, self.full, self.packed_all, 2, self.workspace, stream)
        K.kfac_invert(self.n_all, self.full, self.full, [self.shift] * len(self.n_all), self.info,
                      None, self.workspace, stream)
        if self.refine:
            K.kfac_pack_sym(self.n_all, self.factor_full, self.packed_all, 1, self.workspace, stream)
            K.kfac_invert_refine(self.n_all, self.factor_full, [self.shift] * len(self.n_all), self.full,
                                 self.workspace, stream)

    def precondition(self, grads, weights=None, lr=0.0, stream=None):
        """self.out <- preconditioned gradients; with weights (fp32 [d_g, d_a] per layer)
        also weights -= lr * self.out, in the same kernel."""
        if self.accum == K.KFAC_F64:
            K.kfac_precondition_ex(self.d_g, self.d_a, self.G_inv, self.A_inv, grads, self.out, weights, lr,
                                   self.accum, self.workspace, stream)
        elif weights is None:
            K.kfac_precondition(self.d_g, self.d_a, self.G_inv, self.A_inv, grads, self.out,
                                self.workspace, stream)
        else:
            K.kfac_precondition_update(self.d_g, self.d_a, self.G_inv, self.A_inv, grads, self.out,
                                       weights, lr, self.workspace, stream)

    def bn(self, xhat, bn_gout, ema_decay=0.0, bn_params=None, lr=0.0, stream=None):
        """BN Fisher and preconditioned gradients; with bn_params (fp32 [2, c]: gamma,
        beta) also bn_params -= lr * self.bn_pre."""
        if not self.bn_layers:
            return
        if bn_params is None:
            K.kfac_bn_diag(self.bn_layers, xhat, bn_gout, self.fisher, self.bn_pre, ema_decay,
                           self.bn_shift, self.workspace, stream)
        else:
            K.kfac_bn_update(self.bn_layers, xhat, bn_gout, self.fisher, self.bn_pre, bn_params, lr,
                             ema_decay, self.bn_shift, self.workspace, stream)

    def step(self, act, gout, grads, xhat=(), bn_gout=(), ema_decay=0.0, refresh=True,
             weights=None, bn_params=None, lr=0.0, stream=None):
        """One step. refresh=False is a stale-curvature step: factors and inverses are
        kept, the gradients are preconditioned with them, and BN divides its fresh
        gradient by the stored Fisher (decay 1 keeps it). Given weights and/or
        bn_params, those are updated in place with learning rate lr."""
        if refresh:
            self.factors(act, gout, ema_decay, stream)
            self.invert(stream)
        self.precondition(grads, weights, lr, stream)
        self.bn(xhat, bn_gout, ema_decay if refresh else 1.0, bn_params, lr, stream)
