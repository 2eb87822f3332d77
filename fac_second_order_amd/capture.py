"""Stage 1-2 capture from a network's own forward and backward passes.

Osawa et al. (CVPR 2019), Figure 1 and Section 3: K-FAC takes each layer's input
activations in the forward pass and the gradients at its outputs in the backward
pass, forms the Kronecker factors from them (eq. 5), and updates the parameters with
the preconditioned gradients (eq. 7-8); BatchNorm uses the diagonal Fisher. This
module wires a PyTorch model to the library: hooks hand each convolution's and the
classifier's input and output gradient, and each BatchNorm's normalised input and
output gradient, to KfacStep in the layouts of include/kfac.h. PyTorch runs the
network (forward, backward, loss); every K-FAC number is computed by libkfac.

Layout conventions (the library's):
  * activations and output gradients NHWC fp16; a convolution weight [c_out, c_in,
    kh, kw] is the K-FAC matrix [c_out, (i*kw + j)*c_in + ci] (plus a last bias
    column for the classifier);
  * the loss is a batch mean, so the gradient a hook sees is 1/n of the per-sample
    gradient; it is multiplied by n on capture (the factor G is a per-sample second
    moment, eq. 5, and the BatchNorm Fisher is over per-sample gradients).
"""
from dataclasses import dataclass

import torch
import torch.nn as nn

from .step import KfacStep


# ---------------------------------------------------------------------------
# ResNet-50 (He et al., 2016), v1 layout: the stride of a downsampling bottleneck
# sits on its first 1x1 convolution and on the projection.
# ---------------------------------------------------------------------------

class Bottleneck(nn.Module):
    def __init__(self, c_in, width, c_out, stride):
        super().__init__()
        self.c1 = nn.Conv2d(c_in, width, 1, stride, 0, bias=False)
        self.b1 = nn.BatchNorm2d(width)
        self.c2 = nn.Conv2d(width, width, 3, 1, 1, bias=False)
        self.b2 = nn.BatchNorm2d(width)
        self.c3 = nn.Conv2d(width, c_out, 1, 1, 0, bias=False)
        self.b3 = nn.BatchNorm2d(c_out)
        self.proj = None
        if stride != 1 or c_in != c_out:
            self.proj = nn.Conv2d(c_in, c_out, 1, stride, 0, bias=False)
            self.bp = nn.BatchNorm2d(c_out)
        self.act = nn.ReLU()

    def forward(self, x):
        y = self.act(self.b1(self.c1(x)))
        y = self.act(self.b2(self.c2(y)))
        y = self.b3(self.c3(y))
        s = self.bp(self.proj(x)) if self.proj is not None else x
        return self.act(y + s)

    def kfac_modules(self):
        """(conv, its BatchNorm) in the order the layers are numbered."""
        out = [(self.c1, self.b1), (self.c2, self.b2), (self.c3, self.b3)]
        if self.proj is not None:
            out.append((self.proj, self.bp))
        return out


class ResNet50(nn.Module):
    def __init__(self, classes=1000):
        super().__init__()
        self.conv1 = nn.Conv2d(3, 64, 7, 2, 3, bias=False)
        self.bn1 = nn.BatchNorm2d(64)
        self.act = nn.ReLU()
        self.pool = nn.MaxPool2d(3, 2, 1)
        blocks = []
        c = 64
        for n_blocks, width, c_out, stride in [(3, 64, 256, 1), (4, 128, 512, 2), (6, 256, 1024, 2),
                                               (3, 512, 2048, 2)]:
            for b in range(n_blocks):
                blocks.append(Bottleneck(c, width, c_out, stride if b == 0 else 1))
                c = c_out
        self.blocks = nn.Sequential(*blocks)
        self.fc = nn.Linear(2048, classes)

    def forward(self, x):
        x = self.pool(self.act(self.bn1(self.conv1(x))))
        x = self.blocks(x)
        return self.fc(torch.flatten(x.mean((2, 3)), 1))

    def kfac_modules(self):
        """Convolutions (with their BatchNorm) and the classifier (BatchNorm None), in
        forward order: conv1, then per bottleneck c1, c2, c3 and the projection."""
        out = [(self.conv1, self.bn1)]
        for blk in self.blocks:
            out.extend(blk.kfac_modules())
        out.append((self.fc, None))
        return out


# ---------------------------------------------------------------------------
# capture
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerGeom:
    """The kfac_layer fields of one captured layer."""
    n: int
    h: int
    w: int
    c_in: int
    h_out: int
    w_out: int
    c_out: int
    kh: int
    kw: int
    sh: int
    sw: int
    ph: int
    pw: int
    bias: int


@dataclass(frozen=True)
class BnGeom:
    n: int
    hw: int
    c: int


def _nhwc_half(x):
    """[n, c, h, w] (any memory format) or [n, c] -> contiguous NHWC fp16."""
    if x.dim() == 2:
        return x.detach().to(torch.float16).contiguous()
    return x.detach().permute(0, 2, 3, 1).to(torch.float16).contiguous()


class KfacCapture:
    """K-FAC for a model whose `kfac_modules()` lists (Conv2d or Linear, BatchNorm2d
    or None) pairs. Call `step(lr)` after `loss.backward()`: it forms the factors
    from the captured tensors, inverts them (every `refresh`-th call), preconditions
    the weight gradients and updates the weights and the BatchNorm parameters in
    place (eq. 8) through libkfac. precond_accum and refine_inverse are passed to
    KfacStep: "f64" sums the preconditioning products in fp64, refine_inverse takes
    one fp64-residual refinement step of every inverse. A real gradient lies in the
    range of its layer's factors, so where a factor is rank-deficient (batch smaller
    than its order) and the damping small, the preconditioning products cancel and
    amplify the inverses' fp32 error; the two options remove most of it."""

    def __init__(self, model, damping=1e-3, ema_decay=0.95, refresh_every=1, precond_accum="f32",
                 refine_inverse=False):
        self.model = model
        self.precond_accum = precond_accum
        self.refine_inverse = bool(refine_inverse)
        self.pairs = list(model.kfac_modules())
        self.damping = damping
        self.ema_decay = ema_decay
        self.refresh_every = refresh_every
        self.n = 0
        self.act = [None] * len(self.pairs)
        self.gout = [None] * len(self.pairs)
        self.bns = [bn for _, bn in self.pairs if bn is not None]
        self.xhat = [None] * len(self.bns)
        self.bgout = [None] * len(self.bns)
        self.kstep = None
        self.calls = 0
        self.hooks = []
        for i, (m, _) in enumerate(self.pairs):
            self.hooks.append(m.register_forward_hook(self._fwd(i)))
            self.hooks.append(m.register_full_backward_hook(self._bwd(i)))
        for i, bn in enumerate(self.bns):
            self.hooks.append(bn.register_forward_hook(self._bn_fwd(i)))
            self.hooks.append(bn.register_full_backward_hook(self._bn_bwd(i)))

    def remove(self):
        for h in self.hooks:
            h.remove()
        self.hooks = []

    # hooks ------------------------------------------------------------------
    def _fwd(self, i):
        def hook(mod, inp, out):
            if torch.is_grad_enabled():
                self.n = inp[0].shape[0]
                self.act[i] = _nhwc_half(inp[0])
        return hook

    def _bwd(self, i):
        def hook(mod, grad_in, grad_out):
            self.gout[i] = _nhwc_half(grad_out[0] * self.n)
        return hook

    def _bn_fwd(self, i):
        def hook(mod, inp, out):
            if torch.is_grad_enabled():
                x = inp[0].detach().float()
                var, mean = torch.var_mean(x, dim=(0, 2, 3), unbiased=False, keepdim=True)
                xh = (x - mean) * torch.rsqrt(var + mod.eps)
                self.xhat[i] = xh.permute(0, 2, 3, 1).reshape(x.shape[0], -1, x.shape[1]).to(
                    torch.float16).contiguous()
        return hook

    def _bn_bwd(self, i):
        def hook(mod, grad_in, grad_out):
            g = grad_out[0] * self.n
            self.bgout[i] = g.permute(0, 2, 3, 1).reshape(g.shape[0], -1, g.shape[1]).to(
                torch.float16).contiguous()
        return hook

    # geometry and parameter layouts -------------------------------------------
    def _geometry(self):
        layers = []
        for (m, _), a, g in zip(self.pairs, self.act, self.gout):
            if isinstance(m, nn.Conv2d):
                n, h, w, c_in = a.shape
                _, h_out, w_out, c_out = g.shape
                layers.append(LayerGeom(n, h, w, c_in, h_out, w_out, c_out, m.kernel_size[0], m.kernel_size[1],
                                        m.stride[0], m.stride[1], m.padding[0], m.padding[1],
                                        1 if m.bias is not None else 0))
            else:
                n, c_in = a.shape
                layers.append(LayerGeom(n, 1, 1, c_in, 1, 1, g.shape[1], 1, 1, 1, 1, 0, 0,
                                        1 if m.bias is not None else 0))
        bns = [BnGeom(x.shape[0], x.shape[1], x.shape[2]) for x in self.xhat]
        return layers, bns

    @staticmethod
    def _to_matrix(m, grad=False):
        w = m.weight.grad if grad else m.weight.data
        if isinstance(m, nn.Conv2d):
            mat = w.permute(0, 2, 3, 1).reshape(w.shape[0], -1)
        else:
            mat = w
        if m.bias is not None:
            b = m.bias.grad if grad else m.bias.data
            mat = torch.cat([mat, b[:, None]], 1)
        return mat.float().contiguous()

    @staticmethod
    def _from_matrix(m, mat):
        if m.bias is not None:
            m.bias.data.copy_(mat[:, -1])
            mat = mat[:, :-1]
        if isinstance(m, nn.Conv2d):
            c_out, c_in, kh, kw = m.weight.shape
            m.weight.data.copy_(mat.reshape(c_out, kh, kw, c_in).permute(0, 3, 1, 2))
        else:
            m.weight.data.copy_(mat)

    # the K-FAC step -------------------------------------------------------------
    def step(self, lr):
        if any(a is None for a in self.act) or any(g is None for g in self.gout):
            raise RuntimeError("step() needs one forward and backward pass with the hooks in place")
        dev = self.act[0].device
        if self.kstep is None:
            layers, bns = self._geometry()
            self.kstep = KfacStep(layers, bns, dev, damping=self.damping, precond_accum=self.precond_accum,
                                  refine_inverse=self.refine_inverse)
            self.master = [self._to_matrix(m) for m, _ in self.pairs]
            self.bn_master = [torch.stack([bn.weight.data.float(), bn.bias.data.float()]).contiguous()
                              for bn in self.bns]
        grads = [self._to_matrix(m, grad=True) for m, _ in self.pairs]
        refresh = self.calls % self.refresh_every == 0
        decay = 0.0 if self.calls == 0 else self.ema_decay
        self.kstep.step(self.act, self.gout, grads, self.xhat, self.bgout, ema_decay=decay, refresh=refresh,
                        weights=self.master, bn_params=self.bn_master, lr=lr)
        self.calls += 1
        for (m, _), mat in zip(self.pairs, self.master):
            self._from_matrix(m, mat)
        for bn, p in zip(self.bns, self.bn_master):
            bn.weight.data.copy_(p[0])
            bn.bias.data.copy_(p[1])
