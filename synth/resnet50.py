"""ResNet-50 layer geometry as K-FAC sees it.

The network is the 50-layer residual network of He et al. (2016) that Osawa et al.
train with distributed K-FAC (Section 1, Table 1). Each convolution becomes one
K-FAC layer with an activation tensor (NHWC, the layer's input) and an output
gradient tensor (NHWC, the layer's output); the classifier is the k=1, H=W=1 case.

Reading where the pages are silent: the stride-2 of a downsampling bottleneck sits on
its first 1x1 convolution and on the projection shortcut (the original ResNet v1
layout). Every K-FAC layer carries a bias column (constant 1) in its activation
factor, which makes the 3x3x64 factor 577 wide and the classifier factor 2049 wide.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Layer:
    name: str
    n: int          # batch
    h: int          # input height
    w: int          # input width
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
    bias: int = 1

    @property
    def rows(self) -> int:
        """Patch rows R = N * H_out * W_out."""
        return self.n * self.h_out * self.w_out

    @property
    def d_a(self) -> int:
        return self.c_in * self.kh * self.kw + (1 if self.bias else 0)

    @property
    def d_g(self) -> int:
        return self.c_out

    @property
    def act_shape(self):
        return (self.n, self.h, self.w, self.c_in)

    @property
    def gout_shape(self):
        return (self.n, self.h_out, self.w_out, self.c_out)


@dataclass(frozen=True)
class BNLayer:
    name: str
    n: int
    hw: int
    c: int

    @property
    def shape(self):
        return (self.n, self.hw, self.c)


def _conv(name, n, h, c_in, c_out, k, s, bias=1):
    p = k // 2
    h_out = (h + 2 * p - k) // s + 1
    return Layer(name, n, h, h, c_in, h_out, h_out, c_out, k, k, s, s, p, p, bias)


def conv_layers(batch: int = 32, bias: int = 1):
    """The 53 convolutions and the classifier of ResNet-50 at 224x224 input, in
    forward order. Returns a list of ``Layer``."""
    L = [_conv("conv1", batch, 224, 3, 64, 7, 2, bias)]
    h = 56                       # after the 3x3/2 max-pool
    c_prev = 64
    stages = [(2, 3, 64, 256, 1), (3, 4, 128, 512, 2), (4, 6, 256, 1024, 2), (5, 3, 512, 2048, 2)]
    for st, blocks, width, out, stride in stages:
        for b in range(blocks):
            s = stride if b == 0 else 1
            pre = f"s{st}b{b}"
            L.append(_conv(pre + ".c1", batch, h, c_prev, width, 1, s, bias))
            h2 = L[-1].h_out
            L.append(_conv(pre + ".c2", batch, h2, width, width, 3, 1, bias))
            L.append(_conv(pre + ".c3", batch, h2, width, out, 1, 1, bias))
            if b == 0:
                L.append(_conv(pre + ".proj", batch, h, c_prev, out, 1, s, bias))
            h, c_prev = h2, out
    L.append(Layer("fc", batch, 1, 1, 2048, 1, 1, 1000, 1, 1, 1, 1, 0, 0, bias))
    return L


def bn_layers(batch: int = 32):
    """One BatchNorm layer after each convolution: x-hat and its gradient are
    [N, H_out*W_out, C_out] for that convolution."""
    return [BNLayer("bn_" + l.name, batch, l.h_out * l.w_out, l.c_out)
            for l in conv_layers(batch) if l.name != "fc"]
