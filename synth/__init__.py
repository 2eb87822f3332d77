"""Seeded synthetic inputs for the K-FAC step (shapes and random numbers only).

This package holds no arithmetic of the method. It is the one module that both the
fp64 oracle (under ``oracle/``) and the HIP path are fed from, so that both sides see
bit-identical inputs:

* ``resnet50``: the layer geometry of ResNet-50 (He et al. 2016, the network trained
  in Osawa et al., "Large-scale distributed second-order optimization using
  Kronecker-factored approximate curvature for deep convolutional neural networks",
  Section 1 and Table 1), expressed as convolution/FC layers and BatchNorm layers.
* ``draw``: seeded NumPy draws in fp64, rounded once to the storage dtype.
"""
from .resnet50 import conv_layers, bn_layers, Layer, BNLayer  # noqa: F401
from .draw import (  # noqa: F401
    layer_rng, normal_f16, relu_normal_f16, normal_f32, config_seed,
)
