"""Seeded draws. Every array is drawn in fp64 from NumPy's PCG64 and rounded once
(round-to-nearest-even) to its storage dtype; the GPU and the oracle consume the same
rounded arrays. Config k uses ``default_rng`` streams spawned from ``SeedSequence(k)``,
one stream per (layer, tensor) index, so any single layer can be regenerated alone."""
import numpy as np

# one seed per workload: the fc layer (1), one 3x3 convolution (2), the full
# ResNet-50 step (3), the inversion stress set (4), the stale-curvature schedule (5)
_CONFIG_SEEDS = {"fc": 1, "conv3x3": 2, "resnet50": 3, "invert_stress": 4, "stale": 5}


def config_seed(name: str) -> int:
    return _CONFIG_SEEDS[name]


def layer_rng(seed: int, index: int) -> np.random.Generator:
    """Independent generator for item ``index`` of workload ``seed``."""
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(index,))
    return np.random.default_rng(ss)


def normal_f16(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float16)


def relu_normal_f16(rng, shape, std=1.0):
    return np.maximum(rng.standard_normal(shape) * std, 0.0).astype(np.float16)


def normal_f32(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)
