"""Shared helpers of the GPU parity tests (no arithmetic of the method here)."""
import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def relF(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def say(*a):
    print(*a, flush=True)


S_GAMMA = float(np.float32(np.sqrt(1e-3)))   # per-factor damping sqrt(gamma), gamma = 1e-3
