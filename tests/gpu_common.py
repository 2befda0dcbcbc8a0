"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch

TOL = {"f16": 5e-3, "bf16": 1e-2}


def rel_fro(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-12))


def max_abs(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    i = int(np.argmax(d))
    return float(d.reshape(-1)[i]), np.unravel_index(i, d.shape)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def say(*a):
    print(*a, flush=True)
