"""Helpers shared by the GPU parity tests."""
import numpy as np
import torch

TOL = {"f16": 5e-3, "bf16": 1e-2}
# significand bits of the output dtypes (for the element-wise bound)
_MANT = {"f16": 10, "bf16": 7}


def rel_fro(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-12))


def max_abs(got, ref):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    i = int(np.argmax(d))
    return float(d.reshape(-1)[i]), np.unravel_index(i, d.shape)


def ulp(x, dt: str):
    """Spacing of the output dtype at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -14)))
    return 2.0 ** (e - _MANT[dt])


def elementwise_check(got, ref, dt: str, k: float = 16.0):
    """|G - O| <= k ulp(max(|O|, rms(O))) element by element (k = 16).

    The GPU output is the oracle's fp32 value rounded once to the output
    dtype (half an ulp) plus what the fp16 / bf16 intermediates the GPU
    stores (the oracle keeps fp32) carry forward, a few ulps of the
    output's scale.  The floor at rms(O) keeps outputs near zero from being
    held to their own tiny ulp.  A wrong tile (stale data, a lost release,
    a wrong index) is off by about the output's scale and fails by far.
    Returns (ok, worst ratio, index of the worst element, max-abs)."""
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    scale = max(float(np.sqrt(np.mean(r * r))), 1e-6)
    bound = k * ulp(np.maximum(np.abs(r), scale), dt)
    err = np.abs(g - r)
    err = np.where(np.isnan(g), np.inf, err)
    ratio = err / bound
    i = int(np.argmax(ratio))
    idx = np.unravel_index(i, ratio.shape)
    return bool(ratio.reshape(-1)[i] <= 1.0), float(ratio.reshape(-1)[i]), idx, float(err.max())


def assert_parity(got, ref, dt: str, label: str = "", k: float = 16.0):
    """rel-Frobenius within the dtype's tolerance and the element-wise bound;
    prints and returns (rel, max-abs, index)."""
    rel = rel_fro(got, ref)
    ok, worst, idx, mx = elementwise_check(got, ref, dt, k)
    mabs, at = max_abs(got, ref)
    say(f"  {label} rel={rel:.3e} maxabs={mabs:.3e} at {tuple(int(v) for v in at)} "
        f"worst/bound={worst:.3f} at {tuple(int(v) for v in idx)}")
    assert rel <= TOL[dt], f"{label}: rel {rel} > {TOL[dt]}"
    assert ok, (f"{label}: element {tuple(int(v) for v in idx)} off by {worst:.2f}x its bound "
                f"(got {np.asarray(got).reshape(-1)[np.ravel_multi_index(idx, np.shape(got))]}, "
                f"want {np.asarray(ref).reshape(-1)[np.ravel_multi_index(idx, np.shape(ref))]})")
    return rel, mabs, at


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def say(*a):
    print(*a, flush=True)
