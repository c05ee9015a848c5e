"""Shared helpers for the test suite (marshalling and the tolerance rule)."""
import os

import numpy as np

from selective_scan_segmented_amd import synth

RTOL = {"f32": 1e-5, "bf16": 2e-2}


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_dev(a: np.ndarray, io: str = None):
    """numpy float32 array or uint16 bf16 bit patterns -> CUDA tensor of the same bytes."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.cuda()


def from_dev(t) -> np.ndarray:
    """CUDA tensor (float32 or bfloat16) -> exact float64 numpy array."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


def assert_close(g: np.ndarray, r: np.ndarray, io: str, what: str = ""):
    """Pass iff |g - r| <= rtol * (|r| + rms(r)) elementwise (rtol 1e-5 f32, 2e-2 bf16)."""
    rtol = RTOL[io]
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = rtol * (np.abs(r) + rms)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        worst = float(np.max(err / np.maximum(bound, 1e-300)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {r.size} outside tolerance (rtol {rtol}); "
                             f"worst err/bound {worst:.3g}; first bad at {idx.tolist()}: "
                             f"got {[float(g[tuple(i)]) for i in idx]}, want {[float(r[tuple(i)]) for i in idx]}")
    return float(err.max() / max(np.abs(r).max(), 1e-300)) if r.size else 0.0
