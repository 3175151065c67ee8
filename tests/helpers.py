"""Shared test helpers: device placement of generator inputs, oracle stages
for teacher forcing, and the comparison rules."""
from __future__ import annotations

import numpy as np
import torch

from oracle import svgear_oracle as orc
from synth.gen import bf16_bits


def to_dev(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    """float32 array holding bf16/fp32 values -> device tensor of that dtype (exact)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return torch.from_numpy(bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def i32(a, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def f32(a, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def check_labels_near_ties(X, C, lab_gpu, lab_orc, rel=1e-5):
    """GPU labels may differ from the oracle's only where the two centroids are
    within rel * max(1, D) of each other in squared distance (fp64, same C)."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C, np.float64)
    bad = np.flatnonzero(np.asarray(lab_gpu) != np.asarray(lab_orc))
    for n in bad:
        dg = ((X[n] - C[lab_gpu[n]]) ** 2).sum()
        do = ((X[n] - C[lab_orc[n]]) ** 2).sum()
        assert dg - do <= rel * max(1.0, do), (n, lab_gpu[n], lab_orc[n], dg, do)
    return bad.size


def mean_bound(X, perm, offsets):
    """Rigorous bound on an fp32 segment mean's error: (n + 2) u max|x| per cluster."""
    X = np.abs(np.asarray(X, np.float64))
    C = offsets.shape[0] - 1
    b = np.zeros(C)
    for c in range(C):
        lo, hi = int(offsets[c]), int(offsets[c + 1])
        if hi > lo:
            b[c] = (hi - lo + 2) * 2.0 ** -24 * X[perm[lo:hi]].max() + 1e-30
    return b


def oracle_stage_inputs(q, k, v, cq0, ck0, iters, density, scale):
    """Run the oracle layer for one head (all intermediates)."""
    return orc.layer(q, k, v, cq0, ck0, iters, density, scale)
