"""Seeded synthetic inputs for the SVG-EAR hot path.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, so both the fp64 oracle tests and the HIP path can take
their inputs from it.

The pages measure on real Wan 2.1 / HunyuanVideo activations driven by VBench
prompts; neither the models nor the prompt suite are available, so seeded
Gaussian-mixture Q/K/V stand in for them.  They keep the layer shapes the SVG2
summary gives ("5. Experimental Analysis", base models: 21 frames x 3600 tokens
for Wan 2.1, 33 x 3600 for HunyuanVideo, head dim 128) and the property that
tokens form tight semantic groups with different groupings for Q and K (SVG2
summary, "Semantic-Aware Permutation via k-Means Clustering": Q/K cluster ARI
of only 0.345).

Recipe, per head h with ``r = numpy.random.default_rng([seed, h])``:
  component weights w: uniform, or rank-size Zipf w_c ~ c^-1.1, independently
  permuted for Q and for K; component means MQ, MK, MV ~ N(0, 1) in R^{C x d};
  per-component sigma (0.3, or a 1:2 mix of 0.1 and 0.6); query label a_t ~ w^Q
  and key label b_t ~ w^K drawn independently; q_t = MQ[a_t] + sigma_{a_t} eps,
  k_t = MK[b_t] + sigma_{b_t} eps', v_t = MV[b_t] + sigma_{b_t} eps''; values
  cast to bf16 (round to nearest even) or kept fp32.  Cold k-means starts are
  C distinct token rows, r.choice(N, C, replace=False), one draw each for Q and
  K.  The denoising-step sequence drifts the means by 0.02 N(0, 1) per step
  (draws from default_rng([seed, h, step])) with labels and noise fixed.
  The words a k-means++ seeding consumes (one uniform 64-bit integer per
  seed) come from default_rng([seed, h, 11, 0 for Q / 1 for K]).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str            # "f32" or "bf16"
    comps: int            # mixture components per head
    zipf: Optional[float]  # None = uniform weights
    sigma: float          # component sigma (ignored when sigma_mix)
    Cq: int
    Ck: int
    iters: int
    density: float
    seed: int
    sigma_mix: bool = False
    steps: int = 1        # denoising steps (sequence workload)
    drift: float = 0.0
    iters_warm: int = 1
    densities: Sequence[float] = ()


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 2, 2048, 64, "f32", 16, None, 0.3, 16, 32, 10, 0.30, 0),
    "wan": Workload("wan", 1, 40, 75600, 128, "bf16", 400, 1.1, 0.3, 100, 500, 20, 0.25, 1),
    "hunyuan": Workload("hunyuan", 1, 24, 118800, 128, "bf16", 600, 1.1, 0.3, 100, 500, 20, 0.25, 2),
    "sequence": Workload("sequence", 1, 40, 75600, 128, "bf16", 400, 1.1, 0.3, 100, 500, 40, 0.25, 3,
                         steps=50, drift=0.02, iters_warm=1),
    "sweep": Workload("sweep", 1, 24, 118800, 128, "bf16", 600, 1.1, 0.3, 100, 500, 20, 0.25, 4,
                      sigma_mix=True, densities=(0.10, 0.15, 0.25, 0.40, 1.00)),
}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller test shapes)."""
    return dataclasses.replace(w, **kw)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _cast(w: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_round(x) if w.dtype == "bf16" else x.astype(np.float32, copy=False)


class HeadDraw:
    """All random draws of one (batch, head) slice; tensors for any step."""

    def __init__(self, w: Workload, bh: int):
        self.w = w
        r = np.random.default_rng([w.seed, bh])
        C, N, D = w.comps, w.N, w.D
        if w.zipf is None:
            base = np.full(C, 1.0 / C)
            wq, wk = base, base
        else:
            base = np.arange(1, C + 1, dtype=np.float64) ** (-w.zipf)
            base /= base.sum()
            wq = base[r.permutation(C)]
            wk = base[r.permutation(C)]
        if w.sigma_mix:
            sig = np.full(C, 0.6, dtype=np.float32)
            sig[r.permutation(C)[: C // 3]] = 0.1
        else:
            sig = np.full(C, w.sigma, dtype=np.float32)
        self.mq = r.standard_normal((C, D), dtype=np.float32)
        self.mk = r.standard_normal((C, D), dtype=np.float32)
        self.mv = r.standard_normal((C, D), dtype=np.float32)
        self.a = r.choice(C, size=N, p=wq)
        self.b = r.choice(C, size=N, p=wk)
        self.sig = sig
        self.eq = r.standard_normal((N, D), dtype=np.float32)
        self.ek = r.standard_normal((N, D), dtype=np.float32)
        self.ev = r.standard_normal((N, D), dtype=np.float32)
        self.init_q = r.choice(N, size=w.Cq, replace=False)
        self.init_k = r.choice(N, size=w.Ck, replace=False)
        self.bh = bh

    def drift_increments(self, s: int):
        """The float32 increments of the Q, K, V component means at step s >= 1
        (drift times a standard normal draw from default_rng([seed, h, s]))."""
        rs = np.random.default_rng([self.w.seed, self.bh, s])
        shp = self.mq.shape
        dq = self.w.drift * rs.standard_normal(shp, dtype=np.float32)
        dk = self.w.drift * rs.standard_normal(shp, dtype=np.float32)
        dv = self.w.drift * rs.standard_normal(shp, dtype=np.float32)
        return dq, dk, dv

    def means_at(self, step: int):
        mq, mk, mv = self.mq, self.mk, self.mv
        if step > 0 and self.w.drift > 0:
            mq, mk, mv = mq.copy(), mk.copy(), mv.copy()
            for s in range(1, step + 1):
                dq, dk, dv = self.drift_increments(s)
                mq += dq
                mk += dk
                mv += dv
        return mq, mk, mv

    def noise(self):
        """The per-token float32 offsets from the component means, sigma * eps
        for Q, K and V: a token is (its component's mean) + (its offset),
        added in float32 and then cast to the workload dtype."""
        sa = self.sig[self.a][:, None]
        sb = self.sig[self.b][:, None]
        return sa * self.eq, sb * self.ek, sb * self.ev

    def tensors(self, step: int = 0):
        """q, k, v (float32 arrays holding the values of the workload dtype)."""
        mq, mk, mv = self.means_at(step)
        nq, nk, nv = self.noise()
        q = _cast(self.w, mq[self.a] + nq)
        k = _cast(self.w, mk[self.b] + nk)
        v = _cast(self.w, mv[self.b] + nv)
        return q, k, v


def head_inputs(w: Workload, bh: int, step: int = 0):
    """One head: dict with q, k, v [N, D] and cold starts cq0 [Cq, D], ck0 [Ck, D] (float32)."""
    d = HeadDraw(w, bh)
    q, k, v = d.tensors(step)
    return {
        "q": q, "k": k, "v": v,
        "cq0": q[d.init_q].astype(np.float32),
        "ck0": k[d.init_k].astype(np.float32),
        "labels_q": d.a, "labels_k": d.b,   # generating components (diagnostics only)
    }


def seed_words(w: Workload, bh: int, which: str, C: int) -> np.ndarray:
    """C uniform 64-bit words for the k-means++ seeding of one head's Q
    (which = "q") or K ("k"), from default_rng([seed, bh, 11, 0 or 1])."""
    r = np.random.default_rng([w.seed, bh, 11, 0 if which == "q" else 1])
    return r.integers(0, np.iinfo(np.uint64).max, size=C, dtype=np.uint64, endpoint=True)


def layer_inputs(w: Workload, heads: Optional[Sequence[int]] = None, step: int = 0):
    """Stack heads into [BH, N, D] float32 arrays (heads default: all B*H)."""
    heads = list(range(w.B * w.H)) if heads is None else list(heads)
    out = {key: [] for key in ("q", "k", "v", "cq0", "ck0")}
    for bh in heads:
        hi = head_inputs(w, bh, step)
        for key in out:
            out[key].append(hi[key])
    return {key: np.stack(val) for key, val in out.items()}
