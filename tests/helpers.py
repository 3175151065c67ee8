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


def topp_near_tie_row(P_row, k_sizes, mask_row, p, tol=2e-4):
    """Whether a top-p row (oracle shares P_row, oracle selection mask_row) sits
    within tol of a different selection: the shares summed before or through
    the boundary cluster nearly equal p, or the boundary share nearly ties
    with the first share left out.  Only such rows may differ when the GPU
    computes its own shares."""
    k_sizes = np.asarray(k_sizes)
    order = [j for j in range(len(k_sizes)) if k_sizes[j] > 0]
    order.sort(key=lambda j: (-float(P_row[j]), j))
    Ps = np.array([float(P_row[j]) for j in order])
    cum = np.concatenate([[0.0], np.cumsum(Ps)])
    T = int(np.asarray(mask_row)[order].sum())
    if p >= 1.0 or T == 0:
        return False
    near = abs(cum[T] - p) <= tol or abs(cum[T - 1] - p) <= tol
    if T < len(order):
        near = near or Ps[T] >= (1.0 - tol) * Ps[T - 1]
    return bool(near)


def check_topp_masks(mask_gpu, P_o, mask_o, k_sizes, p, max_rows=None):
    """GPU top-p masks from the GPU's own shares: rows may differ from the
    oracle's only where the oracle's boundary is a near tie, and then in at most
    four clusters.  Returns the rows that differ."""
    rows = np.flatnonzero((np.asarray(mask_gpu) != np.asarray(mask_o)).any(axis=1))
    for i in rows:
        assert topp_near_tie_row(P_o[i], k_sizes, mask_o[i], p), i
        assert (mask_gpu[i] != mask_o[i]).sum() <= 4, i
    if max_rows is not None:
        assert rows.size <= max_rows, rows
    return rows


def check_ratio_masks(mask_gpu, r_o, mask_o, rows=None, rel=4e-3):
    """Masks filled from the GPU's own ratios may differ from the oracle's only
    at ratio near-ties with the row's selection threshold."""
    rowmax = r_o.max(axis=1).astype(np.float64)
    diff_rows = np.flatnonzero((np.asarray(mask_gpu) != np.asarray(mask_o)).any(axis=1))
    n = 0
    for i in diff_rows:
        if rows is not None and i not in rows:
            continue
        thr = r_o[i][mask_o[i] == 1].min()
        diff = np.flatnonzero(mask_gpu[i] != mask_o[i])
        n += diff.size
        assert np.all(np.abs(r_o[i][diff] - thr) <= rel * thr + 1e-7 * rowmax[i]), (i, diff)
    return n


def first_divergence(gpu_labels_after, X, C0, iters, rel=1e-5):
    """Lloyd iterations amplify a near tie (a token whose two nearest
    centroids agree to float32 rounding) into later label changes, so several
    final label sets are correct.  This finds the first round r whose GPU
    labels (``gpu_labels_after(r)``: the head's labels after r rounds from C0)
    differ from the oracle's Lloyd iterate and asserts that there they differ
    only at near ties for the oracle's centroids of round r - 1.  Returns
    (r, number of differing labels), or (None, 0) if no round differs."""
    X = np.asarray(X, np.float64)
    C = np.asarray(C0, np.float64)
    for r in range(1, iters + 1):
        lab_o = orc.assign(X, C)
        lab_g = np.asarray(gpu_labels_after(r))
        if (lab_g != lab_o).any():
            return r, check_labels_near_ties(X, C, lab_g, lab_o, rel)
        C = orc.update(X, lab_o, C)
    return None, 0


def oracle_from_labels(q, k, v, lq, lk, Cq, Ck, scale, density):
    """The oracle's permutation, means, routing ratios and mask for given final
    k-means labels (the GPU's own, once they have been shown valid): every
    stage after the clustering, so that a layer whose labels legitimately
    differ from the oracle's Lloyd iterates is still checked end to end."""
    N = q.shape[0]
    out = {}
    out["pq"], out["oq"] = orc.permute(np.asarray(lq, np.int64), Cq)
    out["pk"], out["ok"] = orc.permute(np.asarray(lk, np.int64), Ck)
    out["qbar"] = orc.means(q, out["pq"], out["oq"])
    out["kbar"] = orc.means(k, out["pk"], out["ok"])
    out["vbar"] = orc.means(v, out["pk"], out["ok"])
    qs, ks = np.diff(out["oq"]), np.diff(out["ok"])
    Kp, Vp = np.asarray(k)[out["pk"]], np.asarray(v)[out["pk"]]
    e, _ = orc.probe_errors(out["qbar"], Kp, Vp, out["kbar"], out["vbar"], out["ok"], scale, q_nonempty=qs > 0)
    out["ratio"] = orc.ratios(e, qs, ks)
    out["mask"] = orc.select(out["ratio"], qs, ks, density, N)
    return out
