"""Plain fp64 CPU oracle for the SVG-EAR sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check of the package entry
point and the CPU-baseline leg of the benchmark may import or run this module.
It shares no code with the HIP path and never imports it.

Everything is numpy float64, one (batch, head) slice at a time, written for
reading rather than speed.  The method is an approximation, so the oracle
follows the pages' steps in order:

  1. ``lloyd``    k-means of Q (C_q clusters) and of K (C_k clusters) from a
                  given start (SVG2 summary, "Semantic-Aware Permutation via
                  k-Means Clustering"; centroid cache in "Efficient
                  System-Algorithm Co-Design").
  2. ``permute``  cluster-contiguous order, K and V sharing one permutation
                  (SVG2 summary, "The permutation operation and its
                  mathematical validity").
  3. ``means``    per-cluster means of Q, K and V (SVG-EAR task page, "What
                  the agent has to build": one routine averages each cluster).
  4. ``route``    the probe error of every (query cluster, key cluster) block,
                  divided by its cost |Q_i| |K_j|, then a greedy fill to the
                  density budget (FrontierCS blog on SVG-EAR, the probe formula
                  and the budget paragraph; Pith review, "What carries the
                  argument").
  5. ``attend``   selected blocks exactly, every skipped non-empty key cluster
                  as one centroid key whose score is raised by ln n_j with the
                  cluster's mean value (FrontierCS blog, toy example: weight
                  n e^{s_bar}; SVG-EAR task page, step 3 of the walkthrough),
                  output in original token order.

Readings taken where the pages are silent (each also listed in the design
notes): squared L2 distance with ties to the lowest index; empty k-means
clusters keep their centroid; stable within-cluster order; the probe error is
stabilised by the row maximum M_i of the probe scores (the per-row ranking is
unchanged by that common factor); the budget is rho * N_k keys per query
cluster and the block that crosses it is included; ties in ratio break to the
lower key-cluster index; compensation uses each query token against the exact
means of the current assignment; no variance term in the plain method.

Variance-corrected compensation (a variant the FrontierCS blog describes in
its paragraph on the centroid's low guess): a skipped cluster's score is
raised by strength * sigma^2 / 2 with sigma^2 = (1/d) sum_i q_i^2 Var(k_i),
the per-coordinate population variance of the cluster's keys.  ``variances``
and the ``kvar`` / ``strength`` arguments of ``attend`` implement it;
strength 0 is the plain method.

k-means++ seeding (SVG2 summary, "Efficient System-Algorithm Co-Design"):
``kmeanspp`` draws cold-start centroids by D^2 sampling from caller-given
uniform 64-bit words.  Readings: squared distances summed in coordinate
order in float64 without fused operations, sampling weights floor(D^2 2^k)
as exact integers, inverse-CDF draws, uniform fallback once every distance
is 0.

FP8 variant (SVG2 summary, results: SVG2 + FP8): ``quantize_e4m3`` gives a
slice's e4m3fn codes and power-of-two scale; the FP8 attention is ``attend``
on the dequantized Q and K (the products of the exact blocks then equal the
kernel's e4m3 products), with the values and the cluster means unquantized.

Top-p budget (SVG2 summary, "Centroid-Based Top-p Selection"; FrontierCS
blog, budget paragraph): ``topp_probs`` estimates each block's share P' of
the attention mass from the centroids, ``topp_select`` is SVG2's own router
(clusters by P' until the shares taken reach p) and ``route_topp`` with
error_ranked=True gives each query cluster that selection's keys as its
budget and spends them by error per pair instead of a fixed density.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# 1. k-means (Lloyd rounds)
# --------------------------------------------------------------------------
def sqdist(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Squared Euclidean distances D[n, c] = ||x_n - c_c||^2 in fp64.

    Euclidean distance on the activation vectors is the clustering metric of
    the SVG2 summary ("What gets clustered and why")."""
    X = np.asarray(X, F64)
    C = np.asarray(C, F64)
    xx = np.einsum("nd,nd->n", X, X)
    cc = np.einsum("cd,cd->c", C, C)
    D = xx[:, None] + cc[None, :] - 2.0 * (X @ C.T)
    return np.maximum(D, 0.0)


def assign(X: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Label of each row = index of its nearest centroid, ties to the lowest index."""
    return np.argmin(sqdist(X, C), axis=1).astype(np.int64)


def update(X: np.ndarray, labels: np.ndarray, C_old: np.ndarray) -> np.ndarray:
    """New centroid = mean of its members; an empty cluster keeps its old centroid."""
    X = np.asarray(X, F64)
    C = np.array(C_old, F64, copy=True)
    k = C.shape[0]
    counts = np.bincount(labels, minlength=k)
    sums = np.zeros_like(C)
    np.add.at(sums, labels, X)
    nz = counts > 0
    C[nz] = sums[nz] / counts[nz, None]
    return C


def lloyd(X: np.ndarray, C0: np.ndarray, iters: int):
    """``iters`` rounds of (assign, update) from the start C0.

    Cold starts come from the caller; warm starts are the previous denoising
    step's centroids (SVG2 summary, centroid cache: 1-3 rounds from the cached
    centroids instead of 100+ from k-means++).  Returns (centroids after the
    last update, labels of the last assignment)."""
    if iters < 1:
        raise ValueError("iters must be >= 1")
    C = np.array(C0, F64, copy=True)
    labels = None
    for _ in range(iters):
        labels = assign(X, C)
        C = update(X, labels, C)
    return C, labels


# --------------------------------------------------------------------------
# 1b. k-means++ cold seeding (SVG2 summary, "Efficient System-Algorithm
#     Co-Design": a cold start uses k-means++ initialisation)
# --------------------------------------------------------------------------
def sqdist_seq(X: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Squared distance of every row of X to c, summed over the coordinates in
    index order in float64, one rounding per product and one per sum (no fused
    multiply-add).  The seeding's random choices depend on these values, so the
    order of operations is fixed here and on the GPU alike."""
    X = np.asarray(X, F64)
    c = np.asarray(c, F64)
    acc = np.zeros(X.shape[0], F64)
    for d in range(X.shape[1]):
        diff = X[:, d] - c[d]
        acc = acc + diff * diff
    return acc


def pp_scale(d2_first: np.ndarray) -> int:
    """Exponent k of the fixed-point sampling weights floor(D^2 * 2^k): the
    largest k with N * max D^2 * 2^k < 2^62, taken from the distances to the
    first seed (later distances only shrink, so every later sum fits)."""
    m = float(np.max(d2_first))
    if m == 0.0:
        return 0
    _, e = math.frexp(float(len(d2_first)) * m)     # N * m < 2^e
    return 62 - e


def pp_weights(d2: np.ndarray, k: int) -> np.ndarray:
    """D^2 as exact non-negative integers floor(D^2 * 2^k) (uint64)."""
    return np.floor(np.ldexp(np.asarray(d2, F64), k)).astype(np.uint64)


def pp_draw(weights: np.ndarray, word: int):
    """Index drawn with probability weight / total by inverting the cumulative
    sum at target = floor(word * total / 2^64), word a uniform 64-bit integer:
    the first index whose inclusive prefix exceeds the target.  None when every
    weight is 0."""
    total = int(np.sum(weights, dtype=np.uint64))
    if total == 0:
        return None
    target = (int(word) * total) >> 64
    cum = np.cumsum(weights, dtype=np.uint64)
    return int(np.searchsorted(cum, np.uint64(target), side="right"))


def kmeanspp(X: np.ndarray, words: np.ndarray, C: int):
    """k-means++ seeds (D^2 sampling): the first seed is token
    floor(words[0] * N / 2^64); each later seed c is drawn with probability
    proportional to the squared distance to the nearest seed so far, using
    words[c].  When every remaining distance is 0 (fewer distinct rows than
    seeds) the draw falls back to the uniform rule.  Returns (seeds as float64
    rows [C, D], their token indices [C])."""
    X = np.asarray(X, F64)
    N = X.shape[0]
    chosen = [(int(words[0]) * N) >> 64]
    d2 = sqdist_seq(X, X[chosen[0]])
    k = pp_scale(d2)
    for c in range(1, C):
        t = pp_draw(pp_weights(d2, k), int(words[c]))
        if t is None:
            t = (int(words[c]) * N) >> 64
        chosen.append(t)
        d2 = np.minimum(d2, sqdist_seq(X, X[t]))
    idx = np.asarray(chosen, dtype=np.int64)
    return X[idx].copy(), idx


def inertia(X: np.ndarray, C: np.ndarray, labels: np.ndarray) -> float:
    X = np.asarray(X, F64)
    return float(((X - np.asarray(C, F64)[labels]) ** 2).sum())


# --------------------------------------------------------------------------
# 2. permutation
# --------------------------------------------------------------------------
def permute(labels: np.ndarray, C: int):
    """Cluster-contiguous order: perm[p] = source token of slot p.

    Tokens of cluster 0 come first, then cluster 1, and so on; inside a
    cluster tokens keep their original order.  offsets[c]..offsets[c+1] is
    cluster c's slot range (SVG2 summary: the permutation groups all tokens
    of cluster 1 first, then cluster 2, ...)."""
    labels = np.asarray(labels)
    counts = np.bincount(labels, minlength=C)
    offsets = np.zeros(C + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    # stable counting sort written out: each token goes to the next free slot
    # of its cluster, scanning tokens in original order
    nxt = offsets[:-1].copy()
    perm = np.empty(labels.shape[0], dtype=np.int64)
    for t, c in enumerate(labels):
        perm[nxt[c]] = t
        nxt[c] += 1
    return perm, offsets


# --------------------------------------------------------------------------
# 3. means
# --------------------------------------------------------------------------
def means(X: np.ndarray, perm: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Mean of each cluster's rows; an empty cluster's mean is defined as 0."""
    X = np.asarray(X, F64)
    C = offsets.shape[0] - 1
    out = np.zeros((C, X.shape[1]), F64)
    for c in range(C):
        lo, hi = int(offsets[c]), int(offsets[c + 1])
        if hi > lo:
            out[c] = X[perm[lo:hi]].mean(axis=0)
    return out


def variances(X: np.ndarray, perm: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Per-coordinate population variance of each cluster's rows, Var(x_i) =
    mean over members of (x_i - mean_i)^2 (FrontierCS blog, variance
    correction: one variance per key coordinate; its two-key example, scores
    0 and 2, has variance 1, i.e. the mean of squared deviations).  An empty
    cluster's variance is defined as 0."""
    X = np.asarray(X, F64)
    C = offsets.shape[0] - 1
    out = np.zeros((C, X.shape[1]), F64)
    for c in range(C):
        lo, hi = int(offsets[c]), int(offsets[c + 1])
        if hi > lo:
            rows = X[perm[lo:hi]]
            out[c] = ((rows - rows.mean(axis=0)) ** 2).mean(axis=0)
    return out


# --------------------------------------------------------------------------
# 4. error-aware routing
# --------------------------------------------------------------------------
def probe_errors(qbar, Kp, Vp, kbar, vbar, k_offsets, scale, q_nonempty=None):
    """Probe error e[i, j] of replacing key cluster j by its centroid, for the
    probe q_bar_i (the mean query of cluster i).

    FrontierCS blog on SVG-EAR, probe paragraph: with s_k the probe's score for
    key k and s_bar, v_bar belonging to the key's cluster, the block's error is
    the sum over its keys of || e^{s_bar} v_bar - e^{s_k} v_k ||^2.  Both
    exponentials are taken relative to the row maximum M_i = max_k s_ik, which
    scales a whole row of errors by e^{-2 M_i} and so leaves the per-row
    ranking unchanged.  Kp, Vp are the keys/values in cluster-contiguous order.
    Returns (e [Cq, Ck], M [Cq])."""
    qbar = np.asarray(qbar, F64)
    Kp = np.asarray(Kp, F64)
    Vp = np.asarray(Vp, F64)
    kbar = np.asarray(kbar, F64)
    vbar = np.asarray(vbar, F64)
    Cq, Ck = qbar.shape[0], kbar.shape[0]
    S = scale * (qbar @ Kp.T)              # probe score of every key, [Cq, N]
    M = S.max(axis=1)
    sbar = scale * (qbar @ kbar.T)         # centroid score, [Cq, Ck]
    e = np.zeros((Cq, Ck), F64)
    for j in range(Ck):
        lo, hi = int(k_offsets[j]), int(k_offsets[j + 1])
        if hi == lo:
            continue
        a = np.exp(sbar[:, j] - M)                         # estimate weight per key
        for c0 in range(lo, hi, 2048):                     # chunk keys to bound memory
            c1 = min(hi, c0 + 2048)
            b = np.exp(S[:, c0:c1] - M[:, None])           # true weight per key
            diff = a[:, None, None] * vbar[j][None, None, :] - b[:, :, None] * Vp[c0:c1][None, :, :]
            e[:, j] += np.einsum("ikd,ikd->i", diff, diff)
    if q_nonempty is not None:
        e[~q_nonempty] = 0.0
        M = np.where(q_nonempty, M, 0.0)
    return e, M


def ratios(e, q_sizes, k_sizes) -> np.ndarray:
    """Error-to-cost ratio r_ij = e_ij / (|Q_i| |K_j|), as float32.

    The blog divides the error by the number of token pairs in the block; the
    Pith review calls it the error-to-cost ratio.  Empty clusters get 0.  The
    selection compares these float32 values."""
    q_sizes = np.asarray(q_sizes, F64)
    k_sizes = np.asarray(k_sizes, F64)
    cost = q_sizes[:, None] * k_sizes[None, :]
    r = np.zeros_like(np.asarray(e, F64))
    nz = cost > 0
    r[nz] = np.asarray(e, F64)[nz] / cost[nz]
    return r.astype(np.float32)


def budget_keys(density: float, Nk: int) -> float:
    """Key budget per query cluster, rho * N_k, with rho read as a float32."""
    return float(np.float32(density)) * float(Nk)


def select_row(r_row: np.ndarray, k_sizes: np.ndarray, budget: float) -> np.ndarray:
    """Greedy fill of one query cluster's row (Pith review, "What carries the
    argument": highest error-to-cost blocks first, under a density budget).

    Order the non-empty key clusters by (ratio descending, index ascending);
    take a cluster while the keys already taken are below the budget, so the
    cluster that crosses the budget is included."""
    k_sizes = np.asarray(k_sizes)
    cand = [j for j in range(r_row.shape[0]) if k_sizes[j] > 0]
    cand.sort(key=lambda j: (-float(r_row[j]), j))
    sel = np.zeros(r_row.shape[0], dtype=np.uint8)
    taken = 0
    for j in cand:
        if taken >= budget:
            break
        sel[j] = 1
        taken += int(k_sizes[j])
    return sel


def select(r: np.ndarray, q_sizes, k_sizes, density: float, Nk: int) -> np.ndarray:
    """Routing mask [Cq, Ck]; rows of empty query clusters stay all zero."""
    budget = budget_keys(density, Nk)
    mask = np.zeros(r.shape, dtype=np.uint8)
    for i in range(r.shape[0]):
        if q_sizes[i] > 0:
            mask[i] = select_row(r[i], k_sizes, budget)
    return mask


def route(qbar, q_offsets, Kp, Vp, kbar, vbar, k_offsets, scale, density):
    """Full routing step: (float32 ratios [Cq, Ck], mask [Cq, Ck])."""
    q_sizes = np.diff(np.asarray(q_offsets))
    k_sizes = np.diff(np.asarray(k_offsets))
    e, _ = probe_errors(qbar, Kp, Vp, kbar, vbar, k_offsets, scale, q_nonempty=q_sizes > 0)
    r = ratios(e, q_sizes, k_sizes)
    return r, select(r, q_sizes, k_sizes, density, Kp.shape[0])


# --------------------------------------------------------------------------
# 4b. the SVG2 top-p budget and the score-ranked router
# --------------------------------------------------------------------------
def topp_probs(qbar, kbar, k_sizes, scale) -> np.ndarray:
    """Estimated attention mass P'[i, j] of key cluster j for query cluster i,
    as float32 (SVG2 summary, "Centroid-Based Top-p Selection").

    The centroid score is S_ij = scale * q_bar_i . k_bar_j, and
    P'_ij = |K_j| e^{S_ij} / sum_l |K_l| e^{S_il}: each key of cluster j is
    taken to score S_ij, so the numerator estimates the cluster's total weight
    and each row sums to 1.  Empty key clusters (|K_j| = 0) get 0 and do not
    take part in the row maximum used to keep the exponentials finite.  The
    selection compares these float32 values."""
    k_sizes = np.asarray(k_sizes)
    S = scale * (np.asarray(qbar, F64) @ np.asarray(kbar, F64).T)
    live = k_sizes > 0
    P = np.zeros(S.shape, F64)
    for i in range(S.shape[0]):
        m = S[i, live].max()
        w = np.where(live, k_sizes * np.exp(np.where(live, S[i] - m, 0.0)), 0.0)
        P[i] = w / w.sum()
    return P.astype(np.float32)


def topp_select_row(P_row: np.ndarray, k_sizes: np.ndarray, p: float) -> np.ndarray:
    """Top-p selection of one query cluster's key clusters (SVG2 summary,
    "Centroid-Based Top-p Selection", steps 1-3).

    Order the non-empty key clusters by (P' descending, index ascending) and
    take them while the P' already taken, summed in that order in float64,
    is below p; the cluster whose P' reaches p is included.  p >= 1 takes
    every non-empty cluster (a sum of rounded terms may touch 1 early)."""
    k_sizes = np.asarray(k_sizes)
    cand = [j for j in range(P_row.shape[0]) if k_sizes[j] > 0]
    cand.sort(key=lambda j: (-float(P_row[j]), j))
    sel = np.zeros(P_row.shape[0], dtype=np.uint8)
    p = float(np.float32(p))
    cum = 0.0
    for j in cand:
        if p < 1.0 and cum >= p:
            break
        sel[j] = 1
        cum += float(P_row[j])
    return sel


def topp_select(P: np.ndarray, q_sizes, k_sizes, p: float) -> np.ndarray:
    """The SVG2 router's mask [Cq, Ck]; rows of empty query clusters are zero."""
    mask = np.zeros(P.shape, dtype=np.uint8)
    for i in range(P.shape[0]):
        if q_sizes[i] > 0:
            mask[i] = topp_select_row(P[i], k_sizes, p)
    return mask


def topp_budgets(topp_mask: np.ndarray, k_sizes) -> np.ndarray:
    """Key budget per query cluster from a top-p selection (FrontierCS blog
    on SVG-EAR, the budget paragraph: the token pairs in the blocks holding a
    fraction p of the estimated weight).  Row i's pairs are |Q_i| times its
    selected keys, so the budget is kept in keys: int64 [Cq]."""
    return (np.asarray(topp_mask, np.int64) * np.asarray(k_sizes, np.int64)[None, :]).sum(axis=1)


def select_budgets(r: np.ndarray, q_sizes, k_sizes, budgets) -> np.ndarray:
    """Greedy fill of each row to its own key budget (the same fill as
    ``select_row``: ratio descending, crossing block included)."""
    mask = np.zeros(r.shape, dtype=np.uint8)
    for i in range(r.shape[0]):
        if q_sizes[i] > 0:
            mask[i] = select_row(r[i], k_sizes, float(budgets[i]))
    return mask


def route_topp(qbar, q_offsets, Kp, Vp, kbar, vbar, k_offsets, scale, p, error_ranked=True):
    """Routing under the SVG2 budget.

    error_ranked=False: the SVG2 router itself, top-p over P'.
    error_ranked=True:  SVG-EAR's use of that budget (FrontierCS blog, budget
    paragraph): each query cluster gets the keys of its top-p selection and
    spends them on the blocks with the highest error per pair.
    Returns (P' float32 [Cq, Ck], ratios float32 [Cq, Ck] or None,
    budgets int64 [Cq], mask [Cq, Ck])."""
    q_sizes = np.diff(np.asarray(q_offsets))
    k_sizes = np.diff(np.asarray(k_offsets))
    P = topp_probs(qbar, kbar, k_sizes, scale)
    P[q_sizes == 0] = 0.0
    tmask = topp_select(P, q_sizes, k_sizes, p)
    budgets = topp_budgets(tmask, k_sizes)
    if not error_ranked:
        return P, None, budgets, tmask
    e, _ = probe_errors(qbar, Kp, Vp, kbar, vbar, k_offsets, scale, q_nonempty=q_sizes > 0)
    r = ratios(e, q_sizes, k_sizes)
    return P, r, budgets, select_budgets(r, q_sizes, k_sizes, budgets)


# --------------------------------------------------------------------------
# 5. sparse attention with centroid compensation
# --------------------------------------------------------------------------
def attend_rows(q_rows, K, V, k_perm, k_offsets, kbar, vbar, sel_row, scale, kvar=None, strength=0.0):
    """Outputs and log-sum-exp for query rows that share one routing row.

    Keys of selected clusters are attended exactly.  Each skipped non-empty
    key cluster j enters as one key k_bar_j with score q.k_bar_j * scale +
    ln n_j and value v_bar_j, i.e. weight n_j e^{q.k_bar_j scale} (FrontierCS
    blog toy example; SVG-EAR task page walkthrough step 3).  With ``kvar``
    (per-cluster coordinate variances) the score also gains
    strength * sigma^2 / 2, sigma^2 = scale^2 sum_i q_i^2 kvar_ji, the
    variance of the query's scores over the cluster under independent
    coordinates (FrontierCS blog, variance-correction paragraph)."""
    q_rows = np.asarray(q_rows, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    kbar = np.asarray(kbar, F64)
    vbar = np.asarray(vbar, F64)
    Ck = kbar.shape[0]
    sizes = np.diff(np.asarray(k_offsets))
    exact_idx = [k_perm[int(k_offsets[j]):int(k_offsets[j + 1])] for j in range(Ck) if sel_row[j]]
    exact_idx = np.concatenate(exact_idx) if exact_idx else np.zeros(0, np.int64)
    comp = [j for j in range(Ck) if (not sel_row[j]) and sizes[j] > 0]
    logits = [scale * (q_rows @ K[exact_idx].T)]
    values = [V[exact_idx]]
    if comp:
        comp = np.asarray(comp)
        pseudo = scale * (q_rows @ kbar[comp].T) + np.log(sizes[comp].astype(F64))[None, :]
        if kvar is not None and strength != 0.0:
            sigma2 = scale * scale * ((q_rows * q_rows) @ np.asarray(kvar, F64)[comp].T)
            pseudo = pseudo + strength * 0.5 * sigma2
        logits.append(pseudo)
        values.append(vbar[comp])
    L = np.concatenate(logits, axis=1)
    Vall = np.concatenate(values, axis=0)
    m = L.max(axis=1, keepdims=True)
    w = np.exp(L - m)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ Vall) / den
    lse = (m + np.log(den))[:, 0]
    return out, lse


def attend(Q, K, V, q_perm, q_offsets, k_perm, k_offsets, kbar, vbar, mask, scale, rows=None, kvar=None,
           strength=0.0):
    """O [N, D] and LSE [N] in original token order (SVG2 summary: the output
    is un-permuted back to the original order).

    ``rows`` optionally restricts the work to some original token indices;
    other outputs are left as NaN."""
    Q = np.asarray(Q, F64)
    N, D = Q.shape
    O = np.full((N, D), np.nan)
    LSE = np.full(N, np.nan)
    want = None if rows is None else set(int(t) for t in rows)
    Cq = q_offsets.shape[0] - 1
    for i in range(Cq):
        toks = q_perm[int(q_offsets[i]):int(q_offsets[i + 1])]
        if want is not None:
            toks = np.asarray([t for t in toks if int(t) in want], dtype=np.int64)
        if toks.size == 0:
            continue
        o, l = attend_rows(Q[toks], K, V, k_perm, k_offsets, kbar, vbar, mask[i], scale, kvar, strength)
        O[toks] = o
        LSE[toks] = l
    return O, LSE


def attend_bruteforce(Q, K, V, q_labels, k_labels, kbar, vbar, mask, scale):
    """Tiny-N cross-check of ``attend`` with explicit loops: one logit per
    (query, key) pair in a selected block, one per (query, skipped non-empty
    cluster), then a plain softmax-weighted average."""
    Q = np.asarray(Q, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    N, D = Q.shape
    Ck = kbar.shape[0]
    sizes = np.bincount(np.asarray(k_labels), minlength=Ck)
    O = np.zeros((N, D))
    for t in range(N):
        i = int(q_labels[t])
        logits, vals = [], []
        for u in range(K.shape[0]):
            if mask[i, int(k_labels[u])]:
                logits.append(scale * float(np.dot(Q[t], K[u])))
                vals.append(V[u])
        for j in range(Ck):
            if not mask[i, j] and sizes[j] > 0:
                logits.append(scale * float(np.dot(Q[t], kbar[j])) + np.log(float(sizes[j])))
                vals.append(np.asarray(vbar[j], F64))
        mx = max(logits)
        w = np.array([np.exp(s - mx) for s in logits])
        O[t] = (w[:, None] * np.array(vals)).sum(0) / w.sum()
    return O


# --------------------------------------------------------------------------
# 6. e4m3 quantisation for the FP8 attention variant (SVG2 summary, results:
#    SVG2 + FP8 on HunyuanVideo; the pages give no scheme)
# --------------------------------------------------------------------------
def e4m3_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (448: the largest finite
    e4m3fn value); 0 for amax = 0.  From amax = f 2^E with 0.5 <= f < 1 and
    448 = 0.875 * 2^9."""
    if not amax > 0.0:
        return 0
    f, E = math.frexp(float(amax))
    return E - 9 if f <= 0.875 else E - 8


def quantize_e4m3(X: np.ndarray):
    """One (batch, head) slice to e4m3fn codes with one power-of-two scale:
    codes = round-to-nearest-even e4m3fn of X * 2^-e (scaled in float32, which
    is exact), X ~ decode(codes) * 2^e.  The rounding is torch's float32 ->
    float8_e4m3fn conversion.  Returns (codes uint8, e)."""
    import torch
    X32 = np.asarray(X, np.float32)
    e = e4m3_exponent(float(np.max(np.abs(X32)))) if X32.size else 0
    scaled = np.ldexp(X32, -e).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(scaled)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, e


def dequantize_e4m3(codes: np.ndarray, e: int) -> np.ndarray:
    """decode(codes) * 2^e in float64 (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return np.ldexp(t.double().numpy(), e)


# --------------------------------------------------------------------------
# whole layer, one head
# --------------------------------------------------------------------------
def layer(q, k, v, cq0, ck0, iters, density, scale=None):
    """All steps for one head; returns a dict of every intermediate."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    Cq, Ck = cq0.shape[0], ck0.shape[0]
    cq, lq = lloyd(q, cq0, iters)
    ck, lk = lloyd(k, ck0, iters)
    pq, oq = permute(lq, Cq)
    pk, ok = permute(lk, Ck)
    qbar = means(q, pq, oq)
    kbar = means(k, pk, ok)
    vbar = means(v, pk, ok)
    r, mask = route(qbar, oq, k[pk], v[pk], kbar, vbar, ok, scale, density)
    O, LSE = attend(q, k, v, pq, oq, pk, ok, kbar, vbar, mask, scale)
    return dict(cq=cq, ck=ck, lq=lq, lk=lk, pq=pq, oq=oq, pk=pk, ok=ok, qbar=qbar, kbar=kbar,
                vbar=vbar, ratio=r, mask=mask, O=O, LSE=LSE, scale=scale)


def full_attention(q, k, v, scale):
    """Dense softmax attention, o = sum_j e^{s_j} v_j / sum_j e^{s_j} (FrontierCS
    blog, the one-query example's formula)."""
    q = np.asarray(q, F64)
    L = scale * (q @ np.asarray(k, F64).T)
    L -= L.max(axis=1, keepdims=True)
    w = np.exp(L)
    return (w @ np.asarray(v, F64)) / w.sum(axis=1, keepdims=True)
