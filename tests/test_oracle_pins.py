"""Pins of the fp64 oracle to facts that do not come from the oracle itself:
values the pages print, closed forms, library special cases, invariants and
brute force on tiny inputs.  CPU only."""
import json
import os
import warnings

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as orc
from synth.gen import WORKLOADS, head_inputs, scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa64(q, k, v, scale):
    """Library dense attention in fp64 on the CPU (torch)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)[0, 0].numpy()


def small_head(seed=0, N=192, D=16, comps=6, Cq=5, Ck=9, sigma=0.3):
    w = scaled(WORKLOADS["tiny"], N=N, D=D, comps=comps, Cq=Cq, Ck=Ck, seed=seed, sigma=sigma)
    return head_inputs(w, 0)


# ---------------------------------------------------------------- the pages' worked example
def toy():
    with open(os.path.join(GOLDEN, "toy_example.json")) as f:
        g = json.load(f)
    s = g["setup"]
    K = np.array(s["keys"], dtype=np.float64)[:, None]
    V = np.array(g["values_fixture"]["values"], dtype=np.float64)[:, None]
    q = np.array([s["q"]], dtype=np.float64)
    lab = np.array(s["key_cluster"])
    return g, q, K, V, lab


def lse_of(q, K, V, lab, mask_row, members=None):
    """Total (estimated) weight exp(LSE) when attending only to the clusters in ``members``."""
    keep = np.arange(K.shape[0]) if members is None else np.flatnonzero(np.isin(lab, members))
    Ks, Vs, ls = K[keep], V[keep], lab[keep]
    C = int(lab.max()) + 1
    perm, off = orc.permute(ls, C)
    kbar = orc.means(Ks, perm, off)
    vbar = orc.means(Vs, perm, off)
    _, lse = orc.attend_rows(q, Ks, Vs, perm, off, kbar, vbar, np.asarray(mask_row), 1.0)
    return float(np.exp(lse[0]))


def test_toy_weights_and_estimates_match_printed_values():
    g, q, K, V, lab = toy()
    p, tol = g["printed"], g["printed_abs_tolerance"]
    wA = lse_of(q, K, V, lab, [1, 0], members=[0])
    wB = lse_of(q, K, V, lab, [0, 1], members=[1])
    tot = lse_of(q, K, V, lab, [1, 1])
    estA = lse_of(q, K, V, lab, [0, 0], members=[0])
    estB = lse_of(q, K, V, lab, [0, 0], members=[1])
    assert abs(wA - p["weight_A"]) < tol and abs(wB - p["weight_B"]) < tol
    assert abs(tot - p["weight_total"]) < tol
    assert abs(estA - p["estimate_A"]) < tol and abs(estB - p["estimate_B"]) < tol
    assert abs((wB - estB) - p["shortfall_B"]) < tol
    # closed forms of the same example: 2e, 1 + e^2, and n e^{s_bar} = 2e for both estimates
    e = np.e
    assert wA == pytest.approx(2 * e, rel=1e-14) and wB == pytest.approx(1 + e * e, rel=1e-14)
    assert estA == pytest.approx(2 * e, rel=1e-14) and estB == pytest.approx(2 * e, rel=1e-14)


def test_toy_error_aware_choice_makes_query_exact():
    g, q, K, V, lab = toy()
    perm, off = orc.permute(lab, 2)
    kbar, vbar = orc.means(K, perm, off), orc.means(V, perm, off)
    q_off = np.array([0, 1])
    # room to compute one cluster of the two: a budget of 2 of the 4 keys
    r, mask = orc.route(q, q_off, K[perm], V[perm], kbar, vbar, off, 1.0, 0.5)
    assert g["printed"]["choice_with_room_for_one_cluster"] == "B"
    assert mask.tolist() == [[0, 1]]
    assert r[0, 0] == 0.0 and r[0, 1] > 0.0
    O, _ = orc.attend(q, K, V, np.array([0]), q_off, perm, off, kbar, vbar, mask, 1.0)
    assert g["printed"]["output_after_error_aware_choice"] == "exact"
    np.testing.assert_allclose(O, sdpa64(q, K, V, 1.0), rtol=0, atol=1e-14)
    # the score-ranked alternative (compute A, estimate B) is not exact
    O2, _ = orc.attend(q, K, V, np.array([0]), q_off, perm, off, kbar, vbar, np.array([[1, 0]], np.uint8), 1.0)
    assert abs(O2[0, 0] - O[0, 0]) > 1e-2


# ---------------------------------------------------------------- P1: rho = 1 is full attention
@pytest.mark.parametrize("seed", [0, 1])
def test_density_one_equals_full_attention(seed):
    h = small_head(seed)
    out = orc.layer(h["q"], h["k"], h["v"], h["cq0"], h["ck0"], iters=3, density=1.0)
    assert out["mask"][np.diff(out["oq"]) > 0].sum() == ((np.diff(out["oq"]) > 0).sum() * (np.diff(out["ok"]) > 0).sum())
    ref = sdpa64(h["q"], h["k"], h["v"], out["scale"])
    np.testing.assert_allclose(out["O"], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.full_attention(h["q"], h["k"], h["v"], out["scale"]), ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P2: singleton clusters
@pytest.mark.parametrize("density", [0.1, 0.3])
def test_singleton_key_clusters_make_compensation_exact(density):
    h = small_head(2, N=96)
    q, k, v = h["q"], h["k"], h["v"]
    out = orc.layer(q, k, v, h["cq0"], k.copy(), iters=2, density=density)
    assert (np.diff(out["ok"]) == 1).all()
    assert out["mask"].sum(axis=1).max() < k.shape[0]       # blocks really are skipped
    np.testing.assert_allclose(out["O"], sdpa64(q, k, v, out["scale"]), rtol=0, atol=1e-12)
    # every probe error vanishes: one key per cluster equals its centroid
    assert np.abs(out["ratio"]).max() == 0.0


# ---------------------------------------------------------------- P3: permutation equivariance
def test_token_permutation_equivariance():
    h = small_head(3)
    q, k, v = h["q"], h["k"], h["v"]
    a = orc.layer(q, k, v, h["cq0"], h["ck0"], iters=4, density=0.3)
    s = np.random.default_rng(7).permutation(q.shape[0])
    b = orc.layer(q[s], k[s], v[s], h["cq0"], h["ck0"], iters=4, density=0.3)
    np.testing.assert_array_equal(b["lq"], a["lq"][s])
    np.testing.assert_array_equal(b["mask"], a["mask"])
    np.testing.assert_allclose(b["O"], a["O"][s], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P4 extras: hand-worked small cases
def test_permute_hand_example():
    perm, off = orc.permute(np.array([2, 0, 2, 1, 0]), 4)
    assert perm.tolist() == [1, 4, 3, 0, 2]
    assert off.tolist() == [0, 2, 3, 5, 5]


def test_means_hand_example_and_empty_cluster():
    X = np.array([[1.0, 10.0], [2.0, 20.0], [3.0, 30.0], [4.0, 40.0]])
    perm, off = orc.permute(np.array([0, 2, 0, 2]), 3)
    m = orc.means(X, perm, off)
    assert m.tolist() == [[2.0, 20.0], [0.0, 0.0], [3.0, 30.0]]


def test_greedy_select_hand_example():
    sizes = np.array([3, 1, 4, 0, 2])
    r = np.array([0.5, 0.9, 0.5, 0.0, 0.1], dtype=np.float32)
    # budget 0.5 * 10 = 5 keys: order 1 (0.9), 0 and 2 (tie at 0.5, lower index first), 4;
    # taken 0 -> take 1 (1 key), 1 -> take 0 (4), 4 -> take 2 (8), 8 >= 5 stop
    assert orc.select_row(r, sizes, orc.budget_keys(0.5, 10)).tolist() == [1, 1, 1, 0, 0]
    # a budget of exactly 1 key takes only the top cluster
    assert orc.select_row(r, sizes, 1.0).tolist() == [0, 1, 0, 0, 0]
    # density 1 takes every non-empty cluster, never the empty one
    assert orc.select_row(r, sizes, 10.0).tolist() == [1, 1, 1, 0, 1]


# ---------------------------------------------------------------- P5: linearity and Jensen
def test_centroid_score_is_mean_score_and_never_overestimates():
    h = small_head(4, N=256, D=32)
    q, k, v = h["q"], h["k"], h["v"]
    ck, lk = orc.lloyd(k, h["ck0"], 3)
    perm, off = orc.permute(lk, ck.shape[0])
    kbar = orc.means(k, perm, off)
    sc = 1 / np.sqrt(32)
    for j in range(kbar.shape[0]):
        idx = perm[off[j]:off[j + 1]]
        if idx.size == 0:
            continue
        s = sc * (np.asarray(q, np.float64) @ np.asarray(k, np.float64)[idx].T)
        sbar = sc * (np.asarray(q, np.float64) @ kbar[j])
        np.testing.assert_allclose(sbar, s.mean(axis=1), rtol=0, atol=1e-12)
        assert (idx.size * np.exp(sbar) <= np.exp(s).sum(axis=1) * (1 + 1e-12)).all()


# ---------------------------------------------------------------- P6: Lloyd
def test_lloyd_matches_scipy_kmeans2_and_invariants():
    from scipy.cluster.vq import kmeans2
    h = small_head(5, N=600, D=16, comps=8, Ck=12)
    X = np.asarray(h["k"], np.float64)
    for T in (1, 2, 5):
        C, lab = orc.lloyd(X, h["ck0"], T)
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            Cs, labs = kmeans2(X, np.asarray(h["ck0"], np.float64), iter=T, minit="matrix")
        np.testing.assert_array_equal(lab, labs)
        np.testing.assert_allclose(C, Cs, rtol=0, atol=1e-12)
    prev = np.inf
    C = np.asarray(h["ck0"], np.float64)
    for _ in range(6):
        C, lab = orc.lloyd(X, C, 1)
        cur = orc.inertia(X, C, lab)
        assert cur <= prev * (1 + 1e-12)
        prev = cur
    perm, off = orc.permute(lab, C.shape[0])
    assert sorted(perm.tolist()) == list(range(X.shape[0]))
    assert (np.diff(lab[perm]) >= 0).all() and off[-1] == X.shape[0]
    for c in range(C.shape[0]):
        seg = perm[off[c]:off[c + 1]]
        assert (np.diff(seg) > 0).all()


def test_lloyd_empty_cluster_keeps_centroid():
    X = np.array([[0.0], [0.1], [10.0]])
    C0 = np.array([[0.0], [10.0], [100.0]])
    C, lab = orc.lloyd(X, C0, 1)
    assert lab.tolist() == [0, 0, 1]
    np.testing.assert_allclose(C, [[0.05], [10.0], [100.0]], rtol=0, atol=1e-15)


def test_assign_ties_go_to_lowest_index():
    X = np.array([[1.0, 0.0]])
    C = np.array([[0.0, 0.0], [2.0, 0.0], [1.0, 1.0]])
    assert orc.assign(X, C).tolist() == [0]


# ---------------------------------------------------------------- P7: brute force
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attend_matches_bruteforce(seed):
    h = small_head(seed, N=128, D=8, comps=5, Cq=4, Ck=7)
    q, k, v = (np.asarray(h[x], np.float64) for x in ("q", "k", "v"))
    _, lq = orc.lloyd(q, h["cq0"], 2)
    _, lk = orc.lloyd(k, h["ck0"], 2)
    pq, oq = orc.permute(lq, 4)
    pk, ok = orc.permute(lk, 7)
    kbar, vbar = orc.means(k, pk, ok), orc.means(v, pk, ok)
    mask = (np.random.default_rng(seed).random((4, 7)) < 0.4).astype(np.uint8)
    sc = 1 / np.sqrt(8)
    O, _ = orc.attend(q, k, v, pq, oq, pk, ok, kbar, vbar, mask, sc)
    Ob = orc.attend_bruteforce(q, k, v, lq, lk, kbar, vbar, mask, sc)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P8: routing invariants
def test_routing_density_bounds_and_nesting():
    h = small_head(6, N=512, D=16, comps=10, Cq=6, Ck=20)
    q, k, v = h["q"], h["k"], h["v"]
    cq, lq = orc.lloyd(q, h["cq0"], 3)
    ck, lk = orc.lloyd(k, h["ck0"], 3)
    pq, oq = orc.permute(lq, 6)
    pk, ok = orc.permute(lk, 20)
    qbar, kbar, vbar = orc.means(q, pq, oq), orc.means(k, pk, ok), orc.means(v, pk, ok)
    sizes = np.diff(ok)
    N = q.shape[0]
    prev = None
    for rho in (0.05, 0.1, 0.25, 0.5, 0.9, 1.0):
        r, mask = orc.route(qbar, oq, k[pk], v[pk], kbar, vbar, ok, 1 / 4.0, rho)
        for i in range(6):
            keys = (mask[i].astype(int) * sizes).sum()
            budget = float(np.float32(rho)) * N
            assert budget <= keys < budget + sizes.max()
            sel, uns = r[i][mask[i] == 1], r[i][(mask[i] == 0) & (sizes > 0)]
            if uns.size:
                assert sel.min() >= uns.max()
        if prev is not None:
            assert (mask >= prev).all()
        prev = mask
    assert (prev[:, sizes > 0] == 1).all() and (prev[:, sizes == 0] == 0).all()


# ---------------------------------------------------------------- P9: error sanity and closed forms
def test_probe_error_closed_forms():
    rng = np.random.default_rng(11)
    D, sc = 6, 0.5
    qbar = rng.standard_normal((3, D))
    # cluster 0: identical keys, spread values -> e = a^2 * sum_k ||v_bar - v_k||^2 = a^2 * n * sum_d var_d
    # cluster 1: spread keys, identical values -> e = ||v_bar||^2 * sum_k (a - b_k)^2
    # cluster 2: identical keys and values -> e = 0
    k0 = np.repeat(rng.standard_normal((1, D)), 5, axis=0)
    v0 = rng.standard_normal((5, D))
    k1 = rng.standard_normal((4, D))
    v1 = np.repeat(rng.standard_normal((1, D)), 4, axis=0)
    k2 = np.repeat(rng.standard_normal((1, D)), 3, axis=0)
    v2 = np.repeat(rng.standard_normal((1, D)), 3, axis=0)
    Kp, Vp = np.vstack([k0, k1, k2]), np.vstack([v0, v1, v2])
    off = np.array([0, 5, 9, 12])
    perm = np.arange(12)
    kbar, vbar = orc.means(Kp, perm, off), orc.means(Vp, perm, off)
    e, M = orc.probe_errors(qbar, Kp, Vp, kbar, vbar, off, sc)
    s_all = sc * qbar @ Kp.T
    np.testing.assert_allclose(M, s_all.max(axis=1), rtol=1e-15)
    a0 = np.exp(sc * qbar @ kbar[0] - M)
    np.testing.assert_allclose(e[:, 0], a0 ** 2 * 5 * np.var(v0, axis=0).sum(), rtol=1e-12)
    a1 = np.exp(sc * qbar @ kbar[1] - M)
    b1 = np.exp(s_all[:, 5:9] - M[:, None])
    np.testing.assert_allclose(e[:, 1], np.dot(v1[0], v1[0]) * ((a1[:, None] - b1) ** 2).sum(1), rtol=1e-12)
    assert np.abs(e[:, 2]).max() < 1e-28
    assert (e >= 0).all()


def test_ratio_divides_by_block_pairs_and_zero_for_empty():
    e = np.array([[6.0, 0.0, 8.0], [1.0, 1.0, 1.0]])
    r = orc.ratios(e, [2, 0], [3, 0, 4])
    assert r.dtype == np.float32
    assert r.tolist() == [[1.0, 0.0, 1.0], [0.0, 0.0, 0.0]]


# ---------------------------------------------------------------- identical members: estimate is exact
@pytest.mark.parametrize("density", [0.05, 0.3])
def test_clusters_of_identical_members_make_compensation_exact(density):
    """Each key cluster holds 3 copies of one (key, value): n_j e^{q.k_bar} v_bar equals the
    block's exact contribution, so any mask gives full attention.  Fails if ln n_j is dropped
    or the wrong value mean is used."""
    h = small_head(8, N=60, D=8)
    k = np.repeat(h["k"][:20], 3, axis=0)
    v = np.repeat(h["v"][:20], 3, axis=0)
    q = h["q"]
    out = orc.layer(q, k, v, h["cq0"], h["k"][:20].copy(), iters=2, density=density)
    assert (np.diff(out["ok"]) == 3).all()
    assert out["mask"].sum(axis=1).max() < 20
    np.testing.assert_allclose(out["O"], sdpa64(q, k, v, out["scale"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- variance-corrected compensation
def lse_corrected(q, K, V, lab, mask_row, members, strength):
    keep = np.flatnonzero(np.isin(lab, members))
    Ks, Vs, ls = K[keep], V[keep], lab[keep]
    C = int(lab.max()) + 1
    perm, off = orc.permute(ls, C)
    kbar, vbar = orc.means(Ks, perm, off), orc.means(Vs, perm, off)
    kvar = orc.variances(Ks, perm, off)
    _, lse = orc.attend_rows(q, Ks, Vs, perm, off, kbar, vbar, np.asarray(mask_row), 1.0, kvar, strength)
    return float(np.exp(lse[0]))


def test_toy_variance_corrected_estimate_matches_printed_value():
    """FrontierCS blog, variance-correction paragraph: B's scores 0 and 2 have
    variance 1 and the corrected estimate is about 9.0 (closed form 2 e^{1.5})."""
    g, q, K, V, lab = toy()
    p, tol = g["printed"], g["printed_abs_tolerance"]
    perm, off = orc.permute(lab, 2)
    var = orc.variances(K, perm, off)
    assert var[1, 0] == 1.0 and var[0, 0] == 0.0
    est = lse_corrected(q, K, V, lab, [0, 0], [1], 1.0)
    assert abs(est - p["variance_corrected_estimate_B"]) < tol
    assert est == pytest.approx(2.0 * np.exp(1.5), rel=1e-14)
    # still closer to the true 8.4 (1 + e^2) than the plain 5.4, and above it
    assert abs(est - (1 + np.e ** 2)) < abs(2 * np.e - (1 + np.e ** 2))
    # strength scales the raised score: strength 1/2 gives 2 e^{1 + 1/4}
    assert lse_corrected(q, K, V, lab, [0, 0], [1], 0.5) == pytest.approx(2.0 * np.exp(1.25), rel=1e-14)


def test_variance_hand_example_and_empty_cluster():
    X = np.array([[0.0, 1.0], [2.0, 1.0], [5.0, -3.0], [1.0, 7.0], [3.0, 9.0]])
    lab = np.array([0, 0, 2, 0, 2])
    perm, off = orc.permute(lab, 3)
    var = orc.variances(X, perm, off)
    # cluster 0: x = 0, 2, 1 (mean 1, deviations -1, 1, 0) and 1, 1, 7 (mean 3, deviations -2, -2, 4)
    np.testing.assert_allclose(var[0], [2.0 / 3.0, 24.0 / 3.0], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(var[1], [0.0, 0.0])             # empty
    np.testing.assert_allclose(var[2], [1.0, 36.0], rtol=0, atol=1e-15)  # 5, 3 and -3, 9


def test_variance_term_in_one_dimension_is_the_score_variance():
    """d = 1: sigma^2 = scale^2 q^2 Var(k) is exactly the variance of the
    query's scores over the cluster, so the corrected pseudo-score of every
    skipped cluster is ln n + mean score + strength * Var(scores) / 2."""
    rng = np.random.default_rng(3)
    K = rng.normal(size=(12, 1))
    V = rng.normal(size=(12, 1))
    lab = np.repeat(np.arange(3), 4)
    q = rng.normal(size=(1, 1))
    scale = 0.7
    perm, off = orc.permute(lab, 3)
    kbar, vbar, kvar = orc.means(K, perm, off), orc.means(V, perm, off), orc.variances(K, perm, off)
    mask = np.array([1, 0, 0], np.uint8)
    for strength in (0.5, 1.0, 1.5):
        _, lse = orc.attend_rows(q, K, V, perm, off, kbar, vbar, mask, scale, kvar, strength)
        total = sum(np.exp(scale * q[0, 0] * K[u, 0]) for u in range(4))
        for j in (1, 2):
            s = scale * q[0, 0] * K[4 * j:4 * j + 4, 0]
            total += 4 * np.exp(s.mean() + strength * 0.5 * s.var())
        assert float(lse[0]) == pytest.approx(np.log(total), rel=1e-13)


def test_variance_correction_is_second_order_and_neutral_at_zero():
    """strength 0 is the plain method bit for bit; clusters of identical keys
    have no variance; for a tight cluster the corrected weight is much closer
    to the exact sum of weights than the plain n e^{s_bar} (second order)."""
    x = small_head(seed=5)
    q, k, v = x["q"], x["k"], x["v"]
    D = q.shape[1]
    sc = 1.0 / np.sqrt(D)
    _, lk = orc.lloyd(k, x["ck0"], 5)
    pk, ok = orc.permute(lk, x["ck0"].shape[0])
    kbar, vbar, kvar = orc.means(k, pk, ok), orc.means(v, pk, ok), orc.variances(k, pk, ok)
    mask = np.zeros((1, kbar.shape[0]), np.uint8)
    plain, lse0 = orc.attend_rows(q[:8], k, v, pk, ok, kbar, vbar, mask[0], sc)
    zero, lsez = orc.attend_rows(q[:8], k, v, pk, ok, kbar, vbar, mask[0], sc, kvar, 0.0)
    np.testing.assert_array_equal(plain, zero)
    np.testing.assert_array_equal(lse0, lsez)
    # identical keys: variance 0, corrected == plain
    kk = np.repeat(k[:3], 4, axis=0)
    lab = np.repeat(np.arange(3), 4)
    p2, o2 = orc.permute(lab, 3)
    kv = orc.variances(kk, p2, o2)
    assert not kv.any()
    # second order: per cluster, exact vs plain vs corrected weights for each query
    worse = 0
    for j in range(kbar.shape[0]):
        lo, hi = int(ok[j]), int(ok[j + 1])
        if hi - lo < 2:
            continue
        s = sc * (q[:8] @ k[pk[lo:hi]].T)
        exact = np.exp(s).sum(axis=1)
        sbar = sc * (q[:8] @ kbar[j])
        plain_w = (hi - lo) * np.exp(sbar)
        corr_w = (hi - lo) * np.exp(sbar + 0.5 * sc * sc * ((q[:8] ** 2) @ kvar[j]))
        assert np.all(plain_w <= exact * (1 + 1e-12))          # Jensen: the plain guess is low
        worse += int(np.sum(np.abs(corr_w - exact) > np.abs(plain_w - exact)))
    assert worse == 0


# ---------------------------------------------------------------- top-p budget and the SVG2 router
def test_toy_topp_shares_tie_and_the_two_routers_split():
    """Blog toy: both centroids score 1 and both clusters hold two keys, so the
    estimated weights tie; with room for one cluster the score-ranked router
    keeps A (tie to the lower index) while the error-ranked one keeps B."""
    g, q, K, V, lab = toy()
    assert g["printed"]["estimated_weight_ranking"] == "tie"
    perm, off = orc.permute(lab, 2)
    kbar, vbar = orc.means(K, perm, off), orc.means(V, perm, off)
    sizes = np.diff(off)
    P = orc.topp_probs(q, kbar, sizes, 1.0)
    assert P.tolist() == [[0.5, 0.5]]
    q_off = np.array([0, 1])
    # p = 0.5: the first cluster's share already reaches p, so one cluster's keys
    _, _, bud, m_score = orc.route_topp(q, q_off, K[perm], V[perm], kbar, vbar, off, 1.0, 0.5, error_ranked=False)
    assert m_score.tolist() == [[1, 0]] and bud.tolist() == [2]
    _, r, bud2, m_err = orc.route_topp(q, q_off, K[perm], V[perm], kbar, vbar, off, 1.0, 0.5, error_ranked=True)
    assert bud2.tolist() == [2]
    assert {"A": [[1, 0]], "B": [[0, 1]]}[g["printed"]["choice_with_room_for_one_cluster"]] == m_err.tolist()
    # p just above one cluster's share needs both
    _, _, bud3, m3 = orc.route_topp(q, q_off, K[perm], V[perm], kbar, vbar, off, 1.0, 0.6, error_ranked=False)
    assert m3.tolist() == [[1, 1]] and bud3.tolist() == [4]


def onehot_mass(qbar, K, lab, C, scale):
    """Dense attention mass per cluster from the library: attend with values
    that are the one-hot cluster indicator."""
    Vh = np.eye(C)[lab]
    return sdpa64(qbar, K, Vh, scale)


def test_topp_probs_equal_dense_mass_for_singleton_and_identical_clusters():
    """P' estimates each key cluster's share of the attention mass.  It is exact
    when every key of a cluster equals the centroid: singleton clusters give the
    dense softmax probabilities, and clusters of identical keys their summed
    probability (the |K_j| factor).  Checked against torch's fp64 attention."""
    rng = np.random.default_rng(21)
    D, scale = 8, 1 / np.sqrt(8)
    qbar = rng.standard_normal((4, D))
    # singletons
    K = rng.standard_normal((12, D))
    lab = np.arange(12)
    perm, off = orc.permute(lab, 12)
    P = orc.topp_probs(qbar, orc.means(K, perm, off), np.diff(off), scale)
    np.testing.assert_allclose(P, onehot_mass(qbar, K, lab, 12, scale), rtol=1e-6, atol=1e-9)
    # identical members, unequal sizes, one empty cluster
    cent = rng.standard_normal((5, D))
    lab = np.array([0, 0, 0, 1, 3, 3, 4, 4, 4, 4, 4, 0])
    K = cent[lab]
    perm, off = orc.permute(lab, 5)
    sizes = np.diff(off)
    assert sizes[2] == 0
    P = orc.topp_probs(qbar, orc.means(K, perm, off), sizes, scale)
    np.testing.assert_allclose(P, onehot_mass(qbar, K, lab, 5, scale), rtol=1e-6, atol=1e-9)
    assert (P[:, 2] == 0).all()
    np.testing.assert_allclose(P.astype(np.float64).sum(axis=1), 1.0, rtol=0, atol=1e-6)


def test_topp_probs_survive_large_scores():
    """Scores far beyond exp's range still give finite shares (the row maximum
    is taken over non-empty clusters only)."""
    qbar = np.array([[1.0]])
    kbar = np.array([[900.0], [899.0], [0.0]])
    P = orc.topp_probs(qbar, kbar, np.array([1, 2, 0]), 1.0)
    e = np.exp(-1.0)
    np.testing.assert_allclose(P[0], [1 / (1 + 2 * e), 2 * e / (1 + 2 * e), 0.0], rtol=1e-6)


def brute_topp_size(P_row, sizes, p):
    """Fewest non-empty clusters whose shares sum to at least p (enumeration)."""
    import itertools
    live = [j for j in range(len(sizes)) if sizes[j] > 0]
    for k in range(1, len(live) + 1):
        if max(sum(float(P_row[j]) for j in c) for c in itertools.combinations(live, k)) >= p:
            return k
    return len(live)


@pytest.mark.parametrize("seed", range(6))
def test_topp_select_is_the_smallest_set_reaching_p_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    C = 7
    sizes = rng.integers(0, 4, C)
    sizes[rng.integers(0, C)] = 2
    kbar = rng.standard_normal((C, 3)) * 2
    qbar = rng.standard_normal((1, 3))
    P = orc.topp_probs(qbar, kbar, sizes, 1.0)[0]
    prev = np.zeros(C, np.uint8)
    for p in (0.05, 0.3, 0.5, 0.77, 0.9, 0.999, 1.0):
        sel = orc.topp_select_row(P, sizes, p)
        assert (sel[sizes == 0] == 0).all()
        if p < 1.0:
            assert sel.sum() == brute_topp_size(P, sizes, float(np.float32(p)))
            assert sum(float(P[j]) for j in np.flatnonzero(sel)) >= float(np.float32(p))
        else:
            assert (sel[sizes > 0] == 1).all()
        # the selection is a prefix of the share order: nothing left out beats what is in
        live_out = (sel == 0) & (sizes > 0)
        if live_out.any() and sel.any():
            assert P[sel == 1].min() >= P[live_out].max()
        assert (sel >= prev).all()          # nested in p
        prev = sel


def test_topp_hand_example():
    sizes = np.array([3, 1, 0, 4, 2])
    P = np.array([0.25, 0.5, 0.0, 0.125, 0.125], dtype=np.float32)
    # order 1 (0.5), 0 (0.25), 3 and 4 (tie at 0.125, lower index first)
    assert orc.topp_select_row(P, sizes, 0.5).tolist() == [0, 1, 0, 0, 0]
    assert orc.topp_select_row(P, sizes, 0.6).tolist() == [1, 1, 0, 0, 0]
    assert orc.topp_select_row(P, sizes, 0.8).tolist() == [1, 1, 0, 1, 0]
    assert orc.topp_select_row(P, sizes, 1.0).tolist() == [1, 1, 0, 1, 1]
    m = orc.topp_select(P[None].repeat(2, 0), np.array([5, 0]), sizes, 0.8)
    assert m.tolist() == [[1, 1, 0, 1, 0], [0, 0, 0, 0, 0]]
    assert orc.topp_budgets(m, sizes).tolist() == [8, 0]


def test_error_ranked_budget_reduces_to_top_p_when_rankings_agree():
    """Spending the top-p keys in the top-p order selects the top-p set again;
    with one common budget it is the density router."""
    h = small_head(9, N=384, D=16, comps=8, Cq=6, Ck=16)
    q, k, v = h["q"], h["k"], h["v"]
    _, lq = orc.lloyd(q, h["cq0"], 3)
    _, lk = orc.lloyd(k, h["ck0"], 3)
    pq, oq = orc.permute(lq, 6)
    pk, ok = orc.permute(lk, 16)
    qbar, kbar = orc.means(q, pq, oq), orc.means(k, pk, ok)
    qs, ks = np.diff(oq), np.diff(ok)
    P = orc.topp_probs(qbar, kbar, ks, 0.25)
    for p in (0.3, 0.6, 0.9):
        tm = orc.topp_select(P, qs, ks, p)
        assert (orc.select_budgets(P, qs, ks, orc.topp_budgets(tm, ks)) == tm).all()
    r = np.random.default_rng(3).random(P.shape).astype(np.float32)
    same = np.full(6, float(np.float32(0.3)) * 384)
    assert (orc.select_budgets(r, qs, ks, same) == orc.select(r, qs, ks, 0.3, 384)).all()


def test_route_topp_budgets_and_bounds():
    h = small_head(10, N=512, D=16, comps=10, Cq=6, Ck=20)
    q, k, v = h["q"], h["k"], h["v"]
    _, lq = orc.lloyd(q, h["cq0"], 3)
    _, lk = orc.lloyd(k, h["ck0"], 3)
    pq, oq = orc.permute(lq, 6)
    pk, ok = orc.permute(lk, 20)
    qbar, kbar, vbar = orc.means(q, pq, oq), orc.means(k, pk, ok), orc.means(v, pk, ok)
    ks = np.diff(ok)
    prev = None
    for p in (0.5, 0.8, 0.9, 1.0):
        P, r, bud, m = orc.route_topp(qbar, oq, k[pk], v[pk], kbar, vbar, ok, 0.25, p)
        Ps, _, bud_s, ms = orc.route_topp(qbar, oq, k[pk], v[pk], kbar, vbar, ok, 0.25, p, error_ranked=False)
        assert (Ps == P).all() and (bud_s == bud).all()
        assert (bud == (ms.astype(np.int64) * ks).sum(axis=1)).all()
        for i in range(6):
            keys = int((m[i].astype(np.int64) * ks).sum())
            assert bud[i] <= keys < bud[i] + ks.max()
            sel, uns = r[i][m[i] == 1], r[i][(m[i] == 0) & (ks > 0)]
            if uns.size:
                assert sel.min() >= uns.max()
        if prev is not None:
            assert (bud >= prev).all()
        prev = bud
    assert (prev == 512).all()


# ---------------------------------------------------------------- k-means++ seeding
def test_kmeanspp_hand_example():
    """Integer points, so every distance and weight is exact: (0,0), (1,0),
    (0,2), (3,0).  Word 0 picks token 0; D^2 = (0, 1, 4, 9) with cumulative
    (0, 1, 5, 14); a word of 2^62 targets 14/4 = 3.5, which falls in token 2's
    range [1, 5); then D^2 = (0, 1, 0, 9), cumulative (0, 1, 1, 10), and 2^63
    targets 5, in token 3's range [1, 10)."""
    X = np.array([[0, 0], [1, 0], [0, 2], [3, 0]], float)
    seeds, idx = orc.kmeanspp(X, np.array([0, 2**62, 2**63], dtype=np.uint64), 3)
    assert idx.tolist() == [0, 2, 3]
    np.testing.assert_array_equal(seeds, X[[0, 2, 3]])
    # the edges of the ranges: 2^60 targets 0.875 (token 1), the largest word
    # targets just below 14 (token 3); the first seed takes floor(word * N / 2^64)
    assert orc.kmeanspp(X, np.array([0, 2**60], dtype=np.uint64), 2)[1].tolist() == [0, 1]
    assert orc.kmeanspp(X, np.array([0, 2**64 - 1], dtype=np.uint64), 2)[1].tolist() == [0, 3]
    assert orc.kmeanspp(X, np.array([3 * 2**62, 0], dtype=np.uint64), 2)[1].tolist() == [3, 0]


def test_kmeanspp_distance_order_and_scale():
    rng = np.random.default_rng(31)
    X = rng.standard_normal((300, 24))
    c = X[17]
    from scipy.spatial.distance import cdist
    d2 = orc.sqdist_seq(X, c)
    np.testing.assert_allclose(d2, cdist(X, c[None], "sqeuclidean")[:, 0], rtol=1e-13, atol=0)
    k = orc.pp_scale(d2)
    assert len(d2) * d2.max() * 2.0**k < 2.0**62 <= 2 * len(d2) * d2.max() * 2.0**k
    w = orc.pp_weights(d2, k)
    assert int(np.sum(w, dtype=np.uint64)) < 2**62 and w[17] == 0


@pytest.mark.parametrize("seed", range(4))
def test_kmeanspp_picks_one_point_per_separated_blob(seed):
    """Eight tight blobs 100 apart: D^2 sampling lands in a new blob at every
    step with probability > 1 - 1e-4, whereas uniform picks would repeat a blob
    with probability 1 - 8!/8^8 > 0.99."""
    rng = np.random.default_rng(200 + seed)
    centers = 100.0 * np.eye(8)
    X = np.concatenate([ctr + 0.01 * rng.standard_normal((20, 8)) for ctr in centers])
    words = rng.integers(0, np.iinfo(np.uint64).max, size=8, dtype=np.uint64, endpoint=True)
    _, idx = orc.kmeanspp(X, words, 8)
    assert sorted((idx // 20).tolist()) == list(range(8))


def test_kmeanspp_distinct_rows_are_each_taken_once_and_duplicates_fall_back():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((12, 4))
    words = rng.integers(0, np.iinfo(np.uint64).max, size=12, dtype=np.uint64, endpoint=True)
    assert sorted(orc.kmeanspp(X, words, 12)[1].tolist()) == list(range(12))
    # three distinct rows, four copies each: the first three seeds cover them,
    # then every distance is 0 and the draw is uniform: floor(word * N / 2^64)
    Y = np.repeat(rng.standard_normal((3, 4)), 4, axis=0)
    words = np.array([0, 2**63, 2**62, 2**63 + 5, 2**62 * 3], dtype=np.uint64)
    seeds, idx = orc.kmeanspp(Y, words, 5)
    assert sorted({int(i) // 4 for i in idx[:3]}) == [0, 1, 2]
    assert idx[3] == ((2**63 + 5) * 12) >> 64 and idx[4] == (3 * 2**62 * 12) >> 64


def test_kmeanspp_second_seed_follows_the_d2_law():
    """Frequencies of the second seed over many words against D^2 / sum D^2
    (distances from scipy), within five binomial standard deviations."""
    from scipy.spatial.distance import cdist
    X = np.array([[0.0, 0.0], [1.0, 0.5], [2.0, -1.0], [0.3, 0.3], [-1.5, 2.0]])
    p = cdist(X, X[:1], "sqeuclidean")[:, 0]
    p = p / p.sum()
    rng = np.random.default_rng(8)
    n = 6000
    counts = np.zeros(5)
    for wd in rng.integers(0, np.iinfo(np.uint64).max, size=n, dtype=np.uint64, endpoint=True):
        counts[orc.kmeanspp(X, np.array([0, wd], dtype=np.uint64), 2)[1][1]] += 1
    assert counts[0] == 0
    assert np.all(np.abs(counts / n - p) <= 5 * np.sqrt(p * (1 - p) / n) + 1e-12)


# ---------------------------------------------------------------- e4m3 quantisation (FP8 variant)
def e4m3_value(code: int) -> float:
    """OCP e4m3fn from its definition: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent field 0 is subnormal; S.1111.111 is NaN; no infinities."""
    s, E, M = code >> 7, (code >> 3) & 15, code & 7
    if E == 15 and M == 7:
        return float("nan")
    v = (M / 8.0) * 2.0 ** -6 if E == 0 else (1 + M / 8.0) * 2.0 ** (E - 7)
    return -v if s else v


def test_e4m3_codes_follow_the_format_definition():
    codes = np.arange(256, dtype=np.uint8)
    dec = orc.dequantize_e4m3(codes, 0)
    ref = np.array([e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(dec[ok], ref[ok])
    assert np.nanmax(dec) == 448.0 and dec[1] == 2.0 ** -9
    # every finite value quantises to itself (scale 2^0 since the max is 448)
    fin = ref[ok]
    c, e = orc.quantize_e4m3(fin)
    assert e == 0 and np.array_equal(orc.dequantize_e4m3(c, e), fin)


def test_e4m3_rounding_is_nearest_even_with_exact_ties():
    # 1 + 1/16 lies halfway between 1 (mantissa 000) and 1.125 (001): even -> 1;
    # 1 + 3/16 between 1.125 (001) and 1.25 (010): even -> 1.25; the same in
    # the subnormal range: 3 * 2^-10 between 2^-9 (001) and 2^-8 (010) -> 2^-8
    x = np.array([448.0, 1.0625, 1.1875, 3 * 2.0 ** -10, -1.0625, 1.0625 + 2 ** -20], np.float32)
    c, e = orc.quantize_e4m3(x)
    assert e == 0
    np.testing.assert_array_equal(orc.dequantize_e4m3(c, e), [448.0, 1.0, 1.25, 2.0 ** -8, -1.0, 1.125])


def test_e4m3_scale_rule_and_error_bound():
    assert orc.e4m3_exponent(448.0) == 0 and orc.e4m3_exponent(448.0001) == 1
    assert orc.e4m3_exponent(224.0) == -1 and orc.e4m3_exponent(0.0) == 0
    rng = np.random.default_rng(3)
    for scale in (1e-3, 0.7, 5.0, 3e4):
        X = (rng.standard_normal((64, 32)) * scale).astype(np.float32)
        c, e = orc.quantize_e4m3(X)
        a = float(np.abs(X).max())
        assert 224.0 < a * 2.0 ** -e <= 448.0
        Y = orc.dequantize_e4m3(c, e)
        big = np.abs(X) >= 2.0 ** (e - 6)                 # normal range of the codes
        assert np.all(np.abs(Y[big] - X[big]) <= 2.0 ** -4 * np.abs(X[big]))
        assert np.all(np.abs(Y[~big] - X[~big]) <= 2.0 ** (e - 10))   # half a subnormal step
