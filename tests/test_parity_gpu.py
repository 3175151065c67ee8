"""GPU parity: every C-ABI call against the fp64 oracle on the same seeded
inputs, teacher-forced (the GPU gets the oracle's inputs to that stage),
at sizes that span several tiles and ragged tails; then end to end.

Tolerances.  Labels: equal except where the GPU's centroid is within
1e-5 * max(1, D) of the oracle's in squared distance.  Means: the rigorous
fp32 summation bound (n + 2) u max|x|.  Masks: bit-exact given the same
float32 ratios.  Attention output vs the fp64 oracle: bf16 inputs max-abs
<= 2e-2 and mean-abs <= 2e-3; fp32 inputs max-abs <= 1e-4 and mean-abs
<= 1e-5 (fp32 MFMA products, fp32 softmax, ~1e-6 relative).  Route ratios:
relative 2e-3 (see the design notes for the derivation)."""
import os

import numpy as np
import pytest
import torch

from oracle import svgear_oracle as orc
from synth.gen import WORKLOADS, layer_inputs, scaled
from tests.helpers import (check_labels_near_ties, check_ratio_masks, check_topp_masks, f32, first_divergence, host,
                           i32, mean_bound, oracle_from_labels, to_dev)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (dtype, B, H, N, D, comps, zipf, Cq, Ck)
    "f32-d64": ("f32", 1, 2, 2500, 64, 12, None, 13, 37),
    "bf16-d128": ("bf16", 1, 2, 5000, 128, 24, 1.1, 16, 53),
    "bf16-d64": ("bf16", 2, 1, 4500, 64, 24, 1.1, 11, 41),
    "f32-d128": ("f32", 1, 1, 3000, 128, 10, None, 9, 40),
}
ATOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-5)}


@pytest.fixture(scope="module")
def sv():
    import sparse_attention_video_amd as pkg
    pkg.load()
    assert torch.cuda.is_available()
    return pkg


def make(name, seed=11):
    dt, B, H, N, D, comps, zipf, Cq, Ck = CASES[name]
    w = scaled(WORKLOADS["tiny"], B=B, H=H, N=N, D=D, dtype=dt, comps=comps, zipf=zipf, Cq=Cq, Ck=Ck,
               seed=seed, density=0.3)
    return w, layer_inputs(w)


def stack(arrs):
    return np.stack(arrs)


def reshape4(a, w):
    return a.reshape(w.B, w.H, *a.shape[1:])


@pytest.fixture(scope="module")
def ref_cache():
    return {}


def oracle_layer(name, ref_cache, iters=3, density=0.3):
    key = (name, iters, density)
    if key not in ref_cache:
        w, x = make(name)
        sc = 1.0 / np.sqrt(w.D)
        outs = [orc.layer(x["q"][h], x["k"][h], x["v"][h], x["cq0"][h], x["ck0"][h], iters, density, sc)
                for h in range(w.B * w.H)]
        ref_cache[key] = (w, x, outs, sc)
    return ref_cache[key]


# ------------------------------------------------------------------ k-means
@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("which", ["q", "k"])
def test_kmeans_rounds_teacher_forced(sv, name, which):
    w, x = make(name)
    X = x[which]
    C = w.Cq if which == "q" else w.Ck
    Cs = x["cq0"] if which == "q" else x["ck0"]
    xd = to_dev(reshape4(X, w), w.dtype)
    for rnd in range(3):
        cent = f32(reshape4(Cs, w))
        lab, perm, off = sv.kmeans(xd, cent, 1)
        lab, perm, off, cent = (host(t).reshape(w.B * w.H, -1) for t in (lab, perm, off, cent))
        cent = cent.reshape(w.B * w.H, C, w.D)
        nxt = []
        for h in range(w.B * w.H):
            lo = orc.assign(X[h], Cs[h])
            nbad = check_labels_near_ties(X[h], Cs[h], lab[h], lo)
            if nbad == 0:
                po, oo = orc.permute(lo, C)
                np.testing.assert_array_equal(perm[h], po)
                np.testing.assert_array_equal(off[h], oo)
                c1 = orc.update(X[h], lo, Cs[h])
                bound = mean_bound(X[h], po, oo)
                err = np.abs(cent[h] - c1).max(axis=1)
                assert np.all(err <= bound + 1e-30), (err.max(), bound.max())
                empty = np.diff(oo) == 0
                np.testing.assert_array_equal(cent[h][empty], Cs[h][empty].astype(np.float32))
            nxt.append(orc.update(X[h], lo, Cs[h]).astype(np.float32))
        Cs = np.stack(nxt)


@pytest.mark.parametrize("name", list(CASES))
def test_kmeans_multi_round_matches_lloyd(sv, name):
    """Six rounds (three full updates, three incremental) against the oracle's
    Lloyd iterates.  Where the final labels differ, the first round that
    differs must differ only at near ties; in every case the centroids are
    the means of the labels the GPU returned (the oracle's when they agree)."""
    w, x = make(name)
    X, C0 = x["k"], x["ck0"]
    BH = w.B * w.H
    xd = to_dev(reshape4(X, w), w.dtype)

    def run(r):
        cent = f32(reshape4(C0, w))
        lab, _, _ = sv.kmeans(xd, cent, r)
        return host(lab).reshape(BH, -1), host(cent).reshape(BH, w.Ck, w.D)

    lab, cent = run(6)
    for h in range(BH):
        Co, lo = orc.lloyd(X[h], C0[h], 6)
        if (lab[h] == lo).all():
            po, oo = orc.permute(lo, w.Ck)
            assert (np.abs(cent[h] - Co).max(axis=1) <= mean_bound(X[h], po, oo) + 1e-6).all()
            continue
        r, n = first_divergence(lambda rr: run(rr)[0][h], X[h], C0[h], 6)
        assert r is not None, "final labels differ although every round agreed"
        print(f"{name} head {h}: labels first differ in round {r} at {n} near ties")
        po, oo = orc.permute(lab[h], w.Ck)
        full = np.diff(oo) > 0
        mu = orc.means(X[h], po, oo)
        assert (np.abs(cent[h] - mu).max(axis=1)[full] <= mean_bound(X[h], po, oo)[full] + 1e-6).all()


# (the last three: ~3 tokens per cluster, so that workgroups span 64 or more
# labels and take every centroid; ~8, around the 32-label limit of chunk 0;
# a ragged size at D = 64)
@pytest.mark.parametrize("D,C,N", [(128, 300, 12000), (64, 256, 9000), (128, 1024, 20000), (128, 1024, 3000),
                                   (128, 512, 4096), (64, 300, 2500)])
def test_kmeans_pruned_rounds_match_lloyd(sv, D, C, N):
    """From the fourth round on, bf16 k-means with a few hundred centroids or
    more assigns each workgroup's tokens only against the centroids that the
    triangle inequality leaves possible (the assignment step itself is
    unchanged: the nearest centroid, SVG2 summary, "Semantic-Aware
    Permutation via k-Means Clustering").  Eight rounds against the oracle's
    Lloyd iterates with the first-divergence near-tie rule, and the centroids
    as the means of the returned labels."""
    w = scaled(WORKLOADS["tiny"], B=1, H=1, N=N, D=D, dtype="bf16", comps=C // 2, zipf=1.1, Cq=16, Ck=C,
               seed=5, density=0.3)
    x = layer_inputs(w)
    X, C0 = x["k"][0], x["ck0"][0]
    xd = to_dev(X.reshape(1, 1, N, D), "bf16")

    def run(r):
        cent = f32(C0.reshape(1, 1, C, D))
        lab, _, _ = sv.kmeans(xd, cent, r)
        return host(lab).reshape(-1), host(cent).reshape(C, D)

    lab, cent = run(8)
    Co, lo = orc.lloyd(X, C0, 8)
    if (lab == lo).all():
        po, oo = orc.permute(lo, C)
        assert (np.abs(cent - Co).max(axis=1) <= mean_bound(X, po, oo) + 1e-6).all()
        return
    r, n = first_divergence(lambda rr: run(rr)[0], X, C0, 8)
    assert r is not None, "final labels differ although every round agreed"
    print(f"pruned k-means D={D} C={C}: labels first differ in round {r} at {n} near ties")
    po, oo = orc.permute(lab, C)
    full = np.diff(oo) > 0
    mu = orc.means(X, po, oo)
    assert (np.abs(cent - mu).max(axis=1)[full] <= mean_bound(X, po, oo)[full] + 1e-6).all()


def test_kmeans_empty_cluster_keeps_centroid(sv):
    w, x = make("bf16-d64")
    X = x["q"]
    C0 = x["cq0"].copy()
    C0[:, 3] = 1000.0          # far away: no member
    C0[:, 5] = C0[:, 4]        # duplicate of centroid 4: ties go to 4, so 5 is empty
    cent = f32(reshape4(C0, w))
    lab, perm, off = sv.kmeans(to_dev(reshape4(X, w), w.dtype), cent, 1)
    lab = host(lab).reshape(w.B * w.H, -1)
    off = host(off).reshape(w.B * w.H, -1)
    cent = host(cent).reshape(w.B * w.H, w.Cq, w.D)
    for h in range(w.B * w.H):
        lo = orc.assign(X[h], C0[h])
        assert check_labels_near_ties(X[h], C0[h], lab[h], lo) == 0
        assert off[h][4] == off[h][3] and off[h][6] == off[h][5]
        np.testing.assert_array_equal(cent[h][3], C0[h][3])
        np.testing.assert_array_equal(cent[h][5], C0[h][5])


@pytest.mark.parametrize("iters", [2, 5])
def test_kmeans_singletons_and_single_cluster(sv, iters):
    """C = N (every token its own cluster) and C = 1; with 5 rounds the last
    two run the incremental update with no token moving."""
    w, x = make("f32-d64")
    X = x["k"][:1, :300]
    for C0 in (X.copy(), X[:, :1].copy()):
        C = C0.shape[1]
        cent = f32(C0[:, None])
        lab, perm, off = sv.kmeans(f32(X[:, None]), cent, iters)
        Co, lo = orc.lloyd(X[0], C0[0], iters)
        np.testing.assert_array_equal(host(lab)[0, 0], lo)
        np.testing.assert_allclose(host(cent)[0, 0], Co, rtol=0, atol=1e-5)


@pytest.mark.parametrize("N,C", [(70, 3), (129, 5), (5, 2)])
def test_kmeans_tiny_ragged_many_rounds(sv, N, C):
    """Token counts that leave partial waves and workgroups, 8 rounds (five
    incremental), two heads: labels, perm and offsets as the oracle's Lloyd
    iterates, centroids within the fp32 mean bound."""
    rng = np.random.default_rng(N * 31 + C)
    X = np.concatenate([rng.normal(3.0 * k, 1.0, (2, N // C + 1, 64)) for k in range(C)], axis=1)[:, :N]
    X = X.astype(np.float32)
    C0 = X[:, :C].copy()
    cent = f32(C0[None])
    lab, perm, off = sv.kmeans(f32(X[None]), cent, 8)
    lab, perm, off, cent = host(lab)[0], host(perm)[0], host(off)[0], host(cent)[0]
    for h in range(2):
        Co, lo = orc.lloyd(X[h].astype(np.float64), C0[h].astype(np.float64), 8)
        np.testing.assert_array_equal(lab[h], lo)
        po, oo = orc.permute(lo, C)
        np.testing.assert_array_equal(perm[h], po)
        np.testing.assert_array_equal(off[h], oo)
        assert (np.abs(cent[h] - Co).max(axis=1) <= mean_bound(X[h], po, oo) + 1e-6).all()


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_kmeans_cluster_emptied_in_later_round(sv, dtype, D):
    """A cluster that loses every member after the first round keeps its
    centroid, and the clusters its members join get the right means.  Along
    the first axis: 40 points near 0, 40 near 4, and two points at 0.9 and
    3.1.  Centroids start at -1.5, 5.5 and 2.0: the two lone points first go
    to the middle centroid; once the outer centroids have moved onto their
    groups each lone point is nearer to an outer one (0.9 against 1.1), so
    the middle cluster empties in the second round and stays empty."""
    from synth.gen import bf16_bits
    rng = np.random.default_rng(7)
    N = 82
    X = rng.normal(0.0, 0.01, (1, N, D))
    X[0, 40:80, 0] += 4.0
    X[0, 80, 0], X[0, 81, 0] = 0.9, 3.1
    X = X.astype(np.float32)
    if dtype == "bf16":
        X = (bf16_bits(X).astype(np.uint32) << 16).view(np.float32)
    C0 = np.zeros((1, 3, D), np.float32)
    C0[0, :, 0] = (-1.5, 5.5, 2.0)
    cent = f32(C0[:, None])
    lab, perm, off = sv.kmeans(to_dev(X[:, None], dtype), cent, 4)
    Co, lo = orc.lloyd(X[0].astype(np.float64), C0[0].astype(np.float64), 4)
    assert (lo[80], lo[81]) == (0, 1) and not (lo == 2).any()
    np.testing.assert_array_equal(host(lab)[0, 0], lo)
    po, oo = orc.permute(lo, 3)
    np.testing.assert_array_equal(host(perm)[0, 0], po)
    np.testing.assert_array_equal(host(off)[0, 0], oo)
    np.testing.assert_allclose(host(cent)[0, 0], Co, rtol=0, atol=1e-5)


def test_kmeans_incremental_bookkeeping_max_clusters(sv):
    """Six rounds at C = 4096 on 8,192 bf16 tokens (clusters of one or two
    tokens, so many change every round): whatever the tie decisions, after
    the last round each non-empty cluster's centroid is the mean of the
    tokens the last assignment gave it, and perm and offsets sort those
    labels stably.  Means and the sort are recomputed here in fp64 / numpy
    from the returned labels (a property of the result, not the oracle)."""
    w = scaled(WORKLOADS["tiny"], B=1, H=1, N=8192, D=64, dtype="bf16", comps=64, zipf=1.1, Cq=4096, Ck=4096,
               seed=29, density=0.3)
    x = layer_inputs(w)
    X, C0 = x["k"][0].astype(np.float64), x["ck0"][0]
    cent = f32(C0[None, None])
    lab, perm, off = sv.kmeans(to_dev(x["k"][0][None, None], "bf16"), cent, 6)
    lab, cent = host(lab)[0, 0], host(cent)[0, 0]
    assert lab.min() >= 0 and lab.max() < 4096
    po = np.argsort(lab, kind="stable")
    oo = np.concatenate([[0], np.cumsum(np.bincount(lab, minlength=4096))])
    np.testing.assert_array_equal(host(perm)[0, 0], po)
    np.testing.assert_array_equal(host(off)[0, 0], oo)
    sums = np.zeros((4096, X.shape[1]))
    np.add.at(sums, lab, X)
    n = np.diff(oo)
    full = n > 0
    means = sums[full] / n[full, None]
    err = np.abs(cent[full] - means).max(axis=1)
    bound = mean_bound(X, po, oo)[full] + 1e-6
    assert (err <= bound).all(), (err.max(), int((err > bound).sum()))


# ------------------------------------------------------------------ centroids
@pytest.mark.parametrize("name", list(CASES))
def test_centroids_gather_and_means(sv, name, ref_cache):
    w, x, outs, sc = oracle_layer(name, ref_cache)
    for which, perm_key, off_key in (("q", "pq", "oq"), ("k", "pk", "ok"), ("v", "pk", "ok")):
        X = x[which]
        perm = np.stack([o[perm_key] for o in outs])
        off = np.stack([o[off_key] for o in outs])
        xp, mu = sv.centroids(to_dev(reshape4(X, w), w.dtype), i32(reshape4(perm, w)), i32(reshape4(off, w)))
        xp = host(xp).reshape(w.B * w.H, w.N, w.D)
        mu = host(mu).reshape(w.B * w.H, off.shape[1] - 1, w.D)
        for h in range(w.B * w.H):
            np.testing.assert_array_equal(xp[h], X[h][perm[h]])
            ref = orc.means(X[h], perm[h], off[h])
            err = np.abs(mu[h] - ref).max(axis=1)
            assert (err <= mean_bound(X[h], perm[h], off[h]) + 1e-30).all()


# ------------------------------------------------------------------ route
@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("density", [0.1, 0.3, 1.0])
def test_route_teacher_forced(sv, name, density, ref_cache):
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    g = lambda key: np.stack([o[key] for o in outs])
    pk = g("pk")
    Kp = np.stack([x["k"][h][pk[h]] for h in range(BH)])
    Vp = np.stack([x["v"][h][pk[h]] for h in range(BH)])
    qbar, kbar, vbar, oq, ok = g("qbar"), g("kbar"), g("vbar"), g("oq"), g("ok")
    args = (f32(reshape4(qbar, w)), i32(reshape4(oq, w)), to_dev(reshape4(Kp, w), w.dtype),
            to_dev(reshape4(Vp, w), w.dtype), f32(reshape4(kbar, w)), f32(reshape4(vbar, w)), i32(reshape4(ok, w)))
    scores, mask = sv.route(*args, sc, density)
    scores = host(scores).reshape(BH, w.Cq, w.Ck)
    mask = host(mask).reshape(BH, w.Cq, w.Ck)
    for h in range(BH):
        r_o, m_o = orc.route(qbar[h], oq[h], Kp[h], Vp[h], kbar[h], vbar[h], ok[h], sc, density)
        rowmax = r_o.max(axis=1, keepdims=True).astype(np.float64)
        err = np.abs(scores[h].astype(np.float64) - r_o)
        assert (err <= 2e-3 * r_o + 1e-7 * rowmax + 1e-37).all(), (err / (r_o + 1e-30)).max()
        # a mask from the GPU's own ratios may differ only at near-ties of the ratios
        for i in np.flatnonzero((mask[h] != m_o).any(axis=1)):
            sel_o = m_o[i] == 1
            thr = r_o[i][sel_o].min()
            diff = np.flatnonzero(mask[h][i] != m_o[i])
            assert np.all(np.abs(r_o[i][diff] - thr) <= 4e-3 * thr + 1e-7 * rowmax[i]), (i, diff)
    # bit-exact selection given the same float32 ratios
    r_all = np.stack([orc.route(qbar[h], oq[h], Kp[h], Vp[h], kbar[h], vbar[h], ok[h], sc, density)[0]
                      for h in range(BH)])
    _, mask2 = sv.route(*args, sc, density, scores_in=f32(reshape4(r_all, w)))
    mask2 = host(mask2).reshape(BH, w.Cq, w.Ck)
    for h in range(BH):
        q_sizes, k_sizes = np.diff(oq[h]), np.diff(ok[h])
        np.testing.assert_array_equal(mask2[h], orc.select(r_all[h], q_sizes, k_sizes, density, w.N))


def test_route_select_ties_and_empty(sv):
    """Hand-built ratios with ties, an empty key cluster and an empty query cluster."""
    N, Cq, Ck = 10, 3, 5
    ok = np.array([[[0, 3, 4, 8, 8, 10]]], dtype=np.int32)        # sizes 3, 1, 4, 0, 2
    oq = np.array([[[0, 6, 6, 10]]], dtype=np.int32)              # query cluster 1 is empty
    r = np.array([[[[0.5, 0.9, 0.5, 0.7, 0.1], [1, 1, 1, 1, 1], [0.0, 0.0, 0.0, 0.0, 0.0]]]], dtype=np.float32)
    kp = torch.zeros((1, 1, N, 64), dtype=torch.float32, device="cuda")
    _, mask = sv.route(None, i32(oq), kp, None, None, None, i32(ok), 0.125, 0.5, scores_in=f32(r))
    mask = host(mask)[0, 0]
    # row 2: all ratios tie at 0, so clusters go in index order: 0 (3 keys), 1 (4), 2 (8 >= 5, stop)
    assert mask.tolist() == [[1, 1, 1, 0, 0], [0, 0, 0, 0, 0], [1, 1, 1, 0, 0]]
    np.testing.assert_array_equal(mask, orc.select(r[0, 0], np.diff(oq[0, 0]), np.diff(ok[0, 0]), 0.5, N))


@pytest.mark.parametrize("Ck", [1, 63, 64, 65, 512, 513])
def test_route_select_given_ratios_both_fill_kernels(sv, Ck):
    """The greedy fill (FrontierCS blog, budget paragraph: clusters by ratio,
    keys until the budget) from given float32 ratios, bit-exact against the
    oracle on both fill kernels (a wave per query cluster while C_k <= 512, a
    sorting workgroup beyond): tied and zero ratios, empty key and query
    clusters, budgets from none to all."""
    rng = np.random.default_rng(Ck)
    Cq, B, H = 7, 1, 2
    ksz = rng.integers(0, 40, (B * H, Ck)) * (rng.random((B * H, Ck)) > 0.15)
    ksz[:, 0] = np.maximum(ksz[:, 0], 1)
    N = int(ksz.sum(axis=1).max()) + 5
    ksz[:, -1] += N - ksz.sum(axis=1)  # every head's sizes sum to N
    ok = np.concatenate([np.zeros((B * H, 1), np.int64), np.cumsum(ksz, axis=1)], axis=1)
    qsz = np.stack([np.diff(np.sort(np.concatenate([[0, N], rng.integers(0, N + 1, Cq - 1)]))) for _ in range(B * H)])
    qsz[:, 2] = 0
    qsz[:, 3] += N - qsz.sum(axis=1)
    oq = np.concatenate([np.zeros((B * H, 1), np.int64), np.cumsum(qsz, axis=1)], axis=1)
    r = rng.random((B * H, Cq, Ck)).astype(np.float32)
    r[:, 0] = np.round(r[:, 0] * 4) / 4         # many ties
    r[:, 1] = 0.0                                # all tied at zero
    r[:, 4, : Ck // 2] = r[:, 4, Ck // 2:][:, : Ck // 2] if Ck > 1 else r[:, 4, :1]
    kp = torch.zeros((B, H, N, 64), dtype=torch.float32, device="cuda")
    for dens in (1e-9, 0.05, 0.3, 0.999, 1.0):
        _, mask = sv.route(None, i32(oq.reshape(B, H, -1)), kp, None, None, None, i32(ok.reshape(B, H, -1)), 0.125,
                           dens, scores_in=f32(r.reshape(B, H, Cq, Ck)))
        mask = host(mask).reshape(B * H, Cq, Ck)
        for h in range(B * H):
            np.testing.assert_array_equal(mask[h], orc.select(r[h], qsz[h], ksz[h], dens, N), err_msg=f"density {dens}")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_route_degenerate_key_clusters_exact(sv, dtype, D):
    """Key clusters whose members all equal their mean (singletons, clusters of
    identical rows) lose nothing to compensation: e_ij = 0 for every query
    cluster (FrontierCS blog, probe paragraph: the error of a block is the
    gap between its centroid's stand-in and its keys).  The GPU's ratios for
    them are exactly 0 (the oracle's are 0 up to fp64 rounding of its two
    score products), and every other ratio matches the oracle."""
    rng = np.random.default_rng(7 + D)
    sizes = [1] * 5 + [3, 7, 16, 33, 40] + [int(n) for n in rng.integers(2, 60, 10)]
    ok = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    N, Ck, Cq = int(ok[-1]), len(sizes), 5
    rnd = lambda a: host(to_dev(a, dtype)).astype(np.float64)  # values exact in the input dtype
    K = rng.standard_normal((N, D)) + 2.0 * rng.standard_normal(D)
    V = rng.standard_normal((N, D)) + 2.0 * rng.standard_normal(D)
    for j in range(5, 10):
        K[ok[j]:ok[j + 1]] = K[ok[j]]
        V[ok[j]:ok[j + 1]] = V[ok[j]]
    K, V = rnd(K), rnd(V)
    ident = np.arange(N)
    kbar, vbar = orc.means(K, ident, ok), orc.means(V, ident, ok)
    qbar = 1.5 * rng.standard_normal((Cq, D))
    oq = np.linspace(0, N, Cq + 1).astype(np.int32)
    sc = 1.0 / np.sqrt(D)
    r4 = lambda a: a.reshape(1, 1, *a.shape)
    scores, mask = sv.route(f32(r4(qbar)), i32(r4(oq)), to_dev(r4(K), dtype), to_dev(r4(V), dtype), f32(r4(kbar)),
                            f32(r4(vbar)), i32(r4(ok)), sc, 0.3)
    scores = host(scores)[0, 0].astype(np.float64)
    r_o, _ = orc.route(qbar, oq, K, V, kbar, vbar, ok, sc, 0.3)
    rowmax = r_o.max(axis=1, keepdims=True)
    assert (r_o[:, :10] <= 1e-20 * rowmax).all()
    assert (scores[:, :10] == 0).all(), scores[:, :10]
    assert (np.abs(scores - r_o) <= 2e-3 * r_o + 1e-7 * rowmax + 1e-37).all()


# ------------------------------------------------------------------ attention
def attn_inputs(w, x, outs, mask=None):
    BH = w.B * w.H
    g = lambda key: np.stack([o[key] for o in outs])
    pq, pk = g("pq"), g("pk")
    take = lambda a, p: np.stack([a[h][p[h]] for h in range(BH)])
    Qp, Kp, Vp = take(x["q"], pq), take(x["k"], pk), take(x["v"], pk)
    m = g("mask") if mask is None else mask
    dev = (to_dev(reshape4(Qp, w), w.dtype), to_dev(reshape4(Kp, w), w.dtype), to_dev(reshape4(Vp, w), w.dtype),
           i32(reshape4(pq, w)), i32(reshape4(g("oq"), w)), i32(reshape4(g("ok"), w)),
           f32(reshape4(g("kbar"), w)), f32(reshape4(g("vbar"), w)),
           torch.from_numpy(reshape4(m.astype(np.uint8), w)).cuda())
    return dev, m


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("maskkind", ["routed", "dense", "none", "random"])
def test_sparse_attn_teacher_forced(sv, name, maskkind, ref_cache):
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    m = np.stack([o["mask"] for o in outs])
    if maskkind == "dense":
        m = np.ones_like(m)
    elif maskkind == "none":
        m = np.zeros_like(m)
    elif maskkind == "random":
        m = (np.random.default_rng(5).random(m.shape) < 0.35).astype(np.uint8)
    dev, m = attn_inputs(w, x, outs, m)
    out, lse = sv.sparse_attn(*dev, sc, want_lse=True)
    out = host(out).reshape(BH, w.N, w.D)
    lse = host(lse).reshape(BH, w.N)
    amax, amean = ATOL[w.dtype]
    for h in range(BH):
        o = outs[h]
        O, L = orc.attend(x["q"][h], x["k"][h], x["v"][h], o["pq"], o["oq"], o["pk"], o["ok"], o["kbar"], o["vbar"],
                          m[h], sc)
        err = np.abs(out[h] - O)
        assert err.max() <= amax and err.mean() <= amean, (err.max(), err.mean())
        assert np.abs(lse[h] - L).max() <= (1e-2 if w.dtype == "bf16" else 1e-4)


def _subset_with_sum(sizes, target, rng):
    """Indices of clusters whose sizes add up to exactly `target`."""
    for _ in range(2000):
        pick, tot = [], 0
        for j in rng.permutation(len(sizes)):
            if tot + sizes[j] <= target:
                pick.append(j)
                tot += sizes[j]
            if tot == target:
                return sorted(pick)
    raise AssertionError(f"no subset sums to {target}")


@pytest.mark.parametrize("D", [128, 64])
def test_sparse_attn_cluster_boundaries_and_ragged_tiles(sv, D):
    """Key clusters of 1..200 keys, so that cluster boundaries fall at every
    offset of a tile's wave bands and long runs have none; selected lists of
    0, 1, 63, 64, 65 keys and more (partial, exact and one-past tiles); query
    clusters of 1, 31-33, 127-129 rows (partly filled waves and tiles)."""
    from synth.gen import bf16_round
    rng = np.random.default_rng(17 + D)
    N = 1536
    ks = [1, 2, 3, 4, 5, 6, 7, 8, 9, 11, 12, 13, 15, 16, 17, 19, 23, 31, 32, 33, 47, 63, 64, 65, 100, 130, 200]
    ks.append(N - sum(ks))
    qs = [1, 31, 32, 33, 127, 128, 129, 64, 200]
    qs.append(N - sum(qs))
    Ck, Cq = len(ks), len(qs)
    lk = rng.permutation(np.repeat(np.arange(Ck), ks))
    lq = rng.permutation(np.repeat(np.arange(Cq), qs))
    q, k, v = (bf16_round(rng.normal(0.0, 1.0, (N, D)).astype(np.float32)) for _ in range(3))
    pq, oq = orc.permute(lq.astype(np.int64), Cq)
    pk, ok = orc.permute(lk.astype(np.int64), Ck)
    kbar, vbar = orc.means(k, pk, ok), orc.means(v, pk, ok)
    sizes = np.diff(ok)
    mask = (rng.random((Cq, Ck)) < 0.5).astype(np.uint8)
    mask[0] = 1                                      # every cluster
    mask[1] = 0                                      # compensation only
    mask[2] = 0
    mask[2, int(np.argmin(sizes))] = 1               # one key
    for row, target in ((3, 63), (4, 64), (5, 65), (6, 129)):
        mask[row] = 0
        mask[row, _subset_with_sum(list(sizes), target, rng)] = 1
    sc = 1.0 / np.sqrt(D)
    dev4 = lambda a: to_dev(a[None, None], "bf16")
    out, _ = sv.sparse_attn(dev4(q[pq]), dev4(k[pk]), dev4(v[pk]), i32(pq[None, None]), i32(oq[None, None]),
                            i32(ok[None, None]), f32(kbar[None, None]), f32(vbar[None, None]),
                            torch.from_numpy(mask[None, None]).cuda(), sc)
    out = host(out)[0, 0]
    O, _ = orc.attend(q, k, v, pq, oq, pk, ok, kbar, vbar, mask, sc)
    err = np.abs(out - O)
    assert err.max() <= ATOL["bf16"][0] and err.mean() <= ATOL["bf16"][1], (err.max(), err.mean())


def test_sparse_attn_density_one_is_full_attention(sv, ref_cache):
    w, x, outs, sc = oracle_layer("bf16-d128", ref_cache)
    m = np.stack([(np.diff(o["ok"]) > 0)[None, :].repeat(w.Cq, 0) for o in outs]).astype(np.uint8)
    dev, _ = attn_inputs(w, x, outs, m)
    out, _ = sv.sparse_attn(*dev, sc)
    out = host(out).reshape(w.B * w.H, w.N, w.D)
    for h in range(w.B * w.H):
        ref = orc.full_attention(x["q"][h], x["k"][h], x["v"][h], sc)
        err = np.abs(out[h] - ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3


# ------------------------------------------------------------------ end to end
def check_layer_end_to_end(sv, w, x, L, out, outs, sc, density, iters, tag):
    """The layer's output against the oracle, whatever valid labels the GPU
    reached.  Labels: equal to the oracle's Lloyd iterates, or the first
    round that differs differs only at near ties.  The oracle then rebuilds
    every later stage from the GPU's own final labels: perm and offsets
    bit-exact, the GPU mask equal to the oracle's except at ratio near ties
    and bit-exact when selected from the oracle's ratios, and the output
    compared on every row against the oracle attending with the GPU's mask."""
    BH = w.B * w.H
    out = host(out).reshape(BH, w.N, w.D)
    lq, lk = host(L.lq).reshape(BH, -1), host(L.lk).reshape(BH, -1)
    pq, pk = host(L.pq).reshape(BH, -1), host(L.pk).reshape(BH, -1)
    mask = host(L.mask).reshape(BH, w.Cq, w.Ck)
    amax, amean = ATOL[w.dtype]
    refs = []
    for h in range(BH):
        o = outs[h]
        for which, lab_g, C0 in (("q", lq[h], x["cq0"][h]), ("k", lk[h], x["ck0"][h])):
            if (lab_g != o["l" + which]).any():
                xd = to_dev(reshape4(x[which], w), w.dtype)

                def after(r, which=which):
                    cent = f32(reshape4(x["c" + which + "0"], w))
                    return host(sv.kmeans(xd, cent, r)[0]).reshape(BH, -1)[h]

                r, n = first_divergence(after, x[which][h], C0, iters)
                assert r is not None, (which, "final labels differ although every round agreed")
                print(f"{tag} head {h}: {which} labels first differ in round {r} at {n} near ties")
        ref = oracle_from_labels(x["q"][h], x["k"][h], x["v"][h], lq[h], lk[h], w.Cq, w.Ck, sc, density)
        np.testing.assert_array_equal(pq[h], ref["pq"])
        np.testing.assert_array_equal(pk[h], ref["pk"])
        nd = check_ratio_masks(mask[h], ref["ratio"], ref["mask"])
        O, _ = orc.attend(x["q"][h], x["k"][h], x["v"][h], ref["pq"], ref["oq"], ref["pk"], ref["ok"], ref["kbar"],
                          ref["vbar"], mask[h], sc)
        err = np.abs(out[h] - O)
        print(f"{tag} head {h}: output vs oracle max {err.max():.3e}, mean {err.mean():.3e}; "
              f"{nd} near-tie mask blocks")
        assert err.max() <= amax and err.mean() <= amean, (err.max(), err.mean())
        refs.append(ref)
    # the selection itself, bit-exact from the oracle's float32 ratios
    r_all = np.stack([r["ratio"] for r in refs])
    _, m2 = sv.route(L.qm, L.oq, L.kp, L.vp, L.km, L.vm, L.ok, sc, density, scores_in=f32(reshape4(r_all, w)))
    m2 = host(m2).reshape(BH, w.Cq, w.Ck)
    for h in range(BH):
        np.testing.assert_array_equal(m2[h], refs[h]["mask"])


@pytest.mark.parametrize("name", ["f32-d64", "bf16-d128"])
def test_layer_end_to_end(sv, name, ref_cache):
    w, x, outs, sc = oracle_layer(name, ref_cache, iters=3, density=0.3)
    L = sv.Layer(w.B, w.H, w.N, w.D, w.Cq, w.Ck, dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    cq, ck = f32(reshape4(x["cq0"], w)), f32(reshape4(x["ck0"], w))
    out = L.forward(to_dev(reshape4(x["q"], w), w.dtype), to_dev(reshape4(x["k"], w), w.dtype),
                    to_dev(reshape4(x["v"], w), w.dtype), cq, ck, 3, 0.3, sc)
    check_layer_end_to_end(sv, w, x, L, out, outs, sc, 0.3, 3, name)


def test_tiny_config_end_to_end(sv):
    """The Tiny workload exactly as specified: 1 x 2 heads x 2,048 tokens x 64,
    fp32 Q/K/V from a 16-component uniform Gaussian mixture (sigma 0.3, seed
    0), 16 query and 32 key clusters, 10 cold k-means rounds, density 0.30;
    the whole layer through the Layer object, output at the fp32 tolerance."""
    w = WORKLOADS["tiny"]
    assert (w.B, w.H, w.N, w.D, w.dtype, w.comps, w.zipf, w.Cq, w.Ck, w.iters, w.density) == \
        (1, 2, 2048, 64, "f32", 16, None, 16, 32, 10, 0.30)
    x = layer_inputs(w)
    sc = 1.0 / np.sqrt(w.D)
    outs = [orc.layer(x["q"][h], x["k"][h], x["v"][h], x["cq0"][h], x["ck0"][h], w.iters, w.density, sc)
            for h in range(w.B * w.H)]
    L = sv.Layer(w.B, w.H, w.N, w.D, w.Cq, w.Ck, dtype=torch.float32)
    cq, ck = f32(reshape4(x["cq0"], w)), f32(reshape4(x["ck0"], w))
    out = L.forward(to_dev(reshape4(x["q"], w), "f32"), to_dev(reshape4(x["k"], w), "f32"),
                    to_dev(reshape4(x["v"], w), "f32"), cq, ck, w.iters, w.density, sc)
    check_layer_end_to_end(sv, w, x, L, out, outs, sc, w.density, w.iters, "tiny")


def test_layer_is_deterministic(sv):
    w, x = make("bf16-d128")
    sc = 1.0 / np.sqrt(w.D)
    L = sv.Layer(w.B, w.H, w.N, w.D, w.Cq, w.Ck)
    res = []
    for _ in range(2):
        cq, ck = f32(reshape4(x["cq0"], w)), f32(reshape4(x["ck0"], w))
        out = L.forward(to_dev(reshape4(x["q"], w), "bf16"), to_dev(reshape4(x["k"], w), "bf16"),
                        to_dev(reshape4(x["v"], w), "bf16"), cq, ck, 4, 0.25, sc)
        res.append((out.clone(), L.scores.clone(), cq.clone(), ck.clone()))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ variance-corrected compensation
@pytest.mark.parametrize("name", list(CASES))
def test_centroid_variances(sv, name, ref_cache):
    """Per-cluster coordinate variances from the oracle's permutation and
    means; bound: (n + 4) u relative (fp32 sums of squares of fp32
    deviations) plus a tiny absolute floor."""
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    for key, p, o, mkey in (("k", "pk", "ok", "kbar"), ("q", "pq", "oq", "qbar")):
        perm = np.stack([oo[p] for oo in outs])
        off = np.stack([oo[o] for oo in outs])
        mu = np.stack([oo[mkey] for oo in outs]).astype(np.float32)
        var = sv.centroid_variances(to_dev(reshape4(x[key], w), w.dtype), i32(reshape4(perm, w)),
                                    i32(reshape4(off, w)), f32(reshape4(mu, w)))
        var = host(var).reshape(BH, off.shape[1] - 1, w.D)
        for h in range(BH):
            ref = orc.variances(x[key][h], perm[h], off[h])
            n = np.diff(off[h]).astype(np.float64)[:, None]
            tol = (n + 4) * 2.0 ** -24 * ref + 1e-12 * max(1.0, float(ref.max()))
            assert np.all(np.abs(var[h] - ref) <= tol), float((np.abs(var[h] - ref) - tol).max())


@pytest.mark.parametrize("name", ["bf16-d128", "bf16-d64"])
@pytest.mark.parametrize("strength", [0.5, 1.0, 1.5])
def test_sparse_attn_variance_corrected(sv, name, strength, ref_cache):
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    m = np.stack([o["mask"] for o in outs])
    dev, m = attn_inputs(w, x, outs, m)
    kvar = np.stack([orc.variances(x["k"][h], outs[h]["pk"], outs[h]["ok"]) for h in range(BH)])
    out, lse = sv.sparse_attn(*dev, sc, want_lse=True, k_vars=f32(reshape4(kvar, w)), strength=strength)
    out = host(out).reshape(BH, w.N, w.D)
    lse = host(lse).reshape(BH, w.N)
    amax, amean = ATOL[w.dtype]
    for h in range(BH):
        o = outs[h]
        O, L = orc.attend(x["q"][h], x["k"][h], x["v"][h], o["pq"], o["oq"], o["pk"], o["ok"], o["kbar"], o["vbar"],
                          m[h], sc, kvar=kvar[h], strength=strength)
        err = np.abs(out[h] - O)
        assert err.max() <= amax and err.mean() <= amean, (err.max(), err.mean())
        assert np.abs(lse[h] - L).max() <= 1e-2


def test_sparse_attn_variance_strength_zero_is_plain(sv, ref_cache):
    # At strength 0 the variance kernel computes the plain method: its output
    # meets the plain oracle at the attention tolerances.  (It is not the plain
    # kernel's output bit for bit: its pseudo-key tiles hold 32 clusters instead
    # of 64, so the online softmax rescales at other points.)
    w, x, outs, sc = oracle_layer("bf16-d128", ref_cache)
    BH = w.B * w.H
    dev, m = attn_inputs(w, x, outs)
    kvar = np.stack([orc.variances(x["k"][h], outs[h]["pk"], outs[h]["ok"]) for h in range(BH)])
    zero, _ = sv.sparse_attn(*dev, sc, k_vars=f32(reshape4(kvar, w)), strength=0.0)
    zero = host(zero).reshape(BH, w.N, w.D)
    amax, amean = ATOL[w.dtype]
    for h in range(BH):
        o = outs[h]
        O, _ = orc.attend(x["q"][h], x["k"][h], x["v"][h], o["pq"], o["oq"], o["pk"], o["ok"], o["kbar"], o["vbar"],
                          m[h], sc)
        err = np.abs(zero[h] - O)
        assert err.max() <= amax and err.mean() <= amean, (err.max(), err.mean())


# ------------------------------------------------------------------ top-p budget (SVG2) routing
def topp_oracle(qbar, oq, kbar, ok, sc, p):
    qs, ks = np.diff(oq), np.diff(ok)
    P = orc.topp_probs(qbar, kbar, ks, sc)
    P[qs == 0] = 0.0
    tm = orc.topp_select(P, qs, ks, p)
    return P, tm, orc.topp_budgets(tm, ks)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("p", [0.5, 0.9, 1.0])
def test_route_topp_teacher_forced(sv, name, p, ref_cache):
    """Shares within fp32 rounding of the oracle's; given the oracle's float32
    shares and ratios, masks and budgets are bit-exact in both modes."""
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    g = lambda key: np.stack([o[key] for o in outs])
    pk = g("pk")
    Kp = np.stack([x["k"][h][pk[h]] for h in range(BH)])
    Vp = np.stack([x["v"][h][pk[h]] for h in range(BH)])
    qbar, kbar, vbar, oq, ok, r_all = g("qbar"), g("kbar"), g("vbar"), g("oq"), g("ok"), g("ratio")
    args = (f32(reshape4(qbar, w)), i32(reshape4(oq, w)), to_dev(reshape4(Kp, w), w.dtype),
            to_dev(reshape4(Vp, w), w.dtype), f32(reshape4(kbar, w)), f32(reshape4(vbar, w)), i32(reshape4(ok, w)))
    ref = [topp_oracle(qbar[h], oq[h], kbar[h], ok[h], sc, p) for h in range(BH)]
    P_all = np.stack([t[0] for t in ref])
    shp = lambda t: host(t).reshape(BH, *t.shape[2:])
    # the GPU's own shares
    probs, _, bud0, m0 = sv.route_topp(*args, sc, p, error_ranked=False)
    probs1, scores1, bud1, m1 = sv.route_topp(*args, sc, p, error_ranked=True, want_scores=True)
    probs, probs1, bud0, bud1, m0, m1 = map(shp, (probs, probs1, bud0, bud1, m0, m1))
    scores1 = shp(scores1)
    np.testing.assert_array_equal(probs, probs1)
    np.testing.assert_array_equal(bud0, bud1)
    for h in range(BH):
        P_o, tm_o, b_o = ref[h]
        ks, qs = np.diff(ok[h]), np.diff(oq[h])
        assert (np.abs(probs[h] - P_o) <= 1e-4 * P_o + 1e-37).all(), np.abs(probs[h] - P_o).max()
        diff_rows = check_topp_masks(m0[h], P_o, tm_o, ks, p)
        same = np.setdiff1d(np.arange(w.Cq), diff_rows)
        np.testing.assert_array_equal(bud0[h][same], b_o[same])
        np.testing.assert_array_equal(bud0[h], (m0[h].astype(np.int64) * ks).sum(axis=1))
        m1_o = orc.select_budgets(r_all[h], qs, ks, b_o)
        check_ratio_masks(m1[h], r_all[h], m1_o, rows=same)
    # bit-exact from the oracle's float32 shares and ratios
    pin, rin = f32(reshape4(P_all, w)), f32(reshape4(r_all, w))
    probs2, _, bud2, m2 = sv.route_topp(*args, sc, p, error_ranked=False, probs_in=pin)
    _, _, bud3, m3 = sv.route_topp(*args, sc, p, error_ranked=True, probs_in=pin, scores_in=rin)
    probs2, bud2, m2, bud3, m3 = map(shp, (probs2, bud2, m2, bud3, m3))
    np.testing.assert_array_equal(probs2, P_all)
    for h in range(BH):
        P_o, tm_o, b_o = ref[h]
        qs, ks = np.diff(oq[h]), np.diff(ok[h])
        np.testing.assert_array_equal(m2[h], tm_o)
        np.testing.assert_array_equal(bud2[h], b_o)
        np.testing.assert_array_equal(bud3[h], b_o)
        np.testing.assert_array_equal(m3[h], orc.select_budgets(r_all[h], qs, ks, b_o))
        if p == 1.0:
            assert (m2[h][qs > 0][:, ks > 0] == 1).all()


def test_route_topp_hand_example(sv):
    """Hand-built shares with ties, an empty key cluster and an empty query
    cluster, in both modes, against the oracle's selection."""
    N, Cq, Ck = 10, 3, 5
    ok = np.array([[[0, 3, 4, 4, 8, 10]]], dtype=np.int32)        # sizes 3, 1, 0, 4, 2
    oq = np.array([[[0, 6, 6, 10]]], dtype=np.int32)              # query cluster 1 is empty
    P = np.array([[[[0.25, 0.5, 0.0, 0.125, 0.125], [0.2, 0.2, 0.0, 0.3, 0.3],
                    [0.1, 0.1, 0.0, 0.1, 0.7]]]], dtype=np.float32)
    r = np.array([[[[0.5, 0.9, 0.0, 0.7, 0.1], [1, 1, 0, 1, 1], [0.3, 0.2, 0.0, 0.1, 0.0]]]], dtype=np.float32)
    kp = torch.zeros((1, 1, N, 64), dtype=torch.float32, device="cuda")
    qs, ks = np.diff(oq[0, 0]), np.diff(ok[0, 0])
    for p in (0.5, 0.6, 0.8, 1.0):
        probs, _, bud, m = sv.route_topp(None, i32(oq), kp, None, None, None, i32(ok), 0.125, p,
                                         error_ranked=False, probs_in=f32(P))
        tm = orc.topp_select(P[0, 0], qs, ks, p)
        np.testing.assert_array_equal(host(m)[0, 0], tm)
        np.testing.assert_array_equal(host(bud)[0, 0], orc.topp_budgets(tm, ks))
        assert host(m)[0, 0][1].sum() == 0 and host(bud)[0, 0][1] == 0
        _, _, bud1, m1 = sv.route_topp(None, i32(oq), kp, None, None, None, i32(ok), 0.125, p,
                                       error_ranked=True, probs_in=f32(P), scores_in=f32(r))
        np.testing.assert_array_equal(host(m1)[0, 0], orc.select_budgets(r[0, 0], qs, ks, orc.topp_budgets(tm, ks)))
    # p = 0.8.  Row 0: order 1 (0.5), 0 (0.25), then 3 and 4 tie at 0.125 and 3 goes
    # first; 0.875 >= 0.8 stops before 4.  Row 2: float32 0.7 + 0.1 summed in double
    # is 0.79999999, below float32 0.8 (0.80000001), so a second 0.1 share is taken.
    _, _, _, m = sv.route_topp(None, i32(oq), kp, None, None, None, i32(ok), 0.125, 0.8, error_ranked=False,
                               probs_in=f32(P))
    assert host(m)[0, 0].tolist() == [[1, 1, 0, 1, 0], [0, 0, 0, 0, 0], [1, 1, 0, 0, 1]]


@pytest.mark.parametrize("name", ["bf16-d128"])
def test_route_topp_then_attention(sv, name, ref_cache):
    """The top-p masks drive the same attention kernel: output within the bf16
    tolerance of the oracle attending with the oracle's top-p mask."""
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    g = lambda key: np.stack([o[key] for o in outs])
    qbar, kbar, oq, ok, r_all = g("qbar"), g("kbar"), g("oq"), g("ok"), g("ratio")
    masks = []
    for h in range(BH):
        P_o, _, b_o = topp_oracle(qbar[h], oq[h], kbar[h], ok[h], sc, 0.9)
        masks.append(orc.select_budgets(r_all[h], np.diff(oq[h]), np.diff(ok[h]), b_o))
    m = np.stack(masks)
    dev, m = attn_inputs(w, x, outs, m)
    out, _ = sv.sparse_attn(*dev, sc)
    out = host(out).reshape(BH, w.N, w.D)
    amax, amean = ATOL[w.dtype]
    for h in range(BH):
        o = outs[h]
        O, _ = orc.attend(x["q"][h], x["k"][h], x["v"][h], o["pq"], o["oq"], o["pk"], o["ok"], o["kbar"], o["vbar"],
                          m[h], sc)
        err = np.abs(out[h] - O)
        assert err.max() <= amax and err.mean() <= amean, (err.max(), err.mean())


# ------------------------------------------------------------------ k-means++ seeding
def words_dev(words, w):
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int64)).reshape(w.B, w.H, -1).cuda()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("which", ["q", "k"])
def test_kmeanspp_matches_oracle(sv, name, which):
    """Every seed index bit-exact (the rules fix every rounding), every seed row
    an exact copy, over all heads, several tiles and a ragged tail."""
    from synth.gen import seed_words
    w, x = make(name)
    BH = w.B * w.H
    C = w.Cq if which == "q" else w.Ck
    words = np.stack([seed_words(w, h, which, C) for h in range(BH)])
    cent, chosen = sv.kmeanspp(to_dev(reshape4(x[which], w), w.dtype), words_dev(words, w), C)
    cent, chosen = host(cent).reshape(BH, C, w.D), host(chosen).reshape(BH, C)
    for h in range(BH):
        seeds, idx = orc.kmeanspp(x[which][h], words[h], C)
        np.testing.assert_array_equal(chosen[h], idx)
        np.testing.assert_array_equal(cent[h].astype(np.float64), seeds)


def test_kmeanspp_edge_cases(sv):
    """One seed; as many seeds as rows (each row once); rows repeated so every
    distance reaches 0 before the last seed (uniform fallback)."""
    rng = np.random.default_rng(77)
    N, D = 300, 64
    X = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    words = rng.integers(0, np.iinfo(np.uint64).max, size=(1, 1, N), dtype=np.uint64, endpoint=True)
    W = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).cuda()
    xd = torch.from_numpy(X).cuda()
    for C in (1, 7, N):
        cent, chosen = sv.kmeanspp(xd, W(words[:, :, :C]), C)
        seeds, idx = orc.kmeanspp(X[0, 0], words[0, 0, :C], C)
        np.testing.assert_array_equal(host(chosen)[0, 0], idx)
        np.testing.assert_array_equal(host(cent)[0, 0].astype(np.float64), seeds)
    assert sorted(host(chosen)[0, 0].tolist()) == list(range(N))
    Y = np.repeat(rng.standard_normal((5, 128)).astype(np.float32), 60, axis=0)[None, None]   # N = 300
    yb = to_dev(Y[0, 0], "bf16")[None, None]
    Yr = host(yb)[0, 0]
    for C in (5, 9):
        cent, chosen = sv.kmeanspp(yb, W(words[:, :, :C]), C)
        seeds, idx = orc.kmeanspp(Yr, words[0, 0, :C], C)
        np.testing.assert_array_equal(host(chosen)[0, 0], idx)
        assert len({int(i) // 60 for i in idx[:5]}) == 5


# ------------------------------------------------------------------ FP8 variant
@pytest.mark.parametrize("name", ["bf16-d128", "bf16-d64", "f32-d64"])
def test_quantize_fp8_matches_oracle(sv, name):
    """e4m3 codes and per-head exponents bit-exact (the scaling is exact and
    both sides round to nearest even)."""
    w, x = make(name)
    BH = w.B * w.H
    for key in ("q", "k"):
        x8, ex = sv.quantize_fp8(to_dev(reshape4(x[key], w), w.dtype))
        x8 = host(x8).reshape(BH, w.N, w.D)
        ex = host(ex).reshape(BH)
        for h in range(BH):
            codes, e = orc.quantize_e4m3(x[key][h])
            assert ex[h] == e
            np.testing.assert_array_equal(x8[h], codes)


def fp8_inputs(w, x, outs):
    """Oracle e4m3 codes of Q and K per head (original order), their exponents
    and dequantised values."""
    BH = w.B * w.H
    q8, k8, qe, ke, qd, kd = [], [], [], [], [], []
    for h in range(BH):
        cq, eq = orc.quantize_e4m3(x["q"][h])
        ck, ek = orc.quantize_e4m3(x["k"][h])
        q8.append(cq[outs[h]["pq"]])
        k8.append(ck[outs[h]["pk"]])
        qe.append(eq)
        ke.append(ek)
        qd.append(orc.dequantize_e4m3(cq, eq))
        kd.append(orc.dequantize_e4m3(ck, ek))
    dev8 = lambda a: torch.from_numpy(reshape4(np.stack(a), w)).cuda()
    devi = lambda a: torch.tensor(np.array(a, np.int32).reshape(w.B, w.H)).cuda()
    return dev8(q8), devi(qe), dev8(k8), devi(ke), qd, kd


@pytest.mark.parametrize("name", ["bf16-d128", "bf16-d64"])
@pytest.mark.parametrize("maskkind", ["routed", "dense", "none"])
def test_sparse_attn_fp8_teacher_forced(sv, name, maskkind, ref_cache):
    """FP8 attention against the oracle attending with the dequantised Q and
    K (the same computation), at the bf16 path's tolerance; the error against
    unquantised attention is reported."""
    w, x, outs, sc = oracle_layer(name, ref_cache)
    BH = w.B * w.H
    m = np.stack([o["mask"] for o in outs])
    if maskkind == "dense":
        m = np.ones_like(m)
    elif maskkind == "none":
        m = np.zeros_like(m)
    dev, m = attn_inputs(w, x, outs, m)
    q8, qe, k8, ke, qd, kd = fp8_inputs(w, x, outs)
    _, _, vp, pq, oq, ok, km, vm, mask = dev
    out, lse = sv.sparse_attn_fp8(q8, qe, k8, ke, vp, pq, oq, ok, km, vm, mask, sc, want_lse=True)
    out = host(out).reshape(BH, w.N, w.D)
    lse = host(lse).reshape(BH, w.N)
    amax, amean = ATOL["bf16"]
    qerr = 0.0
    for h in range(BH):
        o = outs[h]
        O, L = orc.attend(qd[h], kd[h], x["v"][h], o["pq"], o["oq"], o["pk"], o["ok"], o["kbar"], o["vbar"], m[h], sc)
        err = np.abs(out[h] - O)
        assert err.max() <= amax and err.mean() <= amean, (err.max(), err.mean())
        assert np.abs(lse[h] - L).max() <= 1e-2
        O0, _ = orc.attend(x["q"][h], x["k"][h], x["v"][h], o["pq"], o["oq"], o["pk"], o["ok"], o["kbar"],
                           o["vbar"], m[h], sc)
        qerr = max(qerr, float(np.abs(out[h] - O0).max()))
    print(f"[fp8] {name}/{maskkind}: max |O_fp8 - O_unquantised| = {qerr:.3e}", flush=True)


def test_sparse_attn_fp8_exact_codes_equal_bf16_path(sv, ref_cache):
    """Inputs that are already e4m3 values with max|x| = 448 * 2^e quantise
    exactly, so the FP8 path and the bf16 path attend to the same numbers."""
    w, x, outs, sc = oracle_layer("bf16-d128", ref_cache)
    BH = w.B * w.H
    x2 = dict(x)
    for key in ("q", "k"):
        arr = []
        for h in range(BH):
            c, e = orc.quantize_e4m3(x[key][h])
            arr.append(orc.dequantize_e4m3(c, e).astype(np.float32))
        x2[key] = np.stack(arr)
    dev, m = attn_inputs(w, x2, outs)
    q8, qe, k8, ke, _, _ = fp8_inputs(w, x2, outs)
    qp, kp, vp, pq, oq, ok, km, vm, mask = dev
    o8, _ = sv.sparse_attn_fp8(q8, qe, k8, ke, vp, pq, oq, ok, km, vm, mask, sc)
    ob, _ = sv.sparse_attn(qp, kp, vp, pq, oq, ok, km, vm, mask, sc)
    d = (o8.float() - ob.float()).abs()
    assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


@pytest.mark.parametrize("variant", ["topp-error", "topp-score", "variance", "fp8"])
def test_layer_variants_are_the_composed_calls(sv, variant):
    """Layer.forward with a variant option gives bit for bit what the
    individual calls give in sequence (every call is deterministic)."""
    w, x = make("bf16-d128")
    sc = 1.0 / np.sqrt(w.D)
    q, k, v = (to_dev(reshape4(x[key], w), "bf16") for key in ("q", "k", "v"))
    cq0, ck0 = f32(reshape4(x["cq0"], w)), f32(reshape4(x["ck0"], w))
    opts = {"topp-error": dict(top_p=0.9), "topp-score": dict(top_p=0.9, router="score"),
            "variance": dict(strength=1.0), "fp8": dict(fp8=True)}[variant]
    L = sv.Layer(w.B, w.H, w.N, w.D, w.Cq, w.Ck)
    out = L.forward(q, k, v, cq0.clone(), ck0.clone(), 3, 0.3, sc, **opts).clone()
    cq, ck = cq0.clone(), ck0.clone()
    shp = lambda *s_, dt=torch.int32: torch.empty(s_, dtype=dt, device="cuda")
    lq, pq, oq = shp(w.B, w.H, w.N), shp(w.B, w.H, w.N), shp(w.B, w.H, w.Cq + 1)
    lk, pk, ok = shp(w.B, w.H, w.N), shp(w.B, w.H, w.N), shp(w.B, w.H, w.Ck + 1)
    sv.kmeans(k, ck, 3, lk, pk, ok)
    sv.kmeans(q, cq, 3, lq, pq, oq)
    qp, qm = sv.centroids(q, pq, oq)
    kp, km = sv.centroids(k, pk, ok)
    vp, vm = sv.centroids(v, pk, ok)
    if "top_p" in opts:
        _, _, _, mask = sv.route_topp(qm, oq, kp, vp, km, vm, ok, sc, 0.9, error_ranked=(variant == "topp-error"))
    else:
        _, mask = sv.route(qm, oq, kp, vp, km, vm, ok, sc, 0.3)
    if variant == "fp8":
        q8, qe = sv.quantize_fp8(qp)
        k8, ke = sv.quantize_fp8(kp)
        ref, _ = sv.sparse_attn_fp8(q8, qe, k8, ke, vp, pq, oq, ok, km, vm, mask, sc)
    elif variant == "variance":
        kv = sv.centroid_variances(k, pk, ok, km)
        ref, _ = sv.sparse_attn(qp, kp, vp, pq, oq, ok, km, vm, mask, sc, k_vars=kv, strength=1.0)
    else:
        ref, _ = sv.sparse_attn(qp, kp, vp, pq, oq, ok, km, vm, mask, sc)
    assert torch.equal(out, ref)


def test_maximum_cluster_counts(sv):
    """C_q = C_k = 4096, the largest count any call accepts, on 8,192 tokens
    (clusters of one or two tokens): one k-means round, centroids, routing and
    attention, each stage fed the oracle's previous stage."""
    from synth.gen import layer_inputs
    w = scaled(WORKLOADS["tiny"], B=1, H=1, N=8192, D=64, dtype="bf16", comps=64, zipf=1.1, Cq=4096, Ck=4096,
               seed=23, density=0.3)
    x = layer_inputs(w)
    sc = 1.0 / 8.0
    o = orc.layer(x["q"][0], x["k"][0], x["v"][0], x["cq0"][0], x["ck0"][0], 1, 0.3, sc)
    dev = {key: to_dev(x[key][0][None, None], "bf16") for key in ("q", "k", "v")}
    for which, C0, lkey, pkey, okey in (("q", x["cq0"][0], "lq", "pq", "oq"), ("k", x["ck0"][0], "lk", "pk", "ok")):
        lab, perm, off = sv.kmeans(dev[which], f32(C0[None, None]), 1)
        nbad = check_labels_near_ties(x[which][0], C0, host(lab)[0, 0], o[lkey])
        if nbad == 0:
            np.testing.assert_array_equal(host(perm)[0, 0], o[pkey])
            np.testing.assert_array_equal(host(off)[0, 0], o[okey])
    pq, oq, pk, ok = (i32(o[key][None, None]) for key in ("pq", "oq", "pk", "ok"))
    qp, qm = sv.centroids(dev["q"], pq, oq)
    kp, km = sv.centroids(dev["k"], pk, ok)
    vp, vm = sv.centroids(dev["v"], pk, ok)
    for mu, key, X, perm, off in ((qm, "qbar", x["q"][0], o["pq"], o["oq"]), (km, "kbar", x["k"][0], o["pk"], o["ok"]),
                                  (vm, "vbar", x["v"][0], o["pk"], o["ok"])):
        err = np.abs(host(mu)[0, 0] - o[key]).max(axis=1)
        assert (err <= mean_bound(X, perm, off) + 1e-30).all()
    qbar, kbar, vbar = (f32(o[key][None, None]) for key in ("qbar", "kbar", "vbar"))
    _, mask = sv.route(qbar, oq, kp, vp, kbar, vbar, ok, sc, 0.3, scores_in=f32(o["ratio"][None, None]))
    np.testing.assert_array_equal(host(mask)[0, 0], o["mask"])
    scores, _ = sv.route(qbar, oq, kp, vp, kbar, vbar, ok, sc, 0.3)
    r_o = o["ratio"].astype(np.float64)
    rowmax = r_o.max(axis=1, keepdims=True)
    assert (np.abs(host(scores)[0, 0] - r_o) <= 2e-3 * r_o + 1e-7 * rowmax + 1e-37).all()
    m = torch.from_numpy(o["mask"][None, None].astype(np.uint8)).cuda()
    out, _ = sv.sparse_attn(qp, kp, vp, pq, oq, ok, kbar, vbar, m, sc)
    err = np.abs(host(out)[0, 0] - o["O"])
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
