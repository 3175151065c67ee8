"""The k-means assign kernel's two rigorous shortcuts, checked in emulated fp32.

Both shortcuts claim that no label can change because of them; the GPU
parity tests see that only through the labels of their inputs.  Here the
claims are checked over many random and adversarial operands with numpy
float32 arithmetic (each operation rounded to fp32, and once more with the
products fused, since the device compiler may contract them):

* windowed key insertion: an estimate V above thr = (kb + W(kb)) (1 + 4 q)
  gives a key (V with its low ib bits replaced by a list index) that lies
  outside the tie window of every final best key k <= kb, where the window is
  W(k) = 2 E0 + q (2 k + 2 E0 + 1) 2.5 and q = 2^(ib - 23);
* centroid distance bounds: lb = s - P / 2 - 0.02 s, with s = |c_a|^2 + |c_c|^2
  and P the fp32 sum of products of the bf16 high halves of -2 c_a and -2 c_c,
  never exceeds |c_a - c_c|^2.

CPU only."""
import numpy as np

F = np.float32


def _fma(a, b, c):
    # fp32 fused multiply-add: the product of two fp32 values is exact in
    # fp64, so one rounding of the fp64 sum (exact here but for a last-bit
    # double rounding, far inside the margins tested) stands in for it
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F)


def _window(k, e0, q, fused):
    two, one, h = F(2), F(1), F(2.5)
    if fused:
        inner = _fma(two, k, _fma(two, e0, one))
        return _fma(q * inner, h, two * e0)
    return two * e0 + q * (two * k + two * e0 + one) * h


def _threshold(kb, e0, q, fused):
    w = _window(kb, e0, q, fused)
    return (kb + w) * (F(1) + F(4) * q)


def _key(v, idx, ib):
    imask = np.uint32((1 << ib) - 1)
    b = v.view(np.uint32)
    return ((b & ~imask) | np.uint32(idx)).view(F)


def test_windowed_insertion_never_skips_a_key_of_the_final_window():
    rng = np.random.default_rng(11)
    n = 200_000
    for ib in (7, 8, 9, 10, 11):
        q = F(2.0 ** (ib - 23))
        # best keys so far: from just above the offset floor (>= 1) to large
        kb = F(10.0) ** rng.uniform(0.0, 4.0, n).astype(F)
        # the kernel's offset keeps kb >= 4 e0, and E0 ~ 1.25 e0
        e0 = (kb * rng.uniform(0.0, 0.33, n)).astype(F)
        for fused in (False, True):
            thr = _threshold(kb, e0, q, fused)
            for ulps in (1, 2, 7, 1000):
                v = thr.view(np.uint32) + np.uint32(ulps)
                v = v.view(F)
                for idx in (0, (1 << ib) - 1):
                    kv = _key(v, idx, ib)
                    # the final best: any key at or below kb, including kb itself
                    for frac in (1.0, 0.999999, 0.99, 0.5, 1e-3):
                        k = (kb * F(frac)).astype(F)
                        gap = kv - k
                        w = _window(k, e0, q, fused)
                        assert np.all(gap > w), (ib, fused, ulps, idx, frac)


def _bf16_round(x):
    # round to nearest even at bf16 (8-bit significand), as the device's
    # fp32 -> bf16 conversion does
    b = x.astype(F).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (r << 16).astype(np.uint32).view(F)


def _bounds(cent):
    hi = _bf16_round(F(-2) * cent)  # [C, D]
    # fp32 accumulation of the products in a fixed order (the matrix unit's
    # own order differs; its error is of the same size)
    P = np.zeros((cent.shape[0], cent.shape[0]), dtype=F)
    for d in range(cent.shape[1]):
        P = (P + np.outer(hi[:, d], hi[:, d]).astype(F)).astype(F)
    n = (cent.astype(np.float64) ** 2).sum(1).astype(F)
    s = (n[:, None] + n[None, :]).astype(F)
    lb = (s - F(0.5) * P - F(0.02) * s).astype(F)
    exact = ((cent[:, None, :].astype(np.float64) - cent[None, :, :].astype(np.float64)) ** 2).sum(-1)
    return lb, exact


def test_centroid_distance_bounds_stay_below_the_exact_distances():
    rng = np.random.default_rng(5)
    for D in (64, 128):
        # a mixture: centroids in tight groups (near-equal pairs), loose ones,
        # large and small norms, a shared offset (large norms, small distances)
        base = rng.normal(0, 1, (1, D)) * 6.0
        tight = base + rng.normal(0, 1e-3, (24, D))
        loose = rng.normal(0, 1, (24, D)) * rng.uniform(0.01, 20.0, (24, 1))
        dup = np.repeat(rng.normal(0, 3, (4, D)), 2, axis=0)
        cent = np.concatenate([tight, loose, dup]).astype(F)
        lb, exact = _bounds(cent)
        assert np.all(lb.astype(np.float64) <= exact), float((lb - exact).max())
        # and it is tight: below the exact distance by at most 2% of the
        # norms' sum plus the high halves' error (2^-7 of it)
        n64 = (cent.astype(np.float64) ** 2).sum(1)
        s64 = n64[:, None] + n64[None, :]
        assert np.all(exact - lb.astype(np.float64) <= 0.03 * s64 + 1e-6)
