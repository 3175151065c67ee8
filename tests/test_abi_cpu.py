"""The C-ABI library loads, exports every symbol include/svgear.h declares,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svgear.h")
LIB = os.path.join(ROOT, "sparse_attention_video_amd", "libsvgear.so")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(svgear_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libsvgear.so is not built (run __graft_entry__.build())")
    from sparse_attention_video_amd import svgear
    return svgear.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared()
    assert len(names) == 19
    for n in names:
        assert hasattr(lib, n), n
    from sparse_attention_video_amd import svgear
    assert sorted(svgear.EXPORTS) == names


def test_version(lib):
    assert lib.svgear_version().decode().startswith("svgear ")


def test_workspace_queries_are_positive_and_monotone(lib):
    a = lib.svgear_kmeans_workspace(1, 40, 75600, 128, 500)
    b = lib.svgear_kmeans_workspace(1, 40, 75600, 128, 100)
    assert a > b > 0
    assert lib.svgear_route_workspace(1, 40, 75600, 128, 100, 500) > 0
    assert lib.svgear_sparse_attn_workspace(1, 40, 75600, 128, 100, 500) > 0
    assert lib.svgear_centroids_workspace(1, 40, 75600, 128, 500) > 0
    assert lib.svgear_kmeans_workspace(1, 1, 10, 96, 2) == 0     # bad D


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def call_kmeans(lib, **kw):
    a = dict(x=FAKE, dt=0, B=1, H=1, N=100, D=64, C=4, iters=1, cent=FAKE, lab=FAKE, perm=FAKE, off=FAKE,
             ws=None, wsb=0)
    a.update(kw)
    return lib.svgear_kmeans(a["x"], a["dt"], a["B"], a["H"], a["N"], a["D"], a["C"], a["iters"], a["cent"],
                             a["lab"], a["perm"], a["off"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=96), 1), (dict(C=0), 1), (dict(C=101), 1), (dict(iters=0), 1), (dict(N=0), 1),
    (dict(dt=7), 1), (dict(x=None), 1), (dict(B=0), 1), (dict(C=5000, N=6000), 1),
    (dict(), 3),                                     # valid arguments but no workspace
    (dict(ws=ctypes.c_void_p(0x1001), wsb=1 << 40), 3),  # misaligned workspace
])
def test_kmeans_validation(lib, kw, status):
    assert call_kmeans(lib, **kw) == status
    assert lib.svgear_last_error().decode()


def test_route_and_attn_validation(lib):
    F = FAKE
    # density out of range, scale not positive
    assert lib.svgear_route(F, F, 4, F, F, 0, F, F, F, 8, 1, 1, 100, 64, ctypes.c_float(0.125),
                            ctypes.c_float(1.5), None, None, F, None, 0, None) == 1
    assert lib.svgear_route(F, F, 4, F, F, 0, F, F, F, 8, 1, 1, 100, 64, ctypes.c_float(-1.0),
                            ctypes.c_float(0.5), None, None, F, None, 0, None) == 1
    assert lib.svgear_sparse_attn(F, F, F, 0, F, F, 4, F, 8, F, F, F, 1, 1, 100, 64, ctypes.c_float(0.125),
                                  None, None, None, 0, None) == 1          # out is null
    assert lib.svgear_sparse_attn(F, F, F, 0, F, F, 4, F, 8, F, F, F, 1, 1, 100, 64, ctypes.c_float(0.125),
                                  F, None, None, 0, None) == 3             # no workspace
    assert lib.svgear_centroids(F, 1, 1, 1, 100, 64, 200, F, F, F, F, None, 0, None) == 1
    # variance variants: bf16 only, strength >= 0, variance table required
    V = lambda dt, kv, strength: lib.svgear_sparse_attn_var(F, F, F, dt, F, F, 4, F, 8, F, F, kv,
                                                             ctypes.c_float(strength), F, 1, 1, 100, 64,
                                                             ctypes.c_float(0.125), F, None, None, 0, None)
    assert V(1, F, 1.0) == 2                 # float32: unsupported
    assert V(0, None, 1.0) == 1              # no variances
    assert V(0, F, -0.5) == 1                # negative strength
    assert V(0, F, 1.0) == 3                 # valid so far, no workspace
    assert lib.svgear_centroid_variances(F, 0, 1, 1, 100, 64, 4, F, F, None, F, None, 0, None) == 1
    assert lib.svgear_centroid_variances(F, 0, 1, 1, 100, 64, 4, F, F, F, F, None, 0, None) == 3
    # top-p routing: p in (0, 1], error_ranked in {0, 1}, ratios only with error ranking
    T = lambda p, er, scores_in=None, mask=F, k_perm=F: lib.svgear_route_topp(
        F, F, 4, k_perm, F, 0, F, F, F, 8, 1, 1, 100, 64, ctypes.c_float(0.125), ctypes.c_float(p), er, None,
        scores_in, None, None, None, mask, None, 0, None)
    assert T(0.0, 1) == 1 and T(1.5, 1) == 1 and T(float("nan"), 0) == 1
    assert T(0.9, 2) == 1                    # error_ranked not 0/1
    assert T(0.9, 0, scores_in=F) == 1       # ratios with the score router
    assert T(0.9, 1, mask=None) == 1         # no mask
    assert T(0.9, 1, k_perm=None) == 1       # the probe needs the keys
    assert T(0.9, 0, k_perm=None) == 3       # the score router does not; no workspace
    assert T(1.0, 1) == 3
    # k-means++ seeding: C in [1, N], words and centroids required
    K = lambda C, words=F, cent=F: lib.svgear_kmeanspp(F, 0, 1, 1, 100, 64, C, words, cent, None, None, 0, None)
    assert K(0) == 1 and K(101) == 1 and K(5, words=None) == 1 and K(5, cent=None) == 1
    assert K(5) == 3 and K(100) == 3
    assert lib.svgear_kmeanspp_workspace(1, 40, 75600, 128) >= 40 * 75600 * 8
    # FP8 variant
    assert lib.svgear_quantize_fp8(F, 0, 1, 1, 100, 64, None, F, None, 0, None) == 1
    assert lib.svgear_quantize_fp8(F, 0, 1, 1, 100, 96, F, F, None, 0, None) == 1
    assert lib.svgear_quantize_fp8(F, 0, 1, 1, 100, 64, F, F, None, 0, None) == 3
    A8 = lambda qe: lib.svgear_sparse_attn_fp8(F, qe, F, F, F, F, F, 4, F, 8, F, F, F, 1, 1, 100, 64,
                                               ctypes.c_float(0.125), F, None, None, 0, None)
    assert A8(None) == 1 and A8(F) == 3


def test_fault_injection_returns_injected_without_work():
    """SVGEAR_FAULT=<call> makes that call report SVGEAR_ERR_INJECTED (a caller's
    dense fallback can be tested with the oracle standing in)."""
    code = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from sparse_attention_video_amd import svgear\n"
        "lib = svgear.load()\n"
        "F = ctypes.c_void_p(0x1000)\n"
        "st = lib.svgear_kmeans(F, 0, 1, 1, 100, 64, 4, 1, F, F, F, F, None, 0, None)\n"
        "st2 = lib.svgear_sparse_attn(F, F, F, 0, F, F, 4, F, 8, F, F, F, 1, 1, 100, 64, ctypes.c_float(0.1), F, None, None, 0, None)\n"
        "print(st, st2)\n"
    )
    env = dict(os.environ, SVGEAR_FAULT="kmeans")
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == ["5", "3"]


def test_binding_refuses_cpu_tensors():
    import torch
    from sparse_attention_video_amd import svgear
    x = torch.zeros((1, 1, 64, 64))
    with pytest.raises(ValueError):
        svgear.kmeans(x, torch.zeros((1, 1, 4, 64)), 1)


def test_attn_grid_limit_at_the_size_boundary(lib):
    """The largest token count the library takes (N = 2^24 - 1) still passes
    validation for one head (its row bytes fit the 32-bit buffer range); a
    grid of query tiles larger than one launch is refused before any launch,
    and its workspace query reports 0."""
    F = FAKE
    N = (1 << 24) - 1
    A = lambda B, H, Cq: lib.svgear_sparse_attn(F, F, F, 0, F, F, Cq, F, 8, F, F, F, B, H, N, 128,
                                                ctypes.c_float(0.125), F, None, None, 0, None)
    assert A(1, 1, 4) == 3                   # valid sizes; only the workspace is missing
    assert lib.svgear_sparse_attn_workspace(1, 1, N, 128, 4, 8) > 0
    assert A(1, 65535, 4096) == 1            # 135,168 tiles per head x 65,535 heads
    assert "grid" in lib.svgear_last_error().decode()
    assert lib.svgear_sparse_attn_workspace(1, 65535, N, 128, 4096, 8) == 0
    assert A(1, 1, 4) == 3


def _cpu_case(B=1, H=2, N=64, D=64, Cq=4, Ck=8):
    import torch
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt)
    i = torch.int32
    return dict(q=z(B, H, N, D), k=z(B, H, N, D), v=z(B, H, N, D), idx=z(B, H, N, dt=i), oq=z(B, H, Cq + 1, dt=i),
                ok=z(B, H, Ck + 1, dt=i), km=z(B, H, Ck, D), vm=z(B, H, Ck, D), qm=z(B, H, Cq, D),
                mask=z(B, H, Cq, Ck, dt=torch.uint8))


@pytest.mark.parametrize("bad", [
    dict(oq="int64"), dict(ok="int64"), dict(idx="int64"), dict(mask="bool"), dict(km="float64"),
    dict(k="bfloat16"), dict(mask_shape=(1, 2, 3, 8)), dict(ok_shape=(1, 1, 9)), dict(vm_shape=(1, 2, 7, 64)),
    dict(out="float64"), dict(lse_shape=(1, 2, 63)),
])
def test_binding_validates_attention_tables(bad):
    """Every table's dtype and shape is checked before anything reaches the
    library (int64 offsets, a wrongly shaped mask, ...), so a wrong table can
    never make a kernel index outside its buffers.  CPU tensors: the checks
    run before the device check."""
    import torch
    from sparse_attention_video_amd import svgear
    a = _cpu_case()
    kw = {}
    for key, val in bad.items():
        if key.endswith("_shape"):
            name = key[:-6]
            src = a.get(name)
            shape = val
            dt = src.dtype if src is not None else torch.float32
            a[name] = torch.zeros(shape, dtype=dt)
        elif key in ("out", "lse"):
            kw[key] = torch.zeros(a["q"].shape, dtype=getattr(torch, val))
        else:
            a[key] = a[key].to(getattr(torch, val))
    if "lse" in a:
        kw["lse"] = a.pop("lse")
        kw["want_lse"] = True
    with pytest.raises(ValueError):
        svgear.sparse_attn(a["q"], a["k"], a["v"], a["idx"], a["oq"], a["ok"], a["km"], a["vm"], a["mask"], 0.125,
                           **kw)


def test_binding_validates_other_calls():
    import torch
    from sparse_attention_video_amd import svgear
    a = _cpu_case()
    i32, f32 = torch.int32, torch.float32
    with pytest.raises(ValueError, match="centroids"):
        svgear.kmeans(a["k"], torch.zeros((1, 2, 8, 32)), 1)                 # D mismatch
    with pytest.raises(ValueError, match="offsets"):
        svgear.kmeans(a["k"], a["km"], 1, offsets=torch.zeros((1, 2, 8), dtype=i32))
    with pytest.raises(ValueError, match="perm"):
        svgear.centroids(a["k"], a["idx"].long(), a["ok"])
    with pytest.raises(ValueError, match="means"):
        svgear.centroids(a["k"], a["idx"], a["ok"], means=torch.zeros((1, 2, 9, 64)))
    with pytest.raises(ValueError, match="mask"):
        svgear.route(a["qm"], a["oq"], a["k"], a["v"], a["km"], a["vm"], a["ok"], 0.125, 0.25,
                     mask=torch.zeros((1, 2, 4, 8), dtype=torch.int32))
    with pytest.raises(ValueError, match="v_perm"):
        svgear.route(a["qm"], a["oq"], a["k"], a["v"].bfloat16(), a["km"], a["vm"], a["ok"], 0.125, 0.25)
    with pytest.raises(ValueError, match="scores_in"):
        svgear.route(None, a["oq"], a["k"], None, None, None, a["ok"], 0.125, 0.25,
                     scores_in=torch.zeros((1, 2, 8, 4)))
    with pytest.raises(ValueError, match="probs_in"):
        svgear.route_topp(a["qm"], a["oq"], a["k"], a["v"], a["km"], a["vm"], a["ok"], 0.125, 0.9,
                          probs_in=torch.zeros((1, 2, 4, 8), dtype=torch.float64))
    with pytest.raises(ValueError, match="words"):
        svgear.kmeanspp(a["k"], torch.zeros((1, 2, 4), dtype=i32), 4)
    with pytest.raises(ValueError, match="exps"):
        svgear.quantize_fp8(a["k"], exps=torch.zeros((1, 2), dtype=torch.int64))
    with pytest.raises(ValueError, match="k8"):
        svgear.sparse_attn_fp8(torch.zeros((1, 2, 64, 64), dtype=torch.uint8), torch.zeros((1, 2), dtype=i32),
                               torch.zeros((1, 2, 64, 64)), torch.zeros((1, 2), dtype=i32), a["v"].bfloat16(),
                               a["idx"], a["oq"], a["ok"], a["km"], a["vm"], a["mask"], 0.125)
    with pytest.raises(ValueError, match="vars"):
        svgear.centroid_variances(a["k"], a["idx"], a["ok"], a["km"], vars=torch.zeros((1, 2, 8, 64), dtype=f32)[..., :32])
    with pytest.raises(ValueError, match="ws"):
        svgear.sparse_attn(a["q"], a["k"], a["v"], a["idx"], a["oq"], a["ok"], a["km"], a["vm"], a["mask"], 0.125,
                           ws=torch.zeros(16, dtype=f32))


def test_noalloc_attention_validates_before_touching_the_gpu(lib):
    """The allocation-free attention entry point refuses sizes whose scratch
    exceeds its static array, and bad arguments, before any HIP call."""
    F = FAKE
    A = lambda H, N, Cq, Ck, out=F: lib.svgear_sparse_attn_noalloc(F, F, F, 0, F, F, Cq, F, Ck, F, F, F, 1, H, N, 128,
                                                                   ctypes.c_float(0.088), out, None, None)
    assert lib.svgear_sparse_attn_workspace(1, 200, 75600, 128, 100, 500) > (32 << 20)
    assert A(200, 75600, 100, 500) == 1
    assert "scratch" in lib.svgear_last_error().decode()
    assert A(40, 75600, 0, 500) == 1         # invalid sizes: workspace query 0, validation refuses
    assert A(40, 100, 200, 500) == 1         # Cq > N
