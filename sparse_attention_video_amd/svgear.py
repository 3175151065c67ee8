"""Thin ctypes binding over libsvgear.so (the C ABI in include/svgear.h).

Only argument marshalling happens here: torch supplies device memory (outputs
and workspaces) and the current HIP stream; every step of the path runs in the
library's HIP kernels.  If the library is missing or the tensors are not on a
GPU, calls raise instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvgear.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_INJECTED = range(6)
BF16, F32 = 0, 1

EXPORTS = (
    "svgear_version", "svgear_last_error",
    "svgear_kmeans_workspace", "svgear_kmeans",
    "svgear_centroids_workspace", "svgear_centroids",
    "svgear_route_workspace", "svgear_route",
    "svgear_sparse_attn_workspace", "svgear_sparse_attn",
    "svgear_centroid_variances", "svgear_sparse_attn_var",
    "svgear_route_topp",
    "svgear_kmeanspp_workspace", "svgear_kmeanspp",
    "svgear_quantize_fp8_workspace", "svgear_quantize_fp8", "svgear_sparse_attn_fp8",
    "svgear_sparse_attn_noalloc",
)

_lib = None


class SvgearError(RuntimeError):
    def __init__(self, call: str, status: int, msg: str):
        super().__init__(f"{call} failed with status {status}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with sparse_attention_video_amd/build.py")
    lib = ctypes.CDLL(path)
    P, I, F, Z, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_double
    lib.svgear_version.restype = ctypes.c_char_p
    lib.svgear_last_error.restype = ctypes.c_char_p
    lib.svgear_kmeans_workspace.argtypes = [I, I, I, I, I]
    lib.svgear_kmeans_workspace.restype = Z
    lib.svgear_kmeans.argtypes = [P, I, I, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.svgear_kmeans.restype = I
    lib.svgear_centroids_workspace.argtypes = [I, I, I, I, I]
    lib.svgear_centroids_workspace.restype = Z
    lib.svgear_centroids.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.svgear_centroids.restype = I
    lib.svgear_route_workspace.argtypes = [I, I, I, I, I, I]
    lib.svgear_route_workspace.restype = Z
    lib.svgear_route.argtypes = [P, P, I, P, P, I, P, P, P, I, I, I, I, I, F, F, P, P, P, P, Z, P]
    lib.svgear_route.restype = I
    lib.svgear_sparse_attn_workspace.argtypes = [I, I, I, I, I, I]
    lib.svgear_sparse_attn_workspace.restype = Z
    lib.svgear_sparse_attn.argtypes = [P, P, P, I, P, P, I, P, I, P, P, P, I, I, I, I, F, P, P, P, Z, P]
    lib.svgear_sparse_attn.restype = I
    lib.svgear_centroid_variances.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, Z, P]
    lib.svgear_centroid_variances.restype = I
    lib.svgear_sparse_attn_var.argtypes = [P, P, P, I, P, P, I, P, I, P, P, P, F, P, I, I, I, I, F, P, P, P, Z, P]
    lib.svgear_sparse_attn_var.restype = I
    lib.svgear_route_topp.argtypes = [P, P, I, P, P, I, P, P, P, I, I, I, I, I, F, F, I, P, P, P, P, P, P, P, Z, P]
    lib.svgear_route_topp.restype = I
    lib.svgear_kmeanspp_workspace.argtypes = [I, I, I, I]
    lib.svgear_kmeanspp_workspace.restype = Z
    lib.svgear_kmeanspp.argtypes = [P, I, I, I, I, I, I, P, P, P, P, Z, P]
    lib.svgear_kmeanspp.restype = I
    lib.svgear_quantize_fp8_workspace.argtypes = [I, I]
    lib.svgear_quantize_fp8_workspace.restype = Z
    lib.svgear_quantize_fp8.argtypes = [P, I, I, I, I, I, P, P, P, Z, P]
    lib.svgear_quantize_fp8.restype = I
    lib.svgear_sparse_attn_fp8.argtypes = [P, P, P, P, P, P, P, I, P, I, P, P, P, I, I, I, I, F, P, P, P, Z, P]
    lib.svgear_sparse_attn_fp8.restype = I
    lib.svgear_sparse_attn_noalloc.argtypes = [P, P, P, I, P, P, I, P, I, P, P, P, I, I, I, I, F, P, P, P]
    lib.svgear_sparse_attn_noalloc.restype = I
    _lib = lib
    return lib


def version() -> str:
    return load().svgear_version().decode()


def _check(call: str, status: int) -> None:
    if status != OK:
        raise SvgearError(call, status, load().svgear_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("svgear runs on the GPU only: every tensor must be on a HIP device")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


_FLOAT = (torch.bfloat16, torch.float32)


def _want(name: str, t: Optional[torch.Tensor], dtype, shape=None, optional: bool = True) -> None:
    """Checks one tensor argument before anything is launched: its dtype (one
    dtype or a tuple of allowed ones) and its shape (a tuple whose None
    entries match any size).  Raises ValueError on a mismatch, so that a
    wrong table can never make a kernel index outside its buffers."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in allowed:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in allowed)}, not {t.dtype}")
    if shape is not None:
        ok = t.dim() == len(shape) and all(s is None or int(a) == int(s) for a, s in zip(t.shape, shape))
        if not ok:
            want = "[" + ", ".join("*" if s is None else str(s) for s in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, not {list(t.shape)}")


def _want_ws(ws: Optional[torch.Tensor]) -> None:
    _want("ws", ws, torch.uint8, (None,))


def _dims4(name: str, t: torch.Tensor, dtype=_FLOAT):
    _want(name, t, dtype, (None, None, None, None), optional=False)
    return tuple(int(a) for a in t.shape)


def _offsets(name: str, t: torch.Tensor, B: Optional[int] = None, H: Optional[int] = None) -> int:
    """int32 [B, H, C + 1] offsets; returns C."""
    _want(name, t, torch.int32, (B, H, None), optional=False)
    if t.shape[2] < 2:
        raise ValueError(f"{name} must hold at least one cluster")
    return int(t.shape[2]) - 1


def _workspace(nbytes: int, dev: torch.device) -> torch.Tensor:
    ws = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=dev)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + max(int(nbytes), 1)]


def _route_tables(B, H, Cq, Ck, q_means, k_perm, v_perm, k_means, v_means, needs_probe: bool, D=None) -> None:
    """Shapes and dtypes of the routing inputs that are given (all of them
    when the probe runs)."""
    if k_perm is not None:
        _, _, N, D = _dims4("k_perm", k_perm)
        _want("k_perm", k_perm, _FLOAT, (B, H, N, D))
        _want("v_perm", v_perm, k_perm.dtype, (B, H, N, D), optional=not needs_probe)
    elif needs_probe:
        raise ValueError("k_perm is required")
    _want("q_means", q_means, torch.float32, (B, H, Cq, D), optional=not needs_probe)
    _want("k_means", k_means, torch.float32, (B, H, Ck, D), optional=not needs_probe)
    _want("v_means", v_means, torch.float32, (B, H, Ck, D), optional=not needs_probe)


def _attn_tables(B, H, N, D, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out, out_dtype, lse):
    """Shapes and dtypes of the attention inputs besides Q', K', V'; returns (Cq, Ck)."""
    _want("q_perm_idx", q_perm_idx, torch.int32, (B, H, N), optional=False)
    Cq = _offsets("q_offsets", q_offsets, B, H)
    Ck = _offsets("k_offsets", k_offsets, B, H)
    _want("k_means", k_means, torch.float32, (B, H, Ck, D), optional=False)
    _want("v_means", v_means, torch.float32, (B, H, Ck, D), optional=False)
    _want("mask", mask, torch.uint8, (B, H, Cq, Ck), optional=False)
    _want("out", out, out_dtype, (B, H, N, D))
    _want("lse", lse, torch.float32, (B, H, N))
    return Cq, Ck


# ----------------------------------------------------------------------------
def kmeans(x: torch.Tensor, centroids: torch.Tensor, iters: int, labels=None, perm=None, offsets=None, ws=None):
    """Lloyd k-means; ``centroids`` [B,H,C,D] fp32 is updated in place.

    Returns (labels [B,H,N] int32, perm [B,H,N] int32, offsets [B,H,C+1] int32)."""
    B, H, N, D = _dims4("x", x)
    _want("centroids", centroids, torch.float32, (B, H, None, D), optional=False)
    C = int(centroids.shape[2])
    _want("labels", labels, torch.int32, (B, H, N))
    _want("perm", perm, torch.int32, (B, H, N))
    _want("offsets", offsets, torch.int32, (B, H, C + 1))
    _want_ws(ws)
    dev = _dev(x, centroids, labels, perm, offsets, ws)
    labels = labels if labels is not None else torch.empty((B, H, N), dtype=torch.int32, device=dev)
    perm = perm if perm is not None else torch.empty((B, H, N), dtype=torch.int32, device=dev)
    offsets = offsets if offsets is not None else torch.empty((B, H, C + 1), dtype=torch.int32, device=dev)
    lib = load()
    need = lib.svgear_kmeans_workspace(B, H, N, D, C)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_kmeans", lib.svgear_kmeans(_ptr(x), _dtype(x), B, H, N, D, C, int(iters), _ptr(centroids),
                                              _ptr(labels), _ptr(perm), _ptr(offsets), _ptr(ws), ws.numel(),
                                              _stream(dev)))
    return labels, perm, offsets


def centroids(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, want_perm: bool = True,
              want_means: bool = True, x_perm=None, means=None, ws=None):
    """Returns (x_perm [B,H,N,D] or None, means [B,H,C,D] fp32 or None)."""
    B, H, N, D = _dims4("x", x)
    _want("perm", perm, torch.int32, (B, H, N), optional=False)
    C = _offsets("offsets", offsets, B, H)
    _want("x_perm", x_perm, x.dtype, (B, H, N, D))
    _want("means", means, torch.float32, (B, H, C, D))
    _want_ws(ws)
    dev = _dev(x, perm, offsets, x_perm, means, ws)
    if want_perm and x_perm is None:
        x_perm = torch.empty_like(x)
    if want_means and means is None:
        means = torch.empty((B, H, C, D), dtype=torch.float32, device=dev)
    lib = load()
    need = lib.svgear_centroids_workspace(B, H, N, D, C)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_centroids", lib.svgear_centroids(_ptr(x), _dtype(x), B, H, N, D, C, _ptr(perm), _ptr(offsets),
                                                    _ptr(x_perm if want_perm else None),
                                                    _ptr(means if want_means else None), _ptr(ws), ws.numel(),
                                                    _stream(dev)))
    return (x_perm if want_perm else None), (means if want_means else None)


def route(q_means, q_offsets, k_perm, v_perm, k_means, v_means, k_offsets, scale: float, density: float,
          scores_in: Optional[torch.Tensor] = None, want_scores: bool = True, mask=None, scores=None, ws=None):
    """Returns (scores [B,H,Cq,Ck] fp32 or None, mask [B,H,Cq,Ck] uint8)."""
    Cq = _offsets("q_offsets", q_offsets)
    B, H = int(q_offsets.shape[0]), int(q_offsets.shape[1])
    Ck = _offsets("k_offsets", k_offsets, B, H)
    _route_tables(B, H, Cq, Ck, q_means, k_perm, v_perm, k_means, v_means, needs_probe=scores_in is None)
    for name, t in (("scores_in", scores_in), ("scores", scores)):
        _want(name, t, torch.float32, (B, H, Cq, Ck))
    _want("mask", mask, torch.uint8, (B, H, Cq, Ck))
    _want_ws(ws)
    dev = _dev(q_offsets, k_offsets, mask, scores, ws)
    if scores_in is None:
        _dev(q_means, k_perm, v_perm, k_means, v_means)
        N, D = k_perm.shape[2], k_perm.shape[3]
        dt = _dtype(k_perm)
    else:
        _dev(scores_in)
        N = int(k_perm.shape[2]) if k_perm is not None else None
        D = int(k_perm.shape[3]) if k_perm is not None else 64
        dt = _dtype(k_perm) if k_perm is not None else F32
        if N is None:
            raise ValueError("k_perm (or its shape) is needed for N")
    mask = mask if mask is not None else torch.empty((B, H, Cq, Ck), dtype=torch.uint8, device=dev)
    if want_scores and scores is None:
        scores = torch.empty((B, H, Cq, Ck), dtype=torch.float32, device=dev)
    lib = load()
    need = lib.svgear_route_workspace(B, H, N, D, Cq, Ck)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_route", lib.svgear_route(_ptr(q_means), _ptr(q_offsets), Cq, _ptr(k_perm), _ptr(v_perm), dt,
                                            _ptr(k_means), _ptr(v_means), _ptr(k_offsets), Ck, B, H, N, D,
                                            float(scale), float(density), _ptr(scores_in),
                                            _ptr(scores if want_scores else None), _ptr(mask), _ptr(ws), ws.numel(),
                                            _stream(dev)))
    return (scores if want_scores else None), mask


def kmeanspp(x: torch.Tensor, words: torch.Tensor, C: int, centroids=None, chosen=None, ws=None):
    """k-means++ seeds from one uniform 64-bit word per seed (words: [B,H,C]
    int64 or uint64 tensor, bits taken as unsigned).  Returns (centroids
    [B,H,C,D] fp32, chosen [B,H,C] int32)."""
    B, H, N, D = _dims4("x", x)
    _want("words", words, (torch.int64, torch.uint64), (B, H, C), optional=False)
    _want("centroids", centroids, torch.float32, (B, H, C, D))
    _want("chosen", chosen, torch.int32, (B, H, C))
    _want_ws(ws)
    dev = _dev(x, words, centroids, chosen, ws)
    centroids = centroids if centroids is not None else torch.empty((B, H, C, D), dtype=torch.float32, device=dev)
    chosen = chosen if chosen is not None else torch.empty((B, H, C), dtype=torch.int32, device=dev)
    lib = load()
    need = lib.svgear_kmeanspp_workspace(B, H, N, D)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_kmeanspp", lib.svgear_kmeanspp(_ptr(x), _dtype(x), B, H, N, D, C, _ptr(words), _ptr(centroids),
                                                  _ptr(chosen), _ptr(ws), ws.numel(), _stream(dev)))
    return centroids, chosen


def quantize_fp8(x: torch.Tensor, x8=None, exps=None, ws=None):
    """e4m3fn codes [B,H,N,D] uint8 and per-(batch, head) exponents [B,H] int32."""
    B, H, N, D = _dims4("x", x)
    _want("x8", x8, torch.uint8, (B, H, N, D))
    _want("exps", exps, torch.int32, (B, H))
    _want_ws(ws)
    dev = _dev(x, x8, exps, ws)
    x8 = x8 if x8 is not None else torch.empty((B, H, N, D), dtype=torch.uint8, device=dev)
    exps = exps if exps is not None else torch.empty((B, H), dtype=torch.int32, device=dev)
    lib = load()
    need = lib.svgear_quantize_fp8_workspace(B, H)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_quantize_fp8", lib.svgear_quantize_fp8(_ptr(x), _dtype(x), B, H, N, D, _ptr(x8), _ptr(exps),
                                                          _ptr(ws), ws.numel(), _stream(dev)))
    return x8, exps


def sparse_attn_fp8(q8, q_exp, k8, k_exp, v_perm, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask,
                    scale: float, want_lse: bool = False, out=None, lse=None, ws=None):
    """FP8 variant: e4m3 Q'/K' (from quantize_fp8), bf16 V'.  Returns (out, lse or None)."""
    B, H, N, D = _dims4("v_perm", v_perm, torch.bfloat16)
    _want("q8", q8, torch.uint8, (B, H, N, D), optional=False)
    _want("k8", k8, torch.uint8, (B, H, N, D), optional=False)
    _want("q_exp", q_exp, torch.int32, (B, H), optional=False)
    _want("k_exp", k_exp, torch.int32, (B, H), optional=False)
    Cq, Ck = _attn_tables(B, H, N, D, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out,
                          torch.bfloat16, lse)
    _want_ws(ws)
    dev = _dev(q8, q_exp, k8, k_exp, v_perm, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out, lse, ws)
    out = out if out is not None else torch.empty_like(v_perm)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    lib = load()
    need = lib.svgear_sparse_attn_workspace(B, H, N, D, Cq, Ck)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_sparse_attn_fp8",
           lib.svgear_sparse_attn_fp8(_ptr(q8), _ptr(q_exp), _ptr(k8), _ptr(k_exp), _ptr(v_perm), _ptr(q_perm_idx),
                                      _ptr(q_offsets), Cq, _ptr(k_offsets), Ck, _ptr(k_means), _ptr(v_means),
                                      _ptr(mask), B, H, N, D, float(scale), _ptr(out), _ptr(lse if want_lse else None),
                                      _ptr(ws), ws.numel(), _stream(dev)))
    return out, (lse if want_lse else None)


def route_topp(q_means, q_offsets, k_perm, v_perm, k_means, v_means, k_offsets, scale: float, top_p: float,
               error_ranked: bool = True, probs_in: Optional[torch.Tensor] = None,
               scores_in: Optional[torch.Tensor] = None, want_probs: bool = True, want_scores: bool = False,
               want_budget: bool = True, N: Optional[int] = None, D: Optional[int] = None, ws=None):
    """Routing under the SVG2 top-p budget.  Returns (probs [B,H,Cq,Ck] fp32 or
    None, scores [B,H,Cq,Ck] fp32 or None, budget [B,H,Cq] int32 or None,
    mask [B,H,Cq,Ck] uint8).  N and D default to k_perm's shape."""
    Cq = _offsets("q_offsets", q_offsets)
    B, H = int(q_offsets.shape[0]), int(q_offsets.shape[1])
    Ck = _offsets("k_offsets", k_offsets, B, H)
    _route_tables(B, H, Cq, Ck, q_means, k_perm, v_perm, k_means, v_means,
                  needs_probe=bool(error_ranked) and scores_in is None, D=D)
    for name, t in (("probs_in", probs_in), ("scores_in", scores_in)):
        _want(name, t, torch.float32, (B, H, Cq, Ck))
    _want_ws(ws)
    dev = _dev(q_offsets, k_offsets, ws)
    if k_perm is not None:
        _dev(k_perm)
        N, D, dt = int(k_perm.shape[2]), int(k_perm.shape[3]), _dtype(k_perm)
    else:
        if N is None or D is None:
            raise ValueError("N and D are needed when k_perm is not given")
        dt = F32
    for t in (q_means, v_perm, k_means, v_means, probs_in, scores_in):
        if t is not None:
            _dev(t)
    mk = lambda shape, dtype: torch.empty(shape, dtype=dtype, device=dev)
    mask = mk((B, H, Cq, Ck), torch.uint8)
    probs = mk((B, H, Cq, Ck), torch.float32) if want_probs else None
    scores = mk((B, H, Cq, Ck), torch.float32) if (want_scores and error_ranked) else None
    budget = mk((B, H, Cq), torch.int32) if want_budget else None
    lib = load()
    need = lib.svgear_route_workspace(B, H, N, D, Cq, Ck)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_route_topp",
           lib.svgear_route_topp(_ptr(q_means), _ptr(q_offsets), Cq, _ptr(k_perm), _ptr(v_perm), dt, _ptr(k_means),
                                 _ptr(v_means), _ptr(k_offsets), Ck, B, H, N, D, float(scale), float(top_p),
                                 1 if error_ranked else 0, _ptr(probs_in), _ptr(scores_in), _ptr(probs),
                                 _ptr(scores), _ptr(budget), _ptr(mask), _ptr(ws), ws.numel(), _stream(dev)))
    return probs, scores, budget, mask


def centroid_variances(x: torch.Tensor, perm: torch.Tensor, offsets: torch.Tensor, means: torch.Tensor, vars=None,
                       ws=None):
    """Per-cluster, per-coordinate population variances [B,H,C,D] fp32."""
    B, H, N, D = _dims4("x", x)
    _want("perm", perm, torch.int32, (B, H, N), optional=False)
    C = _offsets("offsets", offsets, B, H)
    _want("means", means, torch.float32, (B, H, C, D), optional=False)
    _want("vars", vars, torch.float32, (B, H, C, D))
    _want_ws(ws)
    dev = _dev(x, perm, offsets, means, vars, ws)
    vars = vars if vars is not None else torch.empty((B, H, C, D), dtype=torch.float32, device=dev)
    lib = load()
    need = lib.svgear_centroids_workspace(B, H, N, D, C)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("svgear_centroid_variances",
           lib.svgear_centroid_variances(_ptr(x), _dtype(x), B, H, N, D, C, _ptr(perm), _ptr(offsets), _ptr(means),
                                         _ptr(vars), _ptr(ws), ws.numel(), _stream(dev)))
    return vars


def sparse_attn(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, scale: float,
                want_lse: bool = False, out=None, lse=None, ws=None, k_vars=None, strength: float = 0.0):
    """Returns (out [B,H,N,D] in original token order, lse [B,H,N] fp32 or None).
    With ``k_vars`` the skipped clusters' scores gain strength * sigma^2 / 2
    (variance-corrected compensation, bf16 only)."""
    B, H, N, D = _dims4("q_perm", q_perm)
    _want("k_perm", k_perm, q_perm.dtype, (B, H, N, D), optional=False)
    _want("v_perm", v_perm, q_perm.dtype, (B, H, N, D), optional=False)
    Cq, Ck = _attn_tables(B, H, N, D, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out, q_perm.dtype,
                          lse)
    _want("k_vars", k_vars, torch.float32, (B, H, Ck, D))
    _want_ws(ws)
    dev = _dev(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out, lse, k_vars, ws)
    out = out if out is not None else torch.empty_like(q_perm)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    lib = load()
    need = lib.svgear_sparse_attn_workspace(B, H, N, D, Cq, Ck)
    ws = ws if ws is not None else _workspace(need, dev)
    if k_vars is None:
        _check("svgear_sparse_attn",
               lib.svgear_sparse_attn(_ptr(q_perm), _ptr(k_perm), _ptr(v_perm), _dtype(q_perm), _ptr(q_perm_idx),
                                      _ptr(q_offsets), Cq, _ptr(k_offsets), Ck, _ptr(k_means), _ptr(v_means),
                                      _ptr(mask), B, H, N, D, float(scale), _ptr(out),
                                      _ptr(lse if want_lse else None), _ptr(ws), ws.numel(), _stream(dev)))
    else:
        _dev(k_vars)
        _check("svgear_sparse_attn_var",
               lib.svgear_sparse_attn_var(_ptr(q_perm), _ptr(k_perm), _ptr(v_perm), _dtype(q_perm),
                                          _ptr(q_perm_idx), _ptr(q_offsets), Cq, _ptr(k_offsets), Ck,
                                          _ptr(k_means), _ptr(v_means), _ptr(k_vars), float(strength), _ptr(mask),
                                          B, H, N, D, float(scale), _ptr(out), _ptr(lse if want_lse else None),
                                          _ptr(ws), ws.numel(), _stream(dev)))
    return out, (lse if want_lse else None)


def sparse_attn_noalloc(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask,
                        scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None):
    """sparse_attn through the entry point that allocates nothing: its scratch
    is the library's static device array (calls that overlap on one GPU
    race).  ``out`` (and ``lse`` if wanted) are the caller's."""
    B, H, N, D = _dims4("q_perm", q_perm)
    _want("k_perm", k_perm, q_perm.dtype, (B, H, N, D), optional=False)
    _want("v_perm", v_perm, q_perm.dtype, (B, H, N, D), optional=False)
    _want("out", out, q_perm.dtype, (B, H, N, D), optional=False)
    Cq, Ck = _attn_tables(B, H, N, D, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out, q_perm.dtype,
                          lse)
    dev = _dev(q_perm, k_perm, v_perm, q_perm_idx, q_offsets, k_offsets, k_means, v_means, mask, out, lse)
    _check("svgear_sparse_attn_noalloc",
           load().svgear_sparse_attn_noalloc(_ptr(q_perm), _ptr(k_perm), _ptr(v_perm), _dtype(q_perm),
                                             _ptr(q_perm_idx), _ptr(q_offsets), Cq, _ptr(k_offsets), Ck,
                                             _ptr(k_means), _ptr(v_means), _ptr(mask), B, H, N, D, float(scale),
                                             _ptr(out), _ptr(lse), _stream(dev)))
    return out, lse


# ----------------------------------------------------------------------------
class Layer:
    """One SVG-EAR attention layer: k-means of Q and K, permuted copies and
    means, routing, sparse attention.  Buffers (including workspaces) are
    allocated once per shape and reused; the centroid tensors are the cache
    carried across denoising steps."""

    def __init__(self, B, H, N, D, Cq, Ck, dtype=torch.bfloat16, device="cuda"):
        dev = torch.device(device)
        self.shape = (B, H, N, D, Cq, Ck)
        lib = load()
        e = lambda *s, dt=torch.int32: torch.empty(s, dtype=dt, device=dev)
        self.lq, self.pq, self.oq = e(B, H, N), e(B, H, N), e(B, H, Cq + 1)
        self.lk, self.pk, self.ok = e(B, H, N), e(B, H, N), e(B, H, Ck + 1)
        self.qp, self.kp, self.vp = (e(B, H, N, D, dt=dtype) for _ in range(3))
        self.qm = e(B, H, Cq, D, dt=torch.float32)
        self.km = e(B, H, Ck, D, dt=torch.float32)
        self.vm = e(B, H, Ck, D, dt=torch.float32)
        self.mask = e(B, H, Cq, Ck, dt=torch.uint8)
        self.scores = e(B, H, Cq, Ck, dt=torch.float32)
        self.out = e(B, H, N, D, dt=dtype)
        need = max(lib.svgear_kmeans_workspace(B, H, N, D, Cq), lib.svgear_kmeans_workspace(B, H, N, D, Ck),
                   lib.svgear_centroids_workspace(B, H, N, D, max(Cq, Ck)),
                   lib.svgear_route_workspace(B, H, N, D, Cq, Ck),
                   lib.svgear_sparse_attn_workspace(B, H, N, D, Cq, Ck))
        self.ws = _workspace(need, dev)
        # k-means of Q and of K are independent: the K clustering runs on a
        # side stream with its own workspace
        self.ws_k = _workspace(lib.svgear_kmeans_workspace(B, H, N, D, Ck), dev)
        self.side = torch.cuda.Stream(device=dev)

    def forward(self, q, k, v, cq, ck, iters, density, scale=None, top_p=None, router="error", strength=0.0,
                fp8=False):
        """One layer.  Variants (default off): ``top_p`` routes under the SVG2
        top-p budget instead of ``density`` (``router`` "error": SVG-EAR spends
        the budget by error; "score": SVG2's own router); ``strength`` > 0
        adds the variance-corrected compensation (bf16); ``fp8`` runs the
        attention with e4m3 Q'/K'."""
        B, H, N, D, Cq, Ck = self.shape
        scale = 1.0 / math.sqrt(D) if scale is None else scale
        if router not in ("error", "score"):
            raise ValueError("router must be 'error' or 'score'")
        if fp8 and strength > 0.0:
            raise ValueError("the FP8 variant has no variance-corrected form")
        main = torch.cuda.current_stream(self.side.device)
        self.side.wait_stream(main)
        with torch.cuda.stream(self.side):
            kmeans(k, ck, iters, self.lk, self.pk, self.ok, ws=self.ws_k)
        kmeans(q, cq, iters, self.lq, self.pq, self.oq, ws=self.ws)
        # Q's permuted copy and means overlap the tail of K's clustering
        centroids(q, self.pq, self.oq, x_perm=self.qp, means=self.qm, ws=self.ws)
        main.wait_stream(self.side)
        centroids(k, self.pk, self.ok, x_perm=self.kp, means=self.km, ws=self.ws)
        centroids(v, self.pk, self.ok, x_perm=self.vp, means=self.vm, ws=self.ws)
        if top_p is None:
            route(self.qm, self.oq, self.kp, self.vp, self.km, self.vm, self.ok, scale, density, mask=self.mask,
                  scores=self.scores, ws=self.ws)
        else:
            _, _, _, m = route_topp(self.qm, self.oq, self.kp, self.vp, self.km, self.vm, self.ok, scale, top_p,
                                    error_ranked=(router == "error"), want_probs=False, want_budget=False,
                                    ws=self.ws)
            self.mask.copy_(m)
        if fp8:
            if not hasattr(self, "q8"):
                self.q8 = torch.empty(self.qp.shape, dtype=torch.uint8, device=self.qp.device)
                self.k8 = torch.empty_like(self.q8)
                self.qe = torch.empty((B, H), dtype=torch.int32, device=self.qp.device)
                self.ke = torch.empty_like(self.qe)
            quantize_fp8(self.qp, x8=self.q8, exps=self.qe)
            quantize_fp8(self.kp, x8=self.k8, exps=self.ke)
            sparse_attn_fp8(self.q8, self.qe, self.k8, self.ke, self.vp, self.pq, self.oq, self.ok, self.km,
                            self.vm, self.mask, scale, out=self.out, ws=self.ws)
        elif strength > 0.0:
            if not hasattr(self, "kv"):
                self.kv = torch.empty_like(self.km)
            centroid_variances(k, self.pk, self.ok, self.km, vars=self.kv, ws=self.ws)
            sparse_attn(self.qp, self.kp, self.vp, self.pq, self.oq, self.ok, self.km, self.vm, self.mask, scale,
                        out=self.out, ws=self.ws, k_vars=self.kv, strength=strength)
        else:
            sparse_attn(self.qp, self.kp, self.vp, self.pq, self.oq, self.ok, self.km, self.vm, self.mask, scale,
                        out=self.out, ws=self.ws)
        return self.out
