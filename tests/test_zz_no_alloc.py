"""The allocation-free attention entry point (static device scratch) against
the workspace entry point through the C ABI: bitwise equal outputs and LSE
on two calls in a row, the second with a smaller input, for bf16 and fp32,
and a refused size beyond the scratch limit."""
import numpy as np
import pytest
import torch

from synth.gen import WORKLOADS, layer_inputs, scaled
from tests.helpers import f32, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import sparse_attention_video_amd as pkg
    pkg.load()
    assert torch.cuda.is_available()
    return pkg


def layer_state(sv, dtype, B, H, N, D, Cq, Ck, seed):
    """Permuted tensors, tables and a routed mask from the library's own layer."""
    w = scaled(WORKLOADS["tiny"], B=B, H=H, N=N, D=D, dtype=dtype, comps=24, zipf=1.1, Cq=Cq, Ck=Ck, seed=seed,
               density=0.3)
    x = layer_inputs(w)
    r = lambda a: a.reshape(B, H, *a.shape[1:])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    L = sv.Layer(B, H, N, D, Cq, Ck, dtype=tdt)
    L.forward(to_dev(r(x["q"]), dtype), to_dev(r(x["k"]), dtype), to_dev(r(x["v"]), dtype), f32(r(x["cq0"])),
              f32(r(x["ck0"])), 3, 0.3, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    return L


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_noalloc_matches_workspace_entry_point(sv, dtype, D):
    sizes = [(1, 3, 5000, 16, 53, 3), (1, 2, 3000, 9, 40, 4)]   # second call smaller
    for B, H, N, Cq, Ck, seed in sizes:
        print(f"noalloc {dtype} D={D}: B={B} H={H} N={N} Cq={Cq} Ck={Ck}", flush=True)
        L = layer_state(sv, dtype, B, H, N, D, Cq, Ck, seed)
        sc = 1.0 / np.sqrt(D)
        args = (L.qp, L.kp, L.vp, L.pq, L.oq, L.ok, L.km, L.vm, L.mask)
        ref, ref_lse = sv.sparse_attn(*args, sc, want_lse=True)
        out = torch.full_like(ref, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        sv.sparse_attn_noalloc(*args, sc, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(lse, ref_lse)


def test_noalloc_refuses_sizes_beyond_its_scratch(sv):
    lib = sv.load()
    need = lib.svgear_sparse_attn_workspace(1, 200, 75600, 128, 100, 500)
    assert need > (32 << 20)
    F = __import__("ctypes").c_void_p(0x1000)
    st = lib.svgear_sparse_attn_noalloc(F, F, F, 0, F, F, 100, F, 500, F, F, F, 1, 200, 75600, 128,
                                        __import__("ctypes").c_float(0.088), F, None, None)
    assert st == sv.svgear.ERR_INVALID_ARG
    assert "scratch" in lib.svgear_last_error().decode()
