"""Race check of the LDS rings with the FA_POISON_LDS debug build (libfa_poison.so, built beside
libfa.so by the same build step).

In that build every direct-to-LDS tile load first fills its destination with NaN words and waits for
that store.  A wave that read a stage before its transfer had landed, or after the stage had been
handed to the next tile, would then read NaN rather than plausible stale data.  The build also takes
its work items in reverse workgroup order (other compute units, another order, other neighbours).
With correct waits and barriers, and one writer per output element, the results are bitwise those
of the release build.  Every instantiation family that loads through LDS is run: the forward (dense,
causal, padded, dropout, block-sparse, FP8), the dQ pass and both dK/dV kernels (the K-in-LDS one at
d = 128, the general one at d = 64 and for block masks), at ragged sizes and at the long causal
workload's full size.
"""
import os

import pytest
import torch

import workloads
from parity_util import run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _poison_path(fa):
    path = os.path.join(os.path.dirname(os.path.abspath(fa.__file__)), "libfa_poison.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run exact_io_aware_66_amd/build.py (it builds both libraries)")
    return path


def _with(fa, path, fn):
    """fn() with the binding pointed at the library `path`, the release library restored after."""
    saved = fa._lib
    fa._lib = None
    try:
        fa.load(path)
        return fn()
    finally:
        fa._lib = saved


def _same(a, b, what):
    for name in a:
        assert torch.equal(a[name], b[name]), (what, name)
        assert not torch.isnan(b[name]).any(), (what, name, "NaN")


CASES = [  # (N, d, mask, extra)
    (1000, 128, "causal", None), (1000, 128, "causal+pad", None), (777, 128, "none", None),
    (1000, 64, "causal", None), (500, 64, "pad", None), (300, 64, "none", None),
    (1000, 128, "causal", "dropout"), (700, 64, "causal+pad", "dropout"),
    (1000, 128, "causal+pad", "sparse"), (600, 64, "none", "sparse"),
]


@pytest.mark.parametrize("N,d,mask,extra", CASES)
def test_poisoned_lds_gives_the_release_results(fa, N, d, mask, extra):
    path = _poison_path(fa)
    causal = "causal" in mask
    seqlens = [max(1, N // 2 + 3), max(1, N - 7)] if "pad" in mask else None
    x = workloads.draw_custom(2, 3, N, d, dtype="bf16", causal=causal, seqlens=seqlens, q_std=2.0, seed=8000 + N + d)
    if extra == "dropout":
        x["dropout"] = (0.2, 0xBADC0DE + N, 1)
    if extra == "sparse":
        x["block_mask"] = workloads.draw_block_mask(2, 3, N, "random", density=0.5, window=1, seed=N)
    _say(f"[poison] N={N} d={d} mask={mask} {extra or 'dense'}")
    rel = run_gpu(fa, x)
    poi = _with(fa, path, lambda: run_gpu(fa, x))
    _same(rel, poi, (N, d, mask, extra))


def test_poisoned_lds_long_causal_workload(fa):
    """The long causal workload at its full size (B = 2, H = 16, N = 4096, d = 128): the launch
    configuration the benchmark times, every workgroup order and ring depth of the real run."""
    path = _poison_path(fa)
    w = workloads.WORKLOADS[4]
    x = workloads.draw(w)
    _say(f"[poison] workload 4 {w.name}")
    rel = run_gpu(fa, x)
    poi = _with(fa, path, lambda: run_gpu(fa, x))
    _same(rel, poi, "workload 4")


def test_poisoned_lds_fp8_forward(fa):
    path = _poison_path(fa)
    B, H, N, d = 2, 2, 1000, 128
    x = workloads.draw_custom(B, H, N, d, dtype="fp32", causal=True, q_std=2.0, seed=8100)
    (q8, sq), (k8, sk), (v8, sv) = (workloads.quantize_fp8(x[n]) for n in ("q", "k", "v"))
    _say("[poison] fp8 forward N=1000 causal")

    def run():
        o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
        fa.fa_forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), sq, sk, sv, o, lse, x["scale"], True, None)
        torch.cuda.synchronize()
        return {"o": o.cpu(), "lse": lse.cpu()}

    rel = run()
    poi = _with(fa, path, run)
    _same(rel, poi, "fp8")
