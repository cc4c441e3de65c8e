"""GPU parity of fused dropout: the keep mask the library generates (fa_dropout_mask) equals the
oracle's Philox4x32-10 mask bit for bit, and the dropped forward and backward (fa_forward_dropout,
fa_backward_dropout) match the fp64 oracle given that mask, with the tolerances of parity_util.
p = 0 reproduces the dense kernels bit for bit."""
import pytest
import torch

import oracle
import workloads
from parity_util import check, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("B,H,N,p,seed,offset", [(1, 1, 64, 0.5, 0, 0), (2, 3, 100, 0.2, 0x123456789ABCDEF0, 9),
                                                 (1, 2, 257, 0.9, 42, 0xFFFFFFF0), (2, 1, 33, 0.0, 7, 1)])
def test_dropout_mask_bitwise(fa, B, H, N, p, seed, offset):
    _say(f"[parity] dropout mask B={B} H={H} N={N} p={p} seed={seed:#x} offset={offset}")
    keep = torch.empty(B, H, N, N, dtype=torch.uint8, device="cuda")
    fa.fa_dropout_mask(B, H, N, p, seed, offset, keep)
    torch.cuda.synchronize()
    want = oracle.dropout_keep(B, H, N, p, seed, offset)
    got = keep.cpu().bool()
    assert torch.equal(got, want), int((got != want).sum())


def _compare(x, got, report):
    p, seed, off = x["dropout"]
    B, H, N, _ = x["q"].shape
    keep = oracle.dropout_keep(B, H, N, p, seed, off)
    s = 256.0 / oracle.keep_threshold(p)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], x["scale"], x["causal"], x["seqlens"], keep=keep, keep_scale=s)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], x["scale"], x["causal"], x["seqlens"], keep=keep,
                                 keep_scale=s)
    fails = []
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        fails += check(name, got[name], ref, x["q"].dtype, name, report, abs_scale=s)
    return fails


CASES = [(300, 64, "none", "bf16", 0.2), (300, 128, "causal", "bf16", 0.5), (1000, 64, "causal+pad", "bf16", 0.1),
         (1000, 128, "pad", "bf16", 0.3), (129, 128, "causal", "bf16", 0.7), (1000, 128, "causal+pad", "bf16", 0.2),
         (500, 64, "causal", "bf16", 0.3), (500, 64, "pad", "bf16", 0.4), (700, 128, "none", "bf16", 0.15),
         (300, 64, "causal+pad", "fp32", 0.2),
         (200, 128, "none", "fp32", 0.5)]


@pytest.mark.parametrize("N,d,mask,dtype,p", CASES)
def test_dropout_parity(fa, N, d, mask, dtype, p):
    causal = "causal" in mask
    B, H = 2, 3
    seqlens = [max(1, N // 2 + 3), max(1, N - 7)] if "pad" in mask else None
    x = workloads.draw_custom(B, H, N, d, dtype=dtype, causal=causal, seqlens=seqlens, q_std=2.0, seed=5000 + N + d)
    x["dropout"] = (p, 0xC0FFEE + N, 3)
    _say(f"[parity] dropout N={N} d={d} mask={mask} {dtype} p={p}")
    got = run_gpu(fa, x)
    report = []
    fails = _compare(x, got, report)
    _say("\n".join(report))
    assert not fails, fails


def test_dropout_long_causal(fa):
    x = workloads.draw_custom(1, 2, 4096, 128, dtype="bf16", causal=True, q_std=4.0, seed=45)
    x["dropout"] = (0.1, 2024, 0)
    _say("[parity] dropout N=4096 d=128 causal p=0.1")
    got = run_gpu(fa, x)
    report = []
    fails = _compare(x, got, report)
    _say("\n".join(report))
    assert not fails, fails


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 128, False), ("bf16", 64, False),
                                           ("fp32", 64, True)])
def test_zero_dropout_is_dense_bitwise(fa, dtype, d, causal):
    x = workloads.draw_custom(2, 2, 333, d, dtype=dtype, causal=causal, seqlens=[333, 200], seed=6)
    dense = run_gpu(fa, x)
    x["dropout"] = (0.0, 99, 5)
    dropped = run_gpu(fa, x)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(dense[name], dropped[name]), name


def test_dropout_determinism_and_offsets(fa):
    x = workloads.draw_custom(2, 2, 500, 128, dtype="bf16", causal=True, seed=7)
    x["dropout"] = (0.3, 11, 0)
    a, b = run_gpu(fa, x), run_gpu(fa, x)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[name], b[name]), name
    x["dropout"] = (0.3, 11, 1)
    c = run_gpu(fa, x)
    assert not torch.equal(a["o"], c["o"]) and torch.equal(a["lse"], c["lse"])  # LSE is undropped


@pytest.mark.parametrize("d,dtype,causal", [(64, "bf16", True), (128, "bf16", True), (128, "bf16", False),
                                            (64, "fp32", True)])
def test_dropout_negative_scale(fa, d, dtype, causal):
    """A negative scale selects the kernels' minimum-tracking forms (the running extreme of the scores is
    a minimum of the raw products): the dropout forms of those must match the oracle too."""
    x = workloads.draw_custom(2, 2, 300, d, dtype=dtype, causal=causal, seqlens=[300, 211], q_std=2.0, seed=5100 + d)
    x["scale"] = -0.2
    x["dropout"] = (0.25, 0xBEEF + d, 2)
    _say(f"[parity] dropout scale=-0.2 N=300 d={d} {dtype} causal={causal}")
    got = run_gpu(fa, x)
    report = []
    fails = _compare(x, got, report)
    _say("\n".join(report))
    assert not fails, fails
