"""GPU parity of block-sparse attention: the HIP path (fa_forward_block_sparse and
fa_backward_block_sparse through the binding) against the fp64 oracle with the same block mask,
element by element, with the tolerances of parity_util; plus structural checks (an all-visible
mask reproduces the dense kernels bit for bit, an all-hidden mask gives O = 0 and LSE = -inf)."""
import pytest
import torch

import oracle
import workloads
from parity_util import check, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _compare(x, got, report):
    bm = x["block_mask"]
    o, lse = oracle.forward(x["q"], x["k"], x["v"], x["scale"], x["causal"], x["seqlens"], block_mask=bm)
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], x["scale"], x["causal"], x["seqlens"], block_mask=bm)
    fails = []
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        fails += check(name, got[name], ref, x["q"].dtype, name, report)
    return fails


CASES = [  # (N, d, mask, dtype, pattern)
    (300, 64, "none", "bf16", "random"), (300, 128, "causal", "bf16", "random"),
    (1000, 64, "causal+pad", "bf16", "random"), (1000, 128, "pad", "bf16", "random"),
    (1000, 128, "causal", "bf16", "local+global"), (700, 64, "causal", "bf16", "local"),
    (1000, 128, "causal+pad", "bf16", "random"), (500, 64, "pad", "bf16", "random"), (700, 128, "none", "bf16", "random"),
    (300, 64, "causal+pad", "fp32", "random"), (260, 128, "none", "fp32", "random"),
]


@pytest.mark.parametrize("N,d,mask,dtype,pattern", CASES)
def test_block_sparse_parity(fa, N, d, mask, dtype, pattern):
    causal = "causal" in mask
    B, H = 2, 3
    seqlens = [max(1, N // 2 + 3), max(1, N - 7)] if "pad" in mask else None
    x = workloads.draw_custom(B, H, N, d, dtype=dtype, causal=causal, seqlens=seqlens, q_std=2.0, seed=4000 + N + d)
    bm = workloads.draw_block_mask(B, H, N, pattern, density=0.5, window=1, seed=N + d)
    bm[1, 2, -1] = 0  # the last query block of one head sees nothing
    x["block_mask"] = bm
    _say(f"[parity] block-sparse N={N} d={d} mask={mask} {dtype} {pattern} ({int(bm.sum())}/{bm.numel()} blocks)")
    got = run_gpu(fa, x)
    report = []
    fails = _compare(x, got, report)
    _say("\n".join(report))
    assert not fails, fails
    rows = slice(128 * (bm.shape[-1] - 1), N)
    assert torch.all(got["o"][1, 2, rows] == 0) and torch.all(torch.isneginf(got["lse"][1, 2, rows]))
    assert torch.all(got["dq"][1, 2, rows] == 0)


def test_block_sparse_long_causal_local(fa):
    """The long-sequence shape (N=4096, d=128, causal, bf16) with a local window of 3 blocks plus a
    global first block, one batch element and two heads against the full oracle."""
    x = workloads.draw_custom(1, 2, 4096, 128, dtype="bf16", causal=True, q_std=4.0, seed=44)
    x["block_mask"] = workloads.draw_block_mask(1, 2, 4096, "local+global", window=1)
    _say("[parity] block-sparse N=4096 d=128 causal local+global")
    got = run_gpu(fa, x)
    report = []
    fails = _compare(x, got, report)
    _say("\n".join(report))
    assert not fails, fails


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 128, False), ("bf16", 64, False),
                                           ("fp32", 64, True)])
def test_all_visible_mask_is_the_dense_result_bitwise(fa, dtype, d, causal):
    N = 520
    x = workloads.draw_custom(2, 2, N, d, dtype=dtype, causal=causal, seqlens=[N, 301], seed=8)
    dense = run_gpu(fa, x)
    x["block_mask"] = torch.ones(2, 2, 5, 5, dtype=torch.uint8)
    sparse = run_gpu(fa, x)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(dense[name], sparse[name]), name


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_all_hidden_mask(fa, dtype):
    x = workloads.draw_custom(1, 2, 300, 64, dtype=dtype, causal=False, seed=2)
    x["block_mask"] = torch.zeros(1, 2, 3, 3, dtype=torch.uint8)
    got = run_gpu(fa, x)
    assert torch.all(got["o"] == 0) and torch.all(torch.isneginf(got["lse"]))
    for g in ("dq", "dk", "dv"):
        assert torch.all(got[g] == 0), g


def test_block_sparse_determinism(fa):
    x = workloads.draw_custom(2, 2, 777, 128, dtype="bf16", causal=True, seed=3)
    x["block_mask"] = workloads.draw_block_mask(2, 2, 777, "random", density=0.6, seed=1)
    runs = [run_gpu(fa, x) for _ in range(2)]
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(runs[0][name], runs[1][name]), name


@pytest.mark.parametrize("d,dtype,causal", [(64, "bf16", True), (128, "bf16", True), (128, "bf16", False),
                                            (64, "fp32", False)])
def test_block_sparse_negative_scale(fa, d, dtype, causal):
    """A negative scale selects the kernels' minimum-tracking forms; their block-sparse forms against the
    oracle with the same mask."""
    N = 520
    x = workloads.draw_custom(2, 2, N, d, dtype=dtype, causal=causal, seqlens=[N, 333], q_std=2.0, seed=4100 + d)
    x["scale"] = -0.2
    x["block_mask"] = workloads.draw_block_mask(2, 2, N, "random", density=0.6, seed=d + 1)
    _say(f"[parity] block-sparse scale=-0.2 N={N} d={d} {dtype} causal={causal}")
    got = run_gpu(fa, x)
    report = []
    fails = _compare(x, got, report)
    _say("\n".join(report))
    assert not fails, fails
