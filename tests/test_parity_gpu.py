"""GPU parity: the HIP path (through the C-ABI binding) against the fp64 oracle, element by element,
on the seeded workloads and on ragged, masked and degenerate edge cases."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity_util import check, run_gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
from make_workload5_keys import input_digest  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _compare_full(x, got, report):
    o, lse = oracle.forward(x["q"], x["k"], x["v"], x["scale"], x["causal"], x["seqlens"])
    dq, dk, dv = oracle.backward(x["q"], x["k"], x["v"], x["do"], x["scale"], x["causal"], x["seqlens"])
    dt = x["q"].dtype
    fails = []
    for name, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        if name in got:
            fails += check(name, got[name], ref, dt, name, report)
    return fails


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_workload_full(fa, wid):
    w = workloads.WORKLOADS[wid]
    _say(f"[parity] workload {wid} {w.name} B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype} causal={w.causal}")
    x = workloads.draw(w)
    got = run_gpu(fa, x)
    report = []
    fails = _compare_full(x, got, report)
    _say("\n".join(report))
    assert not fails, fails


def test_workload5_sampled(fa):
    w = workloads.WORKLOADS[5]
    _say(f"[parity] workload 5 {w.name} sampled rows and keys, all {w.H} heads")
    x = workloads.draw(w)
    # dK, dV on the sampled keys need LSE and D of all 65536 rows of each head: a complete fp64 oracle
    # pass per head, stored once by tests/golden/make_workload5_keys.py (keyed to the inputs' digest)
    gold = np.load(os.path.join(GOLDEN, "workload5_keys.npz"))
    assert str(gold["digest"]) == input_digest(x), "stored oracle values were made from other inputs"
    assert np.array_equal(gold["keys"], x["keys"].numpy())
    got = run_gpu(fa, x)
    report, fails = [], []
    dt = x["q"].dtype
    o_ref, lse_ref, dq_ref, o_got, lse_got, dq_got = [], [], [], [], [], []
    for h in range(w.H):
        rows = x["rows"][h]
        o_r, lse_r = oracle.forward_rows(x["q"], x["k"], x["v"], x["scale"], False, None, 0, h, rows)
        dq_r = oracle.backward_rows(x["q"], x["k"], x["v"], x["do"], x["scale"], False, None, 0, h, rows)
        o_ref.append(o_r); lse_ref.append(lse_r); dq_ref.append(dq_r)
        o_got.append(got["o"][0, h, rows]); lse_got.append(got["lse"][0, h, rows]); dq_got.append(got["dq"][0, h, rows])
    fails += check("o", torch.stack(o_got), torch.stack(o_ref), dt, "o", report)
    fails += check("lse", torch.stack(lse_got), torch.stack(lse_ref), dt, "lse", report)
    fails += check("dq", torch.stack(dq_got), torch.stack(dq_ref), dt, "dq", report)
    keys = x["keys"]
    dk_got = torch.stack([got["dk"][0, h, keys[h]] for h in range(w.H)])
    dv_got = torch.stack([got["dv"][0, h, keys[h]] for h in range(w.H)])
    fails += check("dk", dk_got, torch.from_numpy(gold["dk"]), dt, "dk", report)
    fails += check("dv", dv_got, torch.from_numpy(gold["dv"]), dt, "dv", report)
    # properties at full size, every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (every row sees a key)
    dk_sum = got["dk"].double().sum(2)
    dv_sum = got["dv"].double().sum(2)
    do_sum = x["do"].double().sum(2)
    scale_ref = float(got["dk"].double().abs().sum(2).max())
    report.append(f"sum dK: max {float(dk_sum.abs().max()):.3e} (sum |dK| {scale_ref:.3e}); "
                  f"sum dV - sum dO: max {float((dv_sum - do_sum).abs().max()):.3e}")
    assert float(dk_sum.abs().max()) <= 1e-3 * scale_ref
    assert float((dv_sum - do_sum).abs().max()) <= 1e-3 * float(do_sum.abs().max() + got["dv"].double().abs().sum(2).max())
    _say("\n".join(report))
    assert not fails, fails


def test_long_causal_d128_sampled(fa):
    """N = 16384, d = 128, causal, q_std = 4 (the long-sequence shape at the larger head size: 64 key
    blocks of 256 per head, each with its diagonal tiles): O, LSE and dQ on sampled rows, dK and dV on
    sampled keys (their oracle needs LSE and D of all 16384 rows, one fp64 pass per head, computed
    here), block edges included."""
    N, H = 16384, 2
    x = workloads.draw_custom(1, H, N, 128, dtype="bf16", causal=True, q_std=4.0, seed=16384)
    _say(f"[parity] long causal N={N} d=128 H={H}: sampled rows and keys")
    got = run_gpu(fa, x)
    g = torch.Generator().manual_seed(5)
    edges = [0, 1, 31, 32, 255, 256, 257, 4095, 4096, N - 257, N - 256, N - 2, N - 1]
    pick = lambda: torch.unique(torch.cat([torch.tensor(edges), torch.randint(0, N, (51,), generator=g)]))
    dt = x["q"].dtype
    report, fails = [], []
    for h in range(H):
        rows, keys = pick(), pick()
        o_r, lse_r = oracle.forward_rows(x["q"], x["k"], x["v"], x["scale"], True, None, 0, h, rows)
        dq_r = oracle.backward_rows(x["q"], x["k"], x["v"], x["do"], x["scale"], True, None, 0, h, rows)
        lse, D = oracle.row_stats(x["q"], x["k"], x["v"], x["do"], x["scale"], True, None, 0, h, chunk=2048)
        dk_r, dv_r = oracle.backward_keys(x["q"], x["k"], x["v"], x["do"], x["scale"], True, None, 0, h, keys, lse, D)
        for name, gt, ref in (("o", got["o"][0, h, rows], o_r), ("lse", got["lse"][0, h, rows], lse_r),
                              ("dq", got["dq"][0, h, rows], dq_r), ("dk", got["dk"][0, h, keys], dk_r),
                              ("dv", got["dv"][0, h, keys], dv_r)):
            fails += check(f"{name}[h{h}]", gt[None], ref[None], dt, name, report)
    _say("\n".join(report))
    assert not fails, fails


TAILS = [1, 17, 100, 129, 300, 1000]


@pytest.mark.parametrize("N", TAILS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "pad", "causal+pad"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_tails_and_masks(fa, N, d, mask, dtype):
    causal = "causal" in mask
    B, H = 2, 3
    seqlens = None
    if "pad" in mask:
        seqlens = [max(1, N // 2 + 3), max(1, N - 7)]
    x = workloads.draw_custom(B, H, N, d, dtype=dtype, causal=causal, seqlens=seqlens, q_std=2.0, seed=1000 + N + d)
    _say(f"[parity] tail N={N} d={d} mask={mask} {dtype}")
    got = run_gpu(fa, x)
    report = []
    fails = _compare_full(x, got, report)
    if fails:
        _say("\n".join(report))
    assert not fails, fails


@pytest.mark.parametrize("d", [64, 128])
def test_empty_and_clamped_lengths(fa, d):
    N = 150
    x = workloads.draw_custom(4, 2, N, d, dtype="bf16", causal=False, seqlens=[0, N + 40, -3, 1], seed=77)
    _say(f"[parity] lengths 0, N+40, -3, 1 d={d}")
    got = run_gpu(fa, x)
    for b in (0, 2):  # no visible key at all
        assert torch.all(got["o"][b] == 0) and torch.all(torch.isneginf(got["lse"][b]))
        for g in ("dq", "dk", "dv"):
            assert torch.all(got[g][b] == 0), g
    report = []
    fails = _compare_full(x, got, report)
    assert not fails, (fails, report)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.3])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["causal", "pad", "none"])
def test_unusual_scales(fa, scale, d, mask):
    """scale < 0 selects the minimum-tracking forms of the forward (every mask form); scale 0 gives
    uniform weights over the visible keys."""
    seqlens = [137] if mask == "pad" else None
    x = workloads.draw_custom(1, 2, 300, d, dtype="bf16", causal=mask == "causal", seqlens=seqlens, seed=5)
    x["scale"] = scale
    _say(f"[parity] scale={scale} d={d} N=300 mask={mask}")
    got = run_gpu(fa, x)
    report = []
    fails = _compare_full(x, got, report)
    assert not fails, (fails, report)


def test_high_dynamic_range_rescaling(fa):
    # scores up to |S| ~ 40 move the running maximum across many key tiles
    x = workloads.draw_custom(1, 4, 1500, 128, dtype="bf16", causal=True, q_std=8.0, seed=9)
    _say("[parity] q_std=8, N=1500, d=128 causal")
    got = run_gpu(fa, x)
    report = []
    fails = _compare_full(x, got, report)
    _say("\n".join(report))
    assert not fails, fails


@pytest.mark.parametrize("d,extra", [(128, None), (64, None), (128, "dropout"), (64, "sparse")])
def test_determinism(fa, d, extra):
    """20 runs bitwise identical (single writer per element, fixed summation order)."""
    x = workloads.draw_custom(2, 4, 777, d, dtype="bf16", causal=True, seed=3)
    if extra == "dropout":
        x["dropout"] = (0.1, 77, 0)
    if extra == "sparse":
        x["block_mask"] = workloads.draw_block_mask(2, 4, 777, "random", density=0.5, window=1, seed=3)
    _say(f"[parity] determinism x20 d={d} {extra or 'dense'}")
    first = run_gpu(fa, x)
    for _ in range(19):
        r = run_gpu(fa, x)
        for name in ("o", "lse", "dq", "dk", "dv"):
            assert torch.equal(r[name], first[name]), name


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_backward_stages(fa, dtype):
    """prepare + dkdv + dq equals fa_backward bitwise, in either order of the last two, whatever the
    workspace held before; so does dq_prepare + dkdv, whose workspace equals the prepare stage's."""
    x = workloads.draw_custom(2, 3, 300, 128, dtype=dtype, causal=True, seqlens=[300, 171], seed=5)
    _say(f"[parity] backward stages {dtype}")
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    sl = x["seqlens"].cuda()
    B, H, N, d = q.shape
    o, lse = torch.empty_like(q), torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    fa.fa_forward(q, k, v, o, lse, x["scale"], True, sl)
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d, q.dtype), dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(q) for _ in range(3)]
    fa.fa_backward(q, k, v, o, do, lse, *ref, x["scale"], True, sl, ws)
    for order in ("dkdv_first", "dq_first"):
        ws.fill_(0xFF)  # NaN patterns everywhere: stages must not read what they did not write
        dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)
        fa.fa_backward_prepare(o, do, lse, ws)
        if order == "dq_first":
            fa.fa_backward_dq(q, k, v, do, lse, dq, x["scale"], True, sl, ws)
        fa.fa_backward_dkdv(q, k, v, do, lse, dk, dv, x["scale"], True, sl, ws)
        if order == "dkdv_first":
            fa.fa_backward_dq(q, k, v, do, lse, dq, x["scale"], True, sl, ws)
        torch.cuda.synchronize()
        for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            assert torch.equal(got, want), (order, name)
    # the dQ pass with the prepare stage folded in leaves the prepare stage's workspace, bitwise, and
    # with the dK/dV pass after it gives fa_backward's results
    ws.fill_(0xFF)
    fa.fa_backward_prepare(o, do, lse, ws)
    torch.cuda.synchronize()
    ws_prepared = ws.clone()
    ws.fill_(0xFF)
    dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)
    fa.fa_backward_dq_prepare(q, k, v, o, do, lse, dq, x["scale"], True, sl, ws)
    torch.cuda.synchronize()
    assert torch.equal(ws, ws_prepared), "workspace after fa_backward_dq_prepare"
    fa.fa_backward_dkdv(q, k, v, do, lse, dk, dv, x["scale"], True, sl, ws)
    torch.cuda.synchronize()
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert torch.equal(got, want), ("dq_prepare", name)


def test_no_device_allocation(fa):
    x = workloads.draw_custom(2, 4, 512, 64, dtype="bf16", causal=True, seed=4)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = torch.empty_like(q), torch.empty(2, 4, 512, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_size(2, 4, 512, 64, torch.bfloat16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        fa.fa_forward(q, k, v, o, lse, x["scale"], True)
        fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, x["scale"], True, None, ws)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] == free0


@pytest.mark.parametrize("B,H,N,causal", [(1, 40, 1000, True), (1, 40, 1000, False), (2, 36, 500, True),
                                          (2, 16, 4096, True)])
def test_dkdv_batched_equals_per_head(fa, B, H, N, causal):
    """O, LSE, dQ, dK and dV of a many-head problem (several blocks per compute unit, XCD-grouped
    order) equal bit for bit those of each head run as a problem of its own (a different grid and
    workgroup order): each block's result depends only on its own inputs.  Head (0, 0) is also
    checked against the oracle."""
    x = workloads.draw_custom(B, H, N, 128, dtype="bf16", causal=causal, seed=2000 + N + H)
    _say(f"[parity] dK/dV batched vs per head B={B} H={H} N={N} causal={causal}")
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = torch.empty_like(q), torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    fa.fa_forward(q, k, v, o, lse, x["scale"], causal)
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, 128, q.dtype), dtype=torch.uint8, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, x["scale"], causal, None, ws)
    ws1 = torch.empty(fa.fa_backward_workspace_size(1, 1, N, 128, q.dtype), dtype=torch.uint8, device="cuda")
    for b in range(B):
        for h in range(H):
            sl = [t[b:b + 1, h:h + 1].contiguous() for t in (q, k, v, o, do)]
            o1, lse1 = torch.empty_like(sl[0]), torch.empty(1, 1, N, dtype=torch.float32, device="cuda")
            fa.fa_forward(*sl[:3], o1, lse1, x["scale"], causal)
            torch.cuda.synchronize()
            assert torch.equal(o1[0, 0], o[b, h]), ("o", b, h)
            assert torch.equal(lse1[0, 0], lse[b, h]), ("lse", b, h)
            g = [torch.empty_like(sl[0]) for _ in range(3)]
            fa.fa_backward(*sl, lse[b:b + 1, h:h + 1].contiguous(), *g, x["scale"], causal, None, ws1)
            torch.cuda.synchronize()
            assert torch.equal(g[0][0, 0], dq[b, h]), ("dq", b, h)
            assert torch.equal(g[1][0, 0], dk[b, h]), ("dk", b, h)
            assert torch.equal(g[2][0, 0], dv[b, h]), ("dv", b, h)
    one = {n: x[n][:1, :1] for n in ("q", "k", "v", "do")}
    one.update(scale=x["scale"], causal=causal, seqlens=None)
    report = []
    fails = _compare_full(one, {"dk": dk[:1, :1].cpu(), "dv": dv[:1, :1].cpu()}, report)
    _say("\n".join(report))
    assert not fails, fails
