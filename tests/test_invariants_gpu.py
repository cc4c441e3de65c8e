"""Properties of the HIP path's outputs that need no oracle, checked at the workloads' full sizes.

Each follows from the definition of exact attention (NOTE-005: FlashAttention, "Concepts"; the
aicassindra page, "End-to-end flow", the exactness of the tiled result):
  - the rows of P = softmax(S) sum to one, which the stored LSE must reproduce: sum_j exp(S_ij - LSE_i) = 1;
  - each output row is a convex combination of the visible value rows, so every O_ic lies between the
    smallest and the largest V_jc over the visible keys j (and equals them when V is constant);
  - the row sums of dS vanish (sum_j P_ij (dP_ij - D_i) = D_i - D_i), hence sum_j dK_j = 0, and the
    columns of P carry dO through: sum_j dV_j = sum_i dO_i;
  - the scores depend on scale * q only: doubling q and halving the scale leaves every score, P, O, LSE,
    dK and dV unchanged and halves dQ.  Doubling a bf16 or fp32 value and halving an fp32 factor are
    exact, so the kernels' arithmetic reproduces this bit for bit.
"""
import pytest
import torch

import workloads
from parity_util import run_gpu

pytestmark = pytest.mark.gpu

BF16_WORKLOADS = [2, 3, 4]
LONG = BF16_WORKLOADS + [5]  # with N = 65536 (its gradient sums are checked beside its parity test)


def _say(msg):
    print(msg, flush=True)


def _visible(B, N, causal, seqlens, dev):
    """[B, N, N] bool: key j visible to query i."""
    j = torch.arange(N, device=dev)
    vis = torch.ones(B, N, N, dtype=torch.bool, device=dev)
    if causal:
        vis &= (j[None, :] <= j[:, None])[None]
    if seqlens is not None:
        L = seqlens.to(dev).clamp(0, N).long()
        vis &= (j[None, None, :] < L[:, None, None])
    return vis


@pytest.mark.parametrize("wid", LONG)
def test_rows_of_p_sum_to_one(fa, wid):
    """sum_j exp(S_ij - LSE_i) = 1 on sampled rows of every (b, h), S recomputed in fp32 from the
    bf16 inputs.  The kernel's LSE sums bf16-rounded probabilities: round to nearest with 8
    significant bits errs by at most 2^-8 relative per probability, hence in the sum (reached when one
    probability dominates a row, as with the peaked scores of q_std = 4); the scores, accumulated in
    another order, add ~1e-5: bound 2^-8 + 1e-4."""
    w = workloads.WORKLOADS[wid]
    x = workloads.draw(w)
    _say(f"[invariant] rows of P sum to one: workload {wid} {w.name}")
    got = run_gpu(fa, x, backward=False)
    dev = "cuda"
    q, k = x["q"].to(dev).float(), x["k"].to(dev).float()
    lse = got["lse"].to(dev)
    g = torch.Generator().manual_seed(11)
    rows = torch.randint(0, w.N, (48,), generator=g).to(dev)
    vis = _visible(w.B, w.N, w.causal, x["seqlens"], dev)[:, rows]  # [B, R, N]
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            s = (q[b, h, rows] @ k[b, h].T.contiguous()) * x["scale"]  # [R, N]
            s = s.masked_fill(~vis[b], float("-inf"))
            has = vis[b].any(1)
            tot = torch.exp(s[has] - lse[b, h, rows][has, None]).sum(1)
            worst = max(worst, float((tot - 1).abs().max()))
    _say(f"  max |sum_j P_ij - 1| = {worst:.3e}")
    assert worst <= 2.0 ** -8 + 1e-4


@pytest.mark.parametrize("wid", LONG)
def test_output_in_convex_hull(fa, wid):
    """min_j V_jc <= O_ic <= max_j V_jc over the visible keys j, up to O's bf16 rounding (half an ulp,
    2^-8 relative) and fp32 slack: the weights P_ij / l_i the kernel applies are an exact convex
    combination of its rounded probabilities."""
    w = workloads.WORKLOADS[wid]
    x = workloads.draw(w)
    _say(f"[invariant] O in the convex hull of the visible V rows: workload {wid} {w.name}")
    got = run_gpu(fa, x, backward=False)
    dev = "cuda"
    v = x["v"].to(dev).float()
    o = got["o"].to(dev).float()
    assert not (w.causal and x["seqlens"] is not None)  # (no workload combines the two)
    if w.causal:
        hi = torch.cummax(v, dim=2).values  # row i: max over keys 0..i
        lo = torch.cummin(v, dim=2).values
    else:
        L = x["seqlens"].to(dev).long() if x["seqlens"] is not None else torch.full((w.B,), w.N, device=dev)
        keep = torch.arange(w.N, device=dev)[None, :] < L[:, None]  # [B, N]
        big = torch.finfo(torch.float32).max
        hi = v.masked_fill(~keep[:, None, :, None], -big).amax(2, keepdim=True).expand_as(v)
        lo = v.masked_fill(~keep[:, None, :, None], big).amin(2, keepdim=True).expand_as(v)
    slack = torch.maximum(hi.abs(), lo.abs()) * 2.0 ** -8 + 1e-6
    over = torch.clamp(o - (hi + slack), min=0) + torch.clamp((lo - slack) - o, min=0)
    _say(f"  worst excursion beyond the hull: {float(over.max()):.3e} (rows inside: {float((over == 0).float().mean()):.6f})")
    assert float(over.max()) == 0.0


@pytest.mark.parametrize("wid", LONG)
def test_constant_values_give_constant_output(fa, wid):
    """V_j = v for every key j: O_i = v exactly in bf16 (the fp32 result differs from v by sums'
    rounding, ~1e-6 relative, far below half a bf16 ulp), and dS = P (dO.v - dO.O) vanishes up to
    that rounding, so dQ and dK are ~0 against dV."""
    w = workloads.WORKLOADS[wid]
    x = workloads.draw(w)
    vrow = x["v"][:, :, :1, :]
    x["v"] = vrow.expand_as(x["v"]).contiguous()
    _say(f"[invariant] constant V: workload {wid} {w.name}")
    got = run_gpu(fa, x)
    o, v = got["o"].float(), x["v"].float()
    mism = float((o != v).float().mean())
    _say(f"  O != v at a fraction {mism:.2e} of elements; max |O - v| = {float((o - v).abs().max()):.3e}")
    assert float((o - v).abs().max()) <= float(v.abs().max()) * 2.0 ** -8
    assert mism <= 1e-4
    ref = float(got["dv"].float().abs().max())
    dq, dk = float(got["dq"].float().abs().max()), float(got["dk"].float().abs().max())
    _say(f"  max |dQ| = {dq:.3e}, max |dK| = {dk:.3e}, max |dV| = {ref:.3e}")
    assert dq <= 1e-3 * ref and dk <= 1e-3 * ref


@pytest.mark.parametrize("wid", BF16_WORKLOADS)
def test_gradient_sums(fa, wid):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per (b, h) (every row sees at least one key), to
    1e-3 of the sums of magnitudes."""
    w = workloads.WORKLOADS[wid]
    x = workloads.draw(w)
    _say(f"[invariant] gradient sums: workload {wid} {w.name}")
    got = run_gpu(fa, x)
    dk_sum = got["dk"].double().sum(2)
    dv_sum = got["dv"].double().sum(2)
    do_sum = x["do"].double().sum(2)
    dk_mag = float(got["dk"].double().abs().sum(2).max())
    dv_mag = float(got["dv"].double().abs().sum(2).max() + x["do"].double().abs().sum(2).max())
    e_k = float(dk_sum.abs().max())
    e_v = float((dv_sum - do_sum).abs().max())
    _say(f"  max |sum dK| = {e_k:.3e} (of {dk_mag:.3e}); max |sum dV - sum dO| = {e_v:.3e} (of {dv_mag:.3e})")
    assert e_k <= 1e-3 * dk_mag and e_v <= 1e-3 * dv_mag


@pytest.mark.parametrize("wid", [1] + LONG)
def test_scale_folding_is_bitwise(fa, wid):
    """(2 q, scale / 2) against (q, scale): O, LSE, dK and dV bit for bit equal, dQ exactly halved."""
    w = workloads.WORKLOADS[wid]
    x = workloads.draw(w)
    _say(f"[invariant] scale folding: workload {wid} {w.name}")
    a = run_gpu(fa, x)
    y = dict(x)
    y["q"] = x["q"] * 2
    y["scale"] = x["scale"] / 2
    assert torch.equal(y["q"].float(), x["q"].float() * 2)  # exact in the input dtype
    b = run_gpu(fa, y)
    for name in ("o", "lse", "dk", "dv"):
        assert torch.equal(a[name], b[name]), name
    assert torch.equal(b["dq"].float() * 2, a["dq"].float()), "dq"


@pytest.mark.parametrize("wid", [3, 4])
def test_first_causal_row_copies_v(fa, wid):
    """Under the causal mask query 0 sees key 0 only: P_00 = 1, so O_0 = V_0 exactly and
    LSE_0 = scale q_0.k_0."""
    w = workloads.WORKLOADS[wid]
    x = workloads.draw(w)
    _say(f"[invariant] first causal row: workload {wid} {w.name}")
    got = run_gpu(fa, x, backward=False)
    assert torch.equal(got["o"][:, :, 0], x["v"][:, :, 0])
    s00 = (x["q"][:, :, 0].float() * x["k"][:, :, 0].float()).sum(-1) * x["scale"]
    assert float((got["lse"][:, :, 0] - s00).abs().max()) <= 1e-4 * (1 + float(s00.abs().max()))
