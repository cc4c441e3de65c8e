"""GPU parity of the FP8-input forward (fa_forward_fp8): OCP E4M3 Q, K, V with per-tensor descales
against the fp64 oracle on the dequantised inputs (descale * value, exact in fp64).  Every FP8
product is exact in fp32 and V converts exactly to bf16, so the result carries the same rounding
as the bf16 path and is held to the bf16 bounds of parity_util."""
import pytest
import torch

import oracle
import workloads
from parity_util import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,mask,q_std,scale", [(300, "none", 1.0, None), (1000, "causal", 4.0, None),
                                                (1000, "pad", 1.0, None), (4096, "causal", 4.0, None),
                                                (129, "causal+pad", 2.0, None), (300, "causal", 2.0, -0.2),
                                                (520, "pad", 2.0, -0.2)])
def test_fp8_forward_parity(fa, N, mask, q_std, scale):
    """scale < 0 selects the minimum-tracking form of the kernel (the running extreme of the raw
    products is a minimum)."""
    causal = "causal" in mask
    B, H, d = 2, 2, 128
    seqlens = [max(1, N // 2 + 3), max(1, N - 7)] if "pad" in mask else None
    x = workloads.draw_custom(B, H, N, d, dtype="fp32", causal=causal, seqlens=seqlens, q_std=q_std, seed=7000 + N)
    if scale is not None:
        x["scale"] = scale
    (q8, dq), (k8, dk), (v8, dv) = (workloads.quantize_fp8(x[n]) for n in ("q", "k", "v"))
    print(f"[parity] fp8 forward N={N} mask={mask} q_std={q_std} scale={x['scale']}", flush=True)
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    sl = None if seqlens is None else x["seqlens"].cuda()
    fa.fa_forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), dq, dk, dv, o, lse, x["scale"], causal, sl)
    torch.cuda.synchronize()
    deq = [t.to(torch.float64) * s for t, s in ((q8, dq), (k8, dk), (v8, dv))]
    ro, rlse = oracle.forward(*deq, x["scale"], causal, x["seqlens"])
    report, fails = [], []
    fails += check("o", o.cpu(), ro, torch.bfloat16, "o", report)
    fails += check("lse", lse.cpu(), rlse, torch.bfloat16, "lse", report)
    print("\n".join(report), flush=True)
    assert not fails, fails
