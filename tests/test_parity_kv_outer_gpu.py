"""GPU parity of the pages' K/V-outer schedule (fa_forward_kv_outer, the IO-complexity instrument):
the same O and LSE as the fp64 oracle for several LDS budgets (tile sizes), ragged N."""
import pytest
import torch

import oracle
import workloads
from parity_util import check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,d,lds", [(300, 64, 16 * 1024), (300, 128, 64 * 1024), (1000, 128, 128 * 1024),
                                     (257, 64, 128 * 1024), (1000, 64, 4 * 1024)])
def test_kv_outer_parity(fa, N, d, lds):
    print(f"[parity] K/V-outer schedule N={N} d={d} lds={lds}", flush=True)
    x = workloads.draw_custom(2, 2, N, d, dtype="bf16", q_std=2.0, seed=6000 + N + d)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(2, 2, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_forward_kv_outer_workspace_size(2, 2, N, d), dtype=torch.uint8, device="cuda")
    fa.fa_forward_kv_outer(q, k, v, o, lse, x["scale"], lds, ws)
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(x["q"], x["k"], x["v"], x["scale"])
    report, fails = [], []
    fails += check("o", o.cpu(), ro, torch.bfloat16, "o", report)
    fails += check("lse", lse.cpu(), rlse, torch.bfloat16, "lse", report)
    print("\n".join(report), flush=True)
    assert not fails, fails
