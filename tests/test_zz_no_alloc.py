"""fa_backward_noalloc (the backward with the library's static workspace, for callers that cannot
allocate) against fa_backward with a caller workspace: two calls in a row, the second with a smaller
problem than the first, through the C ABI.  The same kernels run on the same inputs with the same
workspace layout, so the results must be bitwise equal, which is stronger than the oracle bounds;
the first problem is also checked against the fp64 oracle.  The calls allocate no device memory."""
import pytest
import torch

import oracle
import workloads
from parity_util import check

pytestmark = pytest.mark.gpu


def _inputs(fa, B, H, N, d, dtype, causal, seqlens, seed):
    x = workloads.draw_custom(B, H, N, d, dtype=dtype, causal=causal, seqlens=seqlens, q_std=2.0, seed=seed)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    sl = None if seqlens is None else x["seqlens"].cuda()
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    fa.fa_forward(q, k, v, o, lse, x["scale"], causal, sl)
    return x, (q, k, v, o, do, lse), sl


def _grads(like):
    return [torch.full_like(like, float("nan")) for _ in range(3)]  # every element must be written


CASES = [  # a larger problem, then a smaller one, in one process
    [(2, 4, 1000, 128, "bf16", True, [1000, 613]), (1, 3, 300, 64, "bf16", False, None)],
    [(2, 2, 257, 64, "fp32", True, [257, 100]), (1, 1, 64, 128, "fp32", False, None)],
]


@pytest.mark.parametrize("seq", CASES)
def test_noalloc_backward_equals_fa_backward(fa, seq):
    for i, (B, H, N, d, dtype, causal, seqlens) in enumerate(seq):
        print(f"[no-alloc] call {i}: B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
        x, (q, k, v, o, do, lse), sl = _inputs(fa, B, H, N, d, dtype, causal, seqlens, seed=900 + i + N)
        ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d, q.dtype), dtype=torch.uint8, device="cuda")
        ref = _grads(q)
        fa.fa_backward(q, k, v, o, do, lse, *ref, x["scale"], causal, sl, ws)
        got = _grads(q)
        torch.cuda.synchronize()
        alloc0 = torch.cuda.memory_allocated()
        fa.fa_backward_noalloc(q, k, v, o, do, lse, *got, x["scale"], causal, sl)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == alloc0
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), (i, name)
        if i == 0:
            g = oracle.backward(x["q"], x["k"], x["v"], x["do"], x["scale"], causal, x["seqlens"])
            report, fails = [], []
            for name, a, r in zip(("dq", "dk", "dv"), got, g):
                fails += check(name, a.cpu(), r, q.dtype, name, report)
            print("\n".join(report), flush=True)
            assert not fails, fails


def test_noalloc_backward_allocates_nothing(fa):
    x, (q, k, v, o, do, lse), sl = _inputs(fa, 2, 4, 512, 128, "bf16", True, None, seed=77)
    got = _grads(q)
    fa.fa_backward_noalloc(q, k, v, o, do, lse, *got, x["scale"], True, None)  # resolves the workspace
    torch.cuda.synchronize()
    free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    for _ in range(3):
        fa.fa_backward_noalloc(q, k, v, o, do, lse, *got, x["scale"], True, None)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] == free0


def test_noalloc_rejects_a_problem_beyond_its_workspace(fa):
    q = torch.empty(1, 16, 65537, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, 16, 65537, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as ei:
        fa.fa_backward_noalloc(q, q, q, q, q, lse, q, q, q, 0.125, True)
    assert ei.value.status == 2 and "fa_backward" in str(ei.value)
