"""No-fallback check from a kernel trace: the GPU work of a forward and backward is exactly this
library's kernels (the aicassindra page, "End-to-end flow" and "The architecture: every piece
explained": the fused kernel must really run; the stackzen glossary entry: no silent fallback).

torch.profiler records every kernel the process launches, including those of libfa.so (launched
through the C ABI), so a fallback to any other implementation would show up as foreign kernels, and
a missing stage as an absent one.
"""
import pytest
import torch
from torch.profiler import ProfilerActivity, profile

import workloads

pytestmark = pytest.mark.gpu


def _kernels(fn):
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    names = {e.name for e in prof.events()}
    return {n for n in names if not n.startswith(("hip", "cuda"))}  # drop runtime API calls


CASES = [  # (d, causal, extra, one substring of each expected mangled kernel name: the template flags
    # are <d, causal, padded, negative scale, block-sparse, dropout, fp8> for the forward,
    # <d, causal, padded, block-sparse, dropout> for the dQ pass and the general dK/dV kernel, and
    # <causal, padded, dropout> for the K-in-LDS dK/dV kernel)
    (128, True, None, ["fwd_bf16_kernelILi128ELb1ELb0ELb0ELb0ELb0ELb0E", "bwd_dq_kernelILi128ELb1ELb0ELb0ELb0E",
                       "bwd_dkdv_kl_kernelILb1ELb0ELb0E"]),
    (128, False, "pad", ["fwd_bf16_kernelILi128ELb0ELb1ELb0ELb0ELb0ELb0E", "bwd_dq_kernelILi128ELb0ELb1ELb0ELb0E",
                         "bwd_dkdv_kl_kernelILb0ELb1ELb0E"]),
    (64, True, None, ["fwd_bf16_kernelILi64ELb1ELb0ELb0ELb0ELb0ELb0E", "bwd_dq_kernelILi64ELb1ELb0ELb0ELb0E",
                      "bwd_dkdv_kernelILi64ELb1ELb0ELb0ELb0E"]),
    (128, True, "dropout", ["fwd_bf16_kernelILi128ELb1ELb0ELb0ELb0ELb1ELb0E", "bwd_dq_kernelILi128ELb1ELb0ELb0ELb1E",
                            "bwd_dkdv_kl_kernelILb1ELb0ELb1E"]),
    (128, True, "sparse", ["fwd_bf16_kernelILi128ELb1ELb0ELb0ELb1ELb0ELb0E", "bwd_dq_kernelILi128ELb1ELb0ELb1ELb0E",
                           "bwd_dkdv_kernelILi128ELb1ELb0ELb1ELb0E"]),
]


@pytest.mark.parametrize("d,causal,extra,expected", CASES)
def test_only_library_kernels_run(fa, d, causal, extra, expected):
    N = 600
    x = workloads.draw_custom(2, 2, N, d, dtype="bf16", causal=causal, seqlens=[N, 411] if extra == "pad" else None,
                              seed=31)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    sl = None if x["seqlens"] is None else x["seqlens"].cuda()
    dr = (0.1, 5, 0) if extra == "dropout" else None
    bm = workloads.draw_block_mask(2, 2, N, "random", density=0.5, window=1, seed=1).cuda() if extra == "sparse" else None
    o, lse = fa.forward(q, k, v, x["scale"], causal, sl, block_mask=bm, dropout=dr)  # (outputs allocated outside)

    def step():
        fa.forward(q, k, v, x["scale"], causal, sl, block_mask=bm, dropout=dr)
        fa.backward(q, k, v, o, do, lse, x["scale"], causal, sl, block_mask=bm, dropout=dr)

    names = _kernels(step)
    print(f"[trace] d={d} causal={causal} {extra or 'dense'}: " + ", ".join(sorted(n[:60] for n in names)), flush=True)
    foreign = [n for n in names if not n.startswith("_ZN2fa")]
    assert not foreign, foreign
    for sub in expected:
        assert any(sub in n for n in names), (sub, names)
