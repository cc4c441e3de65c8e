"""Seeded synthetic inputs for the exact-attention path.

This module only draws random numbers and names shapes; it contains none of
the attention arithmetic, so both the HIP path (through its tests and the
benchmark) and the fp64 oracle can take their inputs from it.

The five workloads take the attention shapes of the pages' benchmark settings
("Benchmark results" of the promptingindex FlashAttention page and "Key
results" of NOTE-005: BERT-large at sequence 512, GPT-2 at 1K, long-range arena
up to 4K, Path-256 at 64K).  No dataset is read: these seeded Gaussian tensors
stand in for those benchmarks.

Recipe (per workload):
  g = torch.Generator('cpu').manual_seed(seed)      # seed = workload number
  q, k, v, dO = torch.randn([B,H,N,d], generator=g, dtype=float32) in that order,
  q is multiplied by q_std; all four are rounded to the workload dtype (RNE).
  Then, in this order: key lengths (workload 2: randint in [256, 512]),
  sampled query rows and key rows per head (workload 5: randperm(N)[:256] each).
  scale = float32(1/sqrt(d)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp32" or "bf16"
    causal: bool
    padded: bool          # key-padding lengths drawn per batch element
    q_std: float = 1.0
    len_range: tuple = (0, 0)      # inclusive range of key lengths when padded
    n_sample: int = 0              # sampled query/key rows per head (0 = check everything)
    description: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return {"fp32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


WORKLOADS = {
    1: Workload(1, "tiny-exact", 1, 1, 128, 64, "fp32", False, False,
                description="tiny exact check, fp32, no mask"),
    2: Workload(2, "bert-large-encoder", 8, 16, 512, 64, "bf16", False, True, len_range=(256, 512),
                description="BERT-large-shaped encoder attention with key padding, lengths U{256..512}"),
    3: Workload(3, "gpt2-causal", 8, 12, 1024, 64, "bf16", True, False,
                description="GPT-2-shaped causal attention"),
    4: Workload(4, "long-causal-n4096-d128", 2, 16, 4096, 128, "bf16", True, False, q_std=4.0,
                description="long causal, d=128, q ~ N(0, 4^2) for high softmax dynamic range"),
    5: Workload(5, "very-long-n65536", 1, 8, 65536, 64, "bf16", False, False, n_sample=256,
                description="very long unmasked O(N)-memory stress, sampled rows checked"),
}


def draw(w: Workload, seed: int | None = None, device: str = "cpu"):
    """Draw the inputs of workload ``w``; returns a dict of tensors (inputs in the workload dtype).

    Keys: q, k, v, do ([B,H,N,d]), seqlens (int32 [B] or None), rows, keys
    (int64 [H, n_sample] per head, or None), scale, causal.
    """
    seed = w.id if seed is None else seed
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (w.B, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.q_std != 1.0:
        q = q * w.q_std
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32)
    dt = w.torch_dtype
    out = {"q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "do": do.to(dt)}
    seqlens = None
    if w.padded:
        lo, hi = w.len_range
        seqlens = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int32)
    rows = keys = None
    if w.n_sample:
        rows = torch.stack([torch.randperm(w.N, generator=g)[: w.n_sample] for _ in range(w.H)])
        keys = torch.stack([torch.randperm(w.N, generator=g)[: w.n_sample] for _ in range(w.H)])
    out.update(seqlens=seqlens, rows=rows, keys=keys, scale=w.scale, causal=w.causal)
    if device != "cpu":
        for name in ("q", "k", "v", "do"):
            out[name] = out[name].to(device)
        if seqlens is not None:
            out["seqlens_dev"] = seqlens.to(device)
    return out


def draw_custom(B, H, N, d, dtype="bf16", causal=False, seqlens=None, q_std=1.0, seed=0):
    """Inputs for an ad-hoc shape (tests: tails, edge cases).  Same draw order as ``draw``."""
    w = Workload(0, "custom", B, H, N, d, dtype, causal, False, q_std=q_std)
    out = draw(w, seed=seed)
    if seqlens is not None:
        out["seqlens"] = torch.as_tensor(seqlens, dtype=torch.int32)
    return out


def draw_block_mask(B, H, N, pattern="random", density=0.5, window=1, seed=0):
    """A [B, H, ceil(N/128), ceil(N/128)] uint8 block mask (1 = block visible) for block-sparse tests.

    pattern "random": each block visible with probability ``density`` (a seeded Bernoulli draw;
    some rows may end up with no visible block).  "local": query block i sees key blocks
    i-window .. i+window.  "local+global": "local" plus the first key block for every query block
    (and every key block for the first query block).  Only random numbers and index patterns.
    """
    nb = (N + 127) // 128
    if pattern == "random":
        g = torch.Generator("cpu").manual_seed(seed)
        m = (torch.rand((B, H, nb, nb), generator=g) < density).to(torch.uint8)
    else:
        i = torch.arange(nb)
        m = ((i[:, None] - i[None, :]).abs() <= window)
        if pattern == "local+global":
            m = m | (i[None, :] == 0) | (i[:, None] == 0)
        elif pattern != "local":
            raise ValueError(pattern)
        m = m.to(torch.uint8)[None, None].expand(B, H, nb, nb).contiguous()
    return m


def quantize_fp8(x: torch.Tensor):
    """Per-tensor OCP FP8 E4M3 quantisation for FP8-input tests: returns (x8, descale) with
    x8 = float8_e4m3fn(x / descale) and descale = max|x| / 448 (448: the largest E4M3 value)."""
    amax = float(x.abs().max())
    descale = amax / 448.0 if amax > 0 else 1.0
    return (x.float() / descale).to(torch.float8_e4m3fn), descale

