"""Pins of the oracle's block-sparse masking (no GPU).

The block mask restricts which 128 x 128 blocks of (query, key) pairs are visible; the pages
describe the block-sparse extension as the tiling applied to a sparse pattern (promptingindex
page, "Benchmark results: speed records without any approximation"; NOTE-005, "Key components").
Relative to its own mask the result is exact, so it has a plain definition, and these tests pin
the oracle's version of it against an independent construction: every query block attends,
densely and without any mask, to the concatenation of its visible key blocks only (torch.softmax
and autograd in fp64).
"""
import math

import pytest
import torch

import oracle
from workloads import draw_block_mask

F64 = torch.float64


def _inputs(B, H, N, d, seed, q_std=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=F64) * q_std
    k = torch.randn(B, H, N, d, generator=g, dtype=F64)
    v = torch.randn(B, H, N, d, generator=g, dtype=F64)
    do = torch.randn(B, H, N, d, generator=g, dtype=F64)
    return q, k, v, do


def _gathered(q, k, v, do, scale, bm, causal, lens):
    """O, LSE, dQ, dK, dV of the block-masked problem, one query block at a time: the block's rows
    attend to the keys of its visible key blocks only (gathered), with the causal/padding mask on
    the original indices; softmax from torch, gradients from autograd."""
    B, H, N, d = q.shape
    nb = (N + 127) // 128
    o = torch.zeros_like(q)
    lse = torch.full((B, H, N), -math.inf, dtype=F64)
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    for b in range(B):
        L = N if lens is None else lens[b]
        for h in range(H):
            for qb in range(nb):
                rows = torch.arange(qb * 128, min(N, qb * 128 + 128))
                kbs = [kb for kb in range(nb) if bm[b, h, qb, kb]]
                if not kbs:
                    continue
                keys = torch.cat([torch.arange(kb * 128, min(N, kb * 128 + 128)) for kb in kbs])
                vis = (keys[None, :] < L).expand(len(rows), len(keys)).clone()
                if causal:
                    vis &= keys[None, :] <= rows[:, None]
                qq = q[b, h, rows].clone().requires_grad_(True)
                kk = k[b, h, keys].clone().requires_grad_(True)
                vv = v[b, h, keys].clone().requires_grad_(True)
                s = (qq @ kk.T * scale).masked_fill(~vis, -math.inf)
                has = vis.any(1)
                p = torch.where(has[:, None], torch.softmax(torch.where(has[:, None], s, torch.zeros_like(s)), 1),
                                torch.zeros_like(s))
                p = torch.where(vis, p, torch.zeros_like(p))
                out = p @ vv
                (out * do[b, h, rows]).sum().backward()
                o[b, h, rows] = out.detach()
                lse[b, h, rows] = torch.where(has, torch.logsumexp(s.detach(), 1), torch.full_like(has, -math.inf, dtype=F64))
                dq[b, h, rows] += qq.grad
                dk[b, h, keys] += kk.grad
                dv[b, h, keys] += vv.grad
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("causal,padded", [(False, False), (True, False), (False, True), (True, True)])
def test_block_mask_equals_gathered_dense(causal, padded):
    B, H, N, d = 2, 2, 300, 4  # 3 blocks per side, the last one ragged
    q, k, v, do = _inputs(B, H, N, d, seed=11 + 2 * causal + padded, q_std=1.5)
    bm = draw_block_mask(B, H, N, "random", density=0.55, seed=3)
    bm[0, 0, 1] = 0  # one query block with no visible key block
    lens = [250, 129] if padded else None
    scale = 0.41
    o, lse = oracle.forward(q, k, v, scale, causal, lens, block_mask=bm)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, causal, lens, block_mask=bm)
    ro, rlse, rdq, rdk, rdv = _gathered(q, k, v, do, scale, bm, causal, lens)
    torch.testing.assert_close(o, ro, rtol=1e-12, atol=1e-13)
    assert torch.equal(torch.isinf(lse), torch.isinf(rlse))
    fin = torch.isfinite(rlse)
    torch.testing.assert_close(lse[fin], rlse[fin], rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(dq, rdq, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(dk, rdk, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(dv, rdv, rtol=1e-11, atol=1e-12)
    # the block row with nothing visible: O = 0, LSE = -inf, no gradient
    assert torch.all(o[0, 0, 128:256] == 0) and torch.all(torch.isinf(lse[0, 0, 128:256]))
    assert torch.all(dq[0, 0, 128:256] == 0)


def test_all_visible_block_mask_is_dense():
    B, H, N, d = 1, 2, 260, 8
    q, k, v, do = _inputs(B, H, N, d, seed=5)
    ones = torch.ones(B, H, 3, 3, dtype=torch.uint8)
    for causal in (False, True):
        a = oracle.forward(q, k, v, 0.3, causal, None)
        b = oracle.forward(q, k, v, 0.3, causal, None, block_mask=ones)
        assert all(torch.equal(x, y) for x, y in zip(a, b))
        a = oracle.backward(q, k, v, do, 0.3, causal, None)
        b = oracle.backward(q, k, v, do, 0.3, causal, None, block_mask=ones)
        assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_block_diagonal_mask_is_independent_blocks():
    """A block-diagonal mask splits the sequence into independent 128-token segments."""
    B, H, N, d = 1, 1, 384, 6
    q, k, v, do = _inputs(B, H, N, d, seed=9)
    bm = torch.eye(3, dtype=torch.uint8)[None, None]
    o, lse = oracle.forward(q, k, v, 0.5, False, None, block_mask=bm)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.5, False, None, block_mask=bm)
    for s in range(3):
        sl = slice(128 * s, 128 * s + 128)
        o_s, lse_s = oracle.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.5)
        g_s = oracle.backward(q[:, :, sl], k[:, :, sl], v[:, :, sl], do[:, :, sl], 0.5)
        torch.testing.assert_close(o[:, :, sl], o_s, rtol=1e-13, atol=1e-14)
        torch.testing.assert_close(lse[:, :, sl], lse_s, rtol=1e-13, atol=1e-14)
        for a, b in zip((dq, dk, dv), g_s):
            torch.testing.assert_close(a[:, :, sl], b, rtol=1e-12, atol=1e-13)


def test_block_mask_row_and_column_views():
    B, H, N, d = 1, 2, 290, 5
    q, k, v, do = _inputs(B, H, N, d, seed=21)
    bm = draw_block_mask(B, H, N, "local+global", window=0)
    o, lse = oracle.forward(q, k, v, 0.6, True, None, block_mask=bm)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.6, True, None, block_mask=bm)
    rows = torch.tensor([0, 127, 128, 200, 289])
    for h in range(H):
        o_r, lse_r = oracle.forward_rows(q, k, v, 0.6, True, None, 0, h, rows, block_mask=bm)
        torch.testing.assert_close(o_r, o[0, h, rows], rtol=1e-13, atol=1e-14)
        dq_r = oracle.backward_rows(q, k, v, do, 0.6, True, None, 0, h, rows, block_mask=bm)
        torch.testing.assert_close(dq_r, dq[0, h, rows], rtol=1e-12, atol=1e-13)
        lse_all, D_all = oracle.row_stats(q, k, v, do, 0.6, True, None, 0, h, chunk=64, block_mask=bm)
        dk_c, dv_c = oracle.backward_keys(q, k, v, do, 0.6, True, None, 0, h, rows, lse_all, D_all, block_mask=bm)
        torch.testing.assert_close(dk_c, dk[0, h, rows], rtol=1e-12, atol=1e-13)
        torch.testing.assert_close(dv_c, dv[0, h, rows], rtol=1e-12, atol=1e-13)


def test_block_mask_shape_is_checked():
    q, k, v, _ = _inputs(1, 1, 200, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, 0.5, False, None, block_mask=torch.ones(1, 1, 3, 3, dtype=torch.uint8))


# ---------------------------------------------------------------- planted mistakes are caught (CPU only)

import types  # noqa: E402

import oracle.attention as real  # noqa: E402

SRC = open(real.__file__).read()
MUTANTS = [
    ("transposed block index", "vis &= bm[(i // MASK_BLOCK)[:, None], (j // MASK_BLOCK)[None, :]]",
     "vis &= bm[(j // MASK_BLOCK)[None, :], (i // MASK_BLOCK)[:, None]]"),
    ("block size 64", "MASK_BLOCK = 128  #", "MASK_BLOCK = 64  #"),
    ("block mask dropped in the key view", "vis_t = visible(N, causal, L, blocks=blocks)[:, keys]",
     "vis_t = visible(N, causal, L)[:, keys]"),
    ("block row of the wrong head", "    return bm[b, h]\n", "    return bm[b, 0]\n"),
]


def _block_pins_fail(m) -> bool:
    B, H, N, d = 1, 2, 300, 4
    q, k, v, do = _inputs(B, H, N, d, seed=31)
    bm = draw_block_mask(B, H, N, "random", density=0.5, seed=8)
    try:
        o, lse = m.forward(q, k, v, 0.5, True, None, block_mask=bm)
        dq, dk, dv = m.backward(q, k, v, do, 0.5, True, None, block_mask=bm)
    except Exception:
        return True
    ro, rlse, rdq, rdk, rdv = _gathered(q, k, v, do, 0.5, bm, True, None)
    if not (torch.allclose(o, ro, atol=1e-12) and torch.allclose(dq, rdq, atol=1e-11)
            and torch.allclose(dk, rdk, atol=1e-11) and torch.allclose(dv, rdv, atol=1e-11)):
        return True
    rows = torch.tensor([0, 130, 299])
    for h in range(H):
        lse_a, D_a = m.row_stats(q, k, v, do, 0.5, True, None, 0, h, chunk=64, block_mask=bm)
        dk_c, dv_c = m.backward_keys(q, k, v, do, 0.5, True, None, 0, h, rows, lse_a, D_a, block_mask=bm)
        if not (torch.allclose(dk_c, dk[0, h, rows], atol=1e-11) and torch.allclose(dv_c, dv[0, h, rows], atol=1e-11)):
            return True
    return False


def _load(src, name):
    mod = types.ModuleType(name)
    mod.__file__ = real.__file__
    exec(compile(src, name, "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_block_pins():
    assert not _block_pins_fail(_load(SRC, "oracle_copy_bs"))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_block_mutant_is_caught(name, old, new):
    assert SRC.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    assert _block_pins_fail(_load(SRC.replace(old, new), "oracle_mutant_bs")), f"mutant '{name}' passed"
