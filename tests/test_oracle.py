"""Pins for the fp64 oracle, independent of the oracle's own code.

Every check here compares the oracle with something other than itself:
hand-worked values, closed forms, a scalar streaming (online-softmax)
computation, torch's own scaled_dot_product_attention and autograd, central
finite differences, and invariants that the definition implies.  None of them
needs a GPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import draw_custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.json")
MASKS = [dict(causal=False, lens=None), dict(causal=True, lens=None),
         dict(causal=False, lens="pad"), dict(causal=True, lens="pad")]


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    env = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0), "inf": math.inf}
    return float(eval(x, {"__builtins__": {}}, env))


def _t(a):
    return torch.tensor([[_num(x) for x in row] for row in a], dtype=torch.float64)[None, None]


def _rand(B, H, N, d, seed, causal=False, lens=None, q_std=1.0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float64) * q_std
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    do = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    seqlens = None
    if lens == "pad":
        seqlens = torch.randint(1, N + 1, (B,), generator=g, dtype=torch.int32)
    return q, k, v, do, seqlens


# ---------------------------------------------------------------- hand-worked values

@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_handworked(case):
    q, k, v, do = (_t(case[n]) for n in ("q", "k", "v", "do"))
    seqlens = case["seqlens"]
    o, lse = oracle.forward(q, k, v, case["scale"], case["causal"], seqlens)
    dq, dk, dv = oracle.backward(q, k, v, do, case["scale"], case["causal"], seqlens)
    torch.testing.assert_close(o, _t(case["o"]), rtol=0, atol=1e-14)
    want_lse = torch.tensor([_num(x) for x in case["lse"]], dtype=torch.float64)[None, None]
    assert torch.equal(torch.isinf(lse), torch.isinf(want_lse))
    fin = torch.isfinite(want_lse)
    torch.testing.assert_close(lse[fin], want_lse[fin], rtol=0, atol=1e-14)
    for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        torch.testing.assert_close(got, _t(case[name]), rtol=0, atol=1e-14, msg=name)


# ---------------------------------------------------------------- streaming (online softmax) brute force

def _streaming_row(qi, keys_vals, scale):
    """One query row by the online-softmax recurrence, one key at a time, in scalar Python.

    The recurrence is the page's (running max m, running normaliser l, output
    rescaled whenever the max grows); it is a different algorithm from the
    oracle's materialised softmax, so agreement pins both.
    """
    d = len(keys_vals[0][1]) if keys_vals else 0
    m, l, acc = -math.inf, 0.0, [0.0] * d
    for kj, vj in keys_vals:
        s = scale * math.fsum(a * b for a, b in zip(qi, kj))
        m_new = max(m, s)
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        p = math.exp(s - m_new)
        l = l * alpha + p
        acc = [a * alpha + p * x for a, x in zip(acc, vj)]
        m = m_new
    if l == 0.0:
        return [0.0] * len(acc), -math.inf
    return [a / l for a in acc], m + math.log(l)


@pytest.mark.parametrize("N", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("mk", range(4))
def test_streaming_bruteforce(N, d, mk):
    mask = MASKS[mk]
    q, k, v, do, seqlens = _rand(2, 2, N, d, seed=100 * N + 10 * d + mk, lens=mask["lens"])
    scale = 0.7
    o, lse = oracle.forward(q, k, v, scale, mask["causal"], seqlens)
    for b in range(2):
        L = N if seqlens is None else int(seqlens[b])
        for h in range(2):
            for i in range(N):
                kv = [(k[b, h, j].tolist(), v[b, h, j].tolist()) for j in range(N)
                      if j < L and (not mask["causal"] or j <= i)]
                o_ref, lse_ref = _streaming_row(q[b, h, i].tolist(), kv, scale)
                assert np.allclose(o[b, h, i].numpy(), o_ref, rtol=1e-12, atol=1e-13)
                assert math.isclose(float(lse[b, h, i]), lse_ref, rel_tol=1e-12, abs_tol=1e-13)


# ---------------------------------------------------------------- library routines

def _additive_mask(N, causal, L):
    m = torch.zeros(N, N, dtype=torch.float64)
    j = torch.arange(N)
    bad = (j[None, :] >= L).expand(N, N).clone()
    if causal:
        bad |= j[None, :] > j[:, None]
    return m.masked_fill(bad, -math.inf)


@pytest.mark.parametrize("mk", range(4))
@pytest.mark.parametrize("N,d", [(7, 3), (33, 16), (64, 64)])
def test_against_torch_sdpa(N, d, mk):
    mask = MASKS[mk]
    q, k, v, do, seqlens = _rand(2, 3, N, d, seed=N * d + mk, lens=mask["lens"], q_std=2.0)
    scale = 1.0 / math.sqrt(d)
    o, _ = oracle.forward(q, k, v, scale, mask["causal"], seqlens)
    for b in range(2):
        L = N if seqlens is None else int(seqlens[b])
        am = _additive_mask(N, mask["causal"], L)
        ref = torch.nn.functional.scaled_dot_product_attention(q[b], k[b], v[b], attn_mask=am, scale=scale)
        torch.testing.assert_close(o[b], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mk", range(4))
def test_backward_against_autograd_of_sdpa(mk):
    mask = MASKS[mk]
    N, d = 19, 8
    q, k, v, do, seqlens = _rand(2, 2, N, d, seed=7 + mk, lens=mask["lens"])
    scale = 0.37
    dq, dk, dv = oracle.backward(q, k, v, do, scale, mask["causal"], seqlens)
    for b in range(2):
        L = N if seqlens is None else int(seqlens[b])
        qq, kk, vv = (x[b].clone().requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=_additive_mask(N, mask["causal"], L), scale=scale)
        out.backward(do[b])
        torch.testing.assert_close(dq[b], qq.grad, rtol=1e-11, atol=1e-12)
        torch.testing.assert_close(dk[b], kk.grad, rtol=1e-11, atol=1e-12)
        torch.testing.assert_close(dv[b], vv.grad, rtol=1e-11, atol=1e-12)


def test_lse_against_scipy_logsumexp():
    from scipy.special import logsumexp
    q, k, v, _, _ = _rand(1, 2, 40, 8, seed=3, q_std=6.0)
    scale = 0.5
    _, lse = oracle.forward(q, k, v, scale, causal=True)
    for h in range(2):
        s = (q[0, h].numpy() @ k[0, h].numpy().T) * scale
        for i in range(40):
            assert math.isclose(float(lse[0, h, i]), float(logsumexp(s[i, : i + 1])), rel_tol=1e-13, abs_tol=1e-13)


# ---------------------------------------------------------------- closed forms

def test_single_key():
    q, k, v, _, _ = _rand(1, 2, 1, 5, seed=11)
    o, lse = oracle.forward(q, k, v, 0.3)
    torch.testing.assert_close(o, v, rtol=0, atol=1e-15)
    torch.testing.assert_close(lse, 0.3 * (q * k).sum(-1), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("mk", range(4))
def test_zero_query_is_mean_of_visible_values(mk):
    mask = MASKS[mk]
    N = 9
    _, k, v, _, seqlens = _rand(2, 1, N, 4, seed=12 + mk, lens=mask["lens"])
    q = torch.zeros(2, 1, N, 4, dtype=torch.float64)
    o, lse = oracle.forward(q, k, v, 1.0, mask["causal"], seqlens)
    for b in range(2):
        L = N if seqlens is None else int(seqlens[b])
        for i in range(N):
            n_vis = min(L, i + 1) if mask["causal"] else L
            torch.testing.assert_close(o[b, 0, i], v[b, 0, :n_vis].mean(0), rtol=1e-13, atol=1e-14)
            assert math.isclose(float(lse[b, 0, i]), math.log(n_vis), rel_tol=1e-14, abs_tol=1e-15)


def test_two_keys_sigmoid():
    q, k, v, _, _ = _rand(1, 1, 2, 3, seed=13)
    scale = 0.8
    o, lse = oracle.forward(q, k, v, scale)
    for i in range(2):
        s1 = scale * float(q[0, 0, i] @ k[0, 0, 0])
        s2 = scale * float(q[0, 0, i] @ k[0, 0, 1])
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        torch.testing.assert_close(o[0, 0, i], w1 * v[0, 0, 0] + w2 * v[0, 0, 1], rtol=1e-13, atol=1e-14)
        assert math.isclose(float(lse[0, 0, i]), max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))), rel_tol=1e-13)


def test_causal_row0():
    q, k, v, _, _ = _rand(2, 2, 6, 4, seed=14)
    o, lse = oracle.forward(q, k, v, 0.5, causal=True)
    torch.testing.assert_close(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)
    torch.testing.assert_close(lse[:, :, 0], 0.5 * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- invariants of the forward

@pytest.mark.parametrize("mk", range(4))
def test_probabilities_sum_to_one_and_convex_hull(mk):
    mask = MASKS[mk]
    N, d = 23, 6
    q, k, v, _, seqlens = _rand(2, 2, N, d, seed=20 + mk, lens=mask["lens"], q_std=3.0)
    scale = 0.41
    o, lse = oracle.forward(q, k, v, scale, mask["causal"], seqlens)
    for b in range(2):
        L = N if seqlens is None else int(seqlens[b])
        for h in range(2):
            for i in range(N):
                vis = [j for j in range(N) if j < L and (not mask["causal"] or j <= i)]
                total = math.fsum(math.exp(scale * float(q[b, h, i] @ k[b, h, j]) - float(lse[b, h, i])) for j in vis)
                assert abs(total - 1.0) < 1e-12
                lo = v[b, h, vis].min(0).values - 1e-12
                hi = v[b, h, vis].max(0).values + 1e-12
                assert bool(((o[b, h, i] >= lo) & (o[b, h, i] <= hi)).all())


def test_constant_values_give_constant_output():
    q, k, _, _, _ = _rand(1, 2, 17, 5, seed=30, q_std=4.0)
    v = torch.full((1, 2, 17, 5), 2.5, dtype=torch.float64)
    for causal in (False, True):
        o, _ = oracle.forward(q, k, v, 1.0, causal)
        torch.testing.assert_close(o, v, rtol=0, atol=1e-13)


def test_key_permutation_and_query_permutation():
    q, k, v, _, _ = _rand(1, 1, 15, 4, seed=31)
    o, lse = oracle.forward(q, k, v, 0.6)
    pk = torch.randperm(15, generator=torch.Generator().manual_seed(1))
    o2, lse2 = oracle.forward(q, k[:, :, pk], v[:, :, pk], 0.6)
    torch.testing.assert_close(o2, o, rtol=1e-13, atol=1e-14)
    torch.testing.assert_close(lse2, lse, rtol=1e-14, atol=1e-14)
    pq = torch.randperm(15, generator=torch.Generator().manual_seed(2))
    o3, lse3 = oracle.forward(q[:, :, pq], k, v, 0.6)
    torch.testing.assert_close(o3, o[:, :, pq], rtol=1e-13, atol=1e-14)
    torch.testing.assert_close(lse3, lse[:, :, pq], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("mk", range(4))
def test_key_shift_invariance(mk):
    mask = MASKS[mk]
    q, k, v, _, seqlens = _rand(2, 1, 12, 3, seed=40 + mk, lens=mask["lens"])
    u = torch.tensor([0.5, -1.0, 2.0], dtype=torch.float64)
    scale = 0.9
    o, lse = oracle.forward(q, k, v, scale, mask["causal"], seqlens)
    o2, lse2 = oracle.forward(q, k + u, v, scale, mask["causal"], seqlens)
    torch.testing.assert_close(o2, o, rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(lse2, lse + scale * (q @ u), rtol=1e-12, atol=1e-12)


def test_causality_and_padding_ignore_hidden_keys():
    q, k, v, _, _ = _rand(1, 1, 10, 4, seed=50)
    o, lse = oracle.forward(q, k, v, 1.0, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 6:] += 5.0
    v2[:, :, 6:] -= 3.0
    o2, lse2 = oracle.forward(q, k2, v2, 1.0, causal=True)
    torch.testing.assert_close(o2[:, :, :6], o[:, :, :6], rtol=0, atol=0)
    torch.testing.assert_close(lse2[:, :, :6], lse[:, :, :6], rtol=0, atol=0)
    assert not torch.allclose(o2[:, :, 6:], o[:, :, 6:])
    o3, lse3 = oracle.forward(q, k, v, 1.0, seqlens=[4])
    k4 = torch.cat([k[:, :, :4], k[:, :, 4:] * 3 + 1], 2)     # change only the padded keys
    v4 = torch.cat([v[:, :, :4], v[:, :, 4:] + 9], 2)
    o4, lse4 = oracle.forward(q, k4, v4, 1.0, seqlens=[4])
    torch.testing.assert_close(o4, o3, rtol=0, atol=0)
    torch.testing.assert_close(lse4, lse3, rtol=0, atol=0)


def test_seqlens_clamped_and_empty_rows():
    q, k, v, do, _ = _rand(3, 1, 5, 2, seed=51)
    o, lse = oracle.forward(q, k, v, 1.0, seqlens=[-3, 0, 99])
    assert torch.all(o[:2] == 0) and torch.all(torch.isneginf(lse[:2]))
    o_full, lse_full = oracle.forward(q[2:], k[2:], v[2:], 1.0)
    torch.testing.assert_close(o[2:], o_full, rtol=0, atol=0)
    dq, dk, dv = oracle.backward(q, k, v, do, 1.0, seqlens=[-3, 0, 99])
    for g in (dq, dk, dv):
        assert torch.all(g[:2] == 0)


# ---------------------------------------------------------------- backward: finite differences and identities

@pytest.mark.parametrize("mk", range(4))
def test_backward_central_differences(mk):
    mask = MASKS[mk]
    N, d = 6, 3
    q, k, v, do, seqlens = _rand(1, 1, N, d, seed=60 + mk, lens=mask["lens"])
    scale = 0.77
    dq, dk, dv = oracle.backward(q, k, v, do, scale, mask["causal"], seqlens)
    eps = 1e-6

    def loss(qq, kk, vv):
        o, _ = oracle.forward(qq, kk, vv, scale, mask["causal"], seqlens)
        return float((o * do).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        fd = torch.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.clone(), k.clone(), v.clone()]
            args_m = [q.clone(), k.clone(), v.clone()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = float((fd - grad).abs().max())
        assert err <= 1e-6 * max(1.0, float(grad.abs().max())), (which, err)


@pytest.mark.parametrize("mk", range(4))
def test_backward_exact_identities(mk):
    mask = MASKS[mk]
    N, d = 21, 5
    q, k, v, do, seqlens = _rand(2, 2, N, d, seed=70 + mk, lens=mask["lens"], q_std=2.0)
    scale = 0.45
    o, lse = oracle.forward(q, k, v, scale, mask["causal"], seqlens)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, mask["causal"], seqlens)
    # rows of dS sum to zero => sum_j dK_j = 0
    torch.testing.assert_close(dk.sum(2), torch.zeros_like(dk.sum(2)), rtol=0, atol=1e-12)
    # rows of P sum to one (every row has a visible key here) => sum_j dV_j = sum_i dO_i
    torch.testing.assert_close(dv.sum(2), do.sum(2), rtol=1e-12, atol=1e-12)
    # sum_i <q_i, dQ_i> = sum_j <k_j, dK_j>  (both equal scale * sum dS * (Q Kᵀ))
    torch.testing.assert_close((q * dq).sum((2, 3)), (k * dk).sum((2, 3)), rtol=1e-11, atol=1e-12)
    # sum_j <v_j, dV_j> = sum_i <dO_i, O_i>
    torch.testing.assert_close((v * dv).sum((2, 3)), (do * o).sum((2, 3)), rtol=1e-12, atol=1e-12)
    if seqlens is not None:
        for b in range(2):
            L = int(seqlens[b])
            assert torch.all(dk[b, :, L:] == 0) and torch.all(dv[b, :, L:] == 0)
    if mask["causal"]:
        assert torch.all(dq[:, :, 0] == 0)


# ---------------------------------------------------------------- row / column views agree with the full oracle

@pytest.mark.parametrize("mk", range(4))
def test_row_and_column_views(mk):
    mask = MASKS[mk]
    N, d = 40, 8
    q, k, v, do, seqlens = _rand(2, 2, N, d, seed=80 + mk, lens=mask["lens"])
    scale = 0.35
    o, lse = oracle.forward(q, k, v, scale, mask["causal"], seqlens)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, mask["causal"], seqlens)
    rows = torch.tensor([0, 3, 17, 39])
    for b in range(2):
        for h in range(2):
            o_r, lse_r = oracle.forward_rows(q, k, v, scale, mask["causal"], seqlens, b, h, rows)
            torch.testing.assert_close(o_r, o[b, h, rows], rtol=1e-13, atol=1e-14)
            torch.testing.assert_close(lse_r, lse[b, h, rows], rtol=1e-13, atol=1e-14)
            dq_r = oracle.backward_rows(q, k, v, do, scale, mask["causal"], seqlens, b, h, rows)
            torch.testing.assert_close(dq_r, dq[b, h, rows], rtol=1e-12, atol=1e-13)
            lse_all, D_all = oracle.row_stats(q, k, v, do, scale, mask["causal"], seqlens, b, h, chunk=7)
            torch.testing.assert_close(lse_all, lse[b, h], rtol=1e-13, atol=1e-14)
            dk_c, dv_c = oracle.backward_keys(q, k, v, do, scale, mask["causal"], seqlens, b, h, rows, lse_all, D_all)
            torch.testing.assert_close(dk_c, dk[b, h, rows], rtol=1e-12, atol=1e-13)
            torch.testing.assert_close(dv_c, dv[b, h, rows], rtol=1e-12, atol=1e-13)


def test_bf16_inputs_are_promoted_exactly():
    w = draw_custom(1, 1, 16, 8, dtype="bf16", seed=5)
    o, lse = oracle.forward(w["q"], w["k"], w["v"], w["scale"])
    o2, lse2 = oracle.forward(w["q"].double(), w["k"].double(), w["v"].double(), w["scale"])
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
