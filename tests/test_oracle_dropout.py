"""Pins of the oracle's dropout (no GPU): the Philox4x32-10 generator against its published
known-answer vectors, the keep-mask layout against a scalar element-by-element construction and
its keep rate, and the dropped attention with its gradients against torch softmax/autograd of the
explicit expression O = (softmax(S) * Z s) V.  Planted mistakes must fail at least one pin."""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as real_att
import oracle.philox as real_ph

F64 = torch.float64
KAT = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")))["cases"]


def _h(x):
    return [int(w, 16) for w in x]


@pytest.mark.parametrize("case", KAT, ids=lambda c: c["ctr"][0])
def test_philox_known_answers(case):
    out = oracle.philox4x32_10(*_h(case["ctr"]), *_h(case["key"]))
    assert [int(w) for w in out] == _h(case["out"])


def test_keep_mask_layout_against_scalar_construction():
    B, H, N, p, seed, off = 2, 2, 70, 0.35, 0xDEADBEEF12345, 7
    keep = oracle.dropout_keep(B, H, N, p, seed, off)
    t = oracle.keep_threshold(p)
    g = np.random.default_rng(0)
    for _ in range(300):
        b, h, i, j = int(g.integers(B)), int(g.integers(H)), int(g.integers(N)), int(g.integers(N))
        half, within = (j // 4) % 2, j % 32
        word, e = within // 8, within % 4
        out = oracle.philox4x32_10(i, j // 32, b * H + h, 2 * off + half, seed & 0xFFFFFFFF, seed >> 32)
        byte = (int(out[word]) >> (8 * e)) & 0xFF
        assert bool(keep[b, h, i, j]) == (byte < t), (b, h, i, j)


def test_keep_rate_and_threshold():
    assert oracle.keep_threshold(0.0) == 256 and oracle.keep_threshold(0.5) == 128
    with pytest.raises(ValueError):
        oracle.keep_threshold(0.999)
    keep = oracle.dropout_keep(1, 4, 256, 0.2, seed=99, offset=0)
    t = oracle.keep_threshold(0.2)
    n = keep.numel()
    rate = float(keep.float().mean())
    sd = math.sqrt(t / 256 * (1 - t / 256) / n)
    assert abs(rate - t / 256) < 5 * sd
    assert bool(oracle.dropout_keep(1, 1, 40, 0.0, 5, 3).all())
    # different offsets and seeds give different masks
    a = oracle.dropout_keep(1, 1, 64, 0.5, 1, 0)
    assert not torch.equal(a, oracle.dropout_keep(1, 1, 64, 0.5, 1, 1))
    assert not torch.equal(a, oracle.dropout_keep(1, 1, 64, 0.5, 2, 0))


def _explicit(q, k, v, do, scale, causal, lens, keep, s):
    """(softmax(S) * Z s) V and its autograd gradients, head by head (masked softmax from torch)."""
    B, H, N, d = q.shape
    o = torch.zeros_like(q)
    grads = [torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)]
    for b in range(B):
        L = N if lens is None else lens[b]
        vis = oracle.visible(N, causal, L)
        for h in range(H):
            qq, kk, vv = (x[b, h].clone().requires_grad_(True) for x in (q, k, v))
            sc = (qq @ kk.T * scale).masked_fill(~vis, -math.inf)
            has = vis.any(1)
            pr = torch.where(has[:, None], torch.softmax(torch.where(has[:, None], sc, torch.zeros_like(sc)), 1), 0.0)
            pr = torch.where(vis, pr, torch.zeros_like(pr))
            out = (pr * keep[b, h] * s) @ vv
            (out * do[b, h]).sum().backward()
            o[b, h] = out.detach()
            for gsum, x in zip(grads, (qq, kk, vv)):
                gsum[b, h] = x.grad
    return o, grads


def _inputs(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, H, N, d, generator=g, dtype=F64) * (1.5 if i == 0 else 1.0) for i in range(4)]


@pytest.mark.parametrize("causal,lens", [(False, None), (True, None), (True, [30, 17])])
def test_dropped_attention_against_autograd(causal, lens):
    B, H, N, d = 2, 2, 37, 5
    q, k, v, do = _inputs(B, H, N, d, seed=3)
    p = 0.3
    keep = oracle.dropout_keep(B, H, N, p, seed=77, offset=2)
    s = 256.0 / oracle.keep_threshold(p)
    o, lse = oracle.forward(q, k, v, 0.4, causal, lens, keep=keep, keep_scale=s)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.4, causal, lens, keep=keep, keep_scale=s)
    ro, (rdq, rdk, rdv) = _explicit(q, k, v, do, 0.4, causal, lens, keep, s)
    torch.testing.assert_close(o, ro, rtol=1e-12, atol=1e-13)
    torch.testing.assert_close(dq, rdq, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(dk, rdk, rtol=1e-11, atol=1e-12)
    torch.testing.assert_close(dv, rdv, rtol=1e-11, atol=1e-12)
    # LSE is that of the undropped scores
    _, lse0 = oracle.forward(q, k, v, 0.4, causal, lens)
    assert torch.equal(lse, lse0)


def test_keep_everything_is_dense():
    q, k, v, do = _inputs(1, 2, 50, 6, seed=4)
    keep = oracle.dropout_keep(1, 2, 50, 0.0, seed=1, offset=0)
    a = oracle.forward(q, k, v, 0.5, True, None)
    b = oracle.forward(q, k, v, 0.5, True, None, keep=keep, keep_scale=1.0)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    a = oracle.backward(q, k, v, do, 0.5, True, None)
    b = oracle.backward(q, k, v, do, 0.5, True, None, keep=keep, keep_scale=1.0)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


# ---------------------------------------------------------------- planted mistakes are caught (CPU only)

ATT_SRC = open(real_att.__file__).read()
PH_SRC = open(real_ph.__file__).read()
MUTANTS = [
    ("att", "scale of kept P dropped", "p = torch.where(z, p * float(keep_scale), torch.zeros_like(p))",
     "p = torch.where(z, p, torch.zeros_like(p))"),
    ("att", "dV from undropped P", "dv[b, h] = torch.matmul(pz.transpose(0, 1), do[b, h])",
     "dv[b, h] = torch.matmul(p.transpose(0, 1), do[b, h])"),
    ("att", "dP not masked", "                dp = torch.where(z, dp * float(keep_scale), torch.zeros_like(dp))\n",
     "                pass\n"),
    ("att", "D from dropped P", "torch.zeros_like(dp))\n            D = torch.sum(p * dp, dim=1, keepdim=True)",
     "torch.zeros_like(dp))\n            D = torch.sum(pz * dp, dim=1, keepdim=True)"),
    ("ph", "hi and lo swapped", "c = [(p1 >> np.uint64(32)) ^ c[1] ^ k[0], p1 & MASK32,",
     "c = [(p1 & MASK32) ^ c[1] ^ k[0], p1 >> np.uint64(32),"),
    ("ph", "key not bumped", "k = [(k[0] + W0) & MASK32, (k[1] + W1) & MASK32]", "k = [k[0], k[1]]"),
    ("ph", "nine rounds", "for _ in range(10):", "for _ in range(9):"),
    ("ph", "halves of the key block swapped", "full = byte.transpose(0, 1, 3, 2, 4).reshape(N, nb * 32)",
     "full = byte.reshape(N, nb * 32)"),
    ("ph", "threshold compare inverted", "keep[b, hh] = torch.from_numpy(full[:, :N] < t)",
     "keep[b, hh] = torch.from_numpy(full[:, :N] >= 256 - t)"),
]


def _load(src, name, file):
    mod = types.ModuleType(name)
    mod.__file__ = file
    exec(compile(src, name, "exec"), mod.__dict__)
    return mod


def _pins_fail(att, ph) -> bool:
    for c in KAT:
        if [int(w) for w in ph.philox4x32_10(*_h(c["ctr"]), *_h(c["key"]))] != _h(c["out"]):
            return True
    B, H, N, d = 1, 2, 40, 4
    keep = ph.dropout_keep(B, H, N, 0.3, seed=5, offset=1)
    t = ph.keep_threshold(0.3)
    for (b, h, i, j) in [(0, 0, 3, 5), (0, 1, 39, 38), (0, 1, 17, 12), (0, 0, 8, 36), (0, 1, 22, 29), (0, 0, 0, 0)]:
        half, within = (j // 4) % 2, j % 32
        out = real_ph.philox4x32_10(i, j // 32, b * H + h, 2 + half, 5, 0)
        if bool(keep[b, h, i, j]) != (((int(out[within // 8]) >> (8 * (within % 4))) & 0xFF) < t):
            return True
    q, k, v, do = _inputs(B, H, N, d, seed=8)
    s = 256.0 / t
    o, _ = att.forward(q, k, v, 0.4, True, None, keep=keep, keep_scale=s)
    g = att.backward(q, k, v, do, 0.4, True, None, keep=keep, keep_scale=s)
    ro, rg = _explicit(q, k, v, do, 0.4, True, None, keep, s)
    if not torch.allclose(o, ro, atol=1e-12):
        return True
    return not all(torch.allclose(a, b, atol=1e-11) for a, b in zip(g, rg))


def test_unmutated_oracle_passes_dropout_pins():
    assert not _pins_fail(_load(ATT_SRC, "att_copy", real_att.__file__), _load(PH_SRC, "ph_copy", real_ph.__file__))


@pytest.mark.parametrize("where,name,old,new", MUTANTS, ids=[m[1] for m in MUTANTS])
def test_dropout_mutant_is_caught(where, name, old, new):
    src = ATT_SRC if where == "att" else PH_SRC
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    src = src.replace(old, new)
    att = _load(src if where == "att" else ATT_SRC, "att_m", real_att.__file__)
    ph = _load(src if where == "ph" else PH_SRC, "ph_m", real_ph.__file__)
    assert _pins_fail(att, ph), f"mutant '{name}' passed"
