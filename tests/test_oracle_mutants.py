"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins catch each one.

Each mutant is the oracle's source with one textual edit (a dropped term, a
flipped sign or index, a transposed operand), loaded as a separate module.
The check suite below uses only references that are independent of the oracle:
hand-worked values, torch's scaled_dot_product_attention and its autograd,
and internal consistency between the full and the row/column views.
"""
import json
import math
import os
import types

import pytest
import torch

import oracle.attention as real

SRC = open(real.__file__).read()
GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "handworked.json")))["cases"]

MUTANTS = [
    ("drop scale in scores", "s = torch.matmul(q, k.transpose(0, 1)) * scale", "s = torch.matmul(q, k.transpose(0, 1))"),
    ("flip causal direction", "vis &= j[None, :] <= i[:, None]", "vis &= j[None, :] >= i[:, None]"),
    ("padding off by one", "vis = (j[None, :] < L)", "vis = (j[None, :] <= L)"),
    ("drop max in LSE", "lse = m_safe + torch.log(l)", "lse = torch.log(l)"),
    ("transpose P in PV", "o[b, h] = torch.matmul(p, v[b, h])", "o[b, h] = torch.matmul(p.transpose(0, 1), v[b, h])"),
    ("sign of D", "            ds = p * (dp - D)\n", "            ds = p * (dp + D)\n"),
    ("drop scale in dQ", "dq[b, h] = torch.matmul(ds, k[b, h]) * scale", "dq[b, h] = torch.matmul(ds, k[b, h])"),
    ("transpose dS in dK", "dk[b, h] = torch.matmul(ds.transpose(0, 1), q[b, h]) * scale",
     "dk[b, h] = torch.matmul(ds, q[b, h]) * scale"),
    ("transpose P in dV", "dv[b, h] = torch.matmul(pz.transpose(0, 1), do[b, h])", "dv[b, h] = torch.matmul(pz, do[b, h])"),
    ("wrong D in row stats", "D[rows] = torch.sum(o_r * doh[rows], dim=1)", "D[rows] = torch.sum(o_r, dim=1)"),
    ("drop D in column view", "ds = p * (dp - _f64(D)[:, None])", "ds = p * dp"),
    ("dP uses Q in row view", "dp = torch.matmul(doh[rows], vh.transpose(0, 1))",
     "dp = torch.matmul(qh[rows], vh.transpose(0, 1))"),
]


def _load(src, name):
    mod = types.ModuleType(name)
    mod.__file__ = real.__file__
    exec(compile(src, name, "exec"), mod.__dict__)
    return mod


def _num(x):
    if isinstance(x, (int, float)):
        return float(x)
    env = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0), "inf": math.inf}
    return float(eval(x, {"__builtins__": {}}, env))


def _t(a):
    return torch.tensor([[_num(x) for x in row] for row in a], dtype=torch.float64)[None, None]


def _additive_mask(N, causal, L):
    j = torch.arange(N)
    bad = (j[None, :] >= L).expand(N, N).clone()
    if causal:
        bad |= j[None, :] > j[:, None]
    return torch.zeros(N, N, dtype=torch.float64).masked_fill(bad, -math.inf)


def pins_fail(m) -> list:
    """Run the independent pins against module ``m``; return the names of those that fail."""
    failed = []
    for c in GOLDEN:
        q, k, v, do = (_t(c[n]) for n in ("q", "k", "v", "do"))
        o, lse = m.forward(q, k, v, c["scale"], c["causal"], c["seqlens"])
        dq, dk, dv = m.backward(q, k, v, do, c["scale"], c["causal"], c["seqlens"])
        want_lse = torch.tensor([_num(x) for x in c["lse"]], dtype=torch.float64)[None, None]
        fin = torch.isfinite(want_lse)
        ok = (torch.allclose(o, _t(c["o"]), atol=1e-12) and torch.equal(torch.isfinite(lse), fin)
              and torch.allclose(lse[fin], want_lse[fin], atol=1e-12))
        for got, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            ok = ok and torch.allclose(got, _t(c[name]), atol=1e-12)
        if not ok:
            failed.append("handworked:" + c["name"])
    g = torch.Generator().manual_seed(0)
    B, H, N, d = 2, 2, 13, 4
    q, k, v, do = (torch.randn(B, H, N, d, generator=g, dtype=torch.float64) for _ in range(4))
    seqlens = torch.tensor([9, 13], dtype=torch.int32)
    for causal in (False, True):
        for sl in (None, seqlens):
            o, lse = m.forward(q, k, v, 0.6, causal, sl)
            dq, dk, dv = m.backward(q, k, v, do, 0.6, causal, sl)
            for b in range(B):
                L = N if sl is None else int(sl[b])
                qq, kk, vv = (x[b].clone().requires_grad_(True) for x in (q, k, v))
                ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=_additive_mask(N, causal, L),
                                                                       scale=0.6)
                ref.backward(do[b])
                if not torch.allclose(o[b], ref.detach(), atol=1e-11):
                    failed.append("sdpa")
                if not (torch.allclose(dq[b], qq.grad, atol=1e-10) and torch.allclose(dk[b], kk.grad, atol=1e-10)
                        and torch.allclose(dv[b], vv.grad, atol=1e-10)):
                    failed.append("autograd")
                for h in range(H):
                    rows = torch.tensor([0, 5, 12])
                    o_r, lse_r = m.forward_rows(q, k, v, 0.6, causal, sl, b, h, rows)
                    dq_r = m.backward_rows(q, k, v, do, 0.6, causal, sl, b, h, rows)
                    lse_a, D_a = m.row_stats(q, k, v, do, 0.6, causal, sl, b, h, chunk=5)
                    dk_c, dv_c = m.backward_keys(q, k, v, do, 0.6, causal, sl, b, h, rows, lse_a, D_a)
                    if not (torch.allclose(o_r, o[b, h, rows], atol=1e-12) and torch.allclose(dq_r, dq[b, h, rows], atol=1e-11)
                            and torch.allclose(lse_a, lse[b, h], atol=1e-12)
                            and torch.allclose(dk_c, dk[b, h, rows], atol=1e-11)
                            and torch.allclose(dv_c, dv[b, h, rows], atol=1e-11)):
                        failed.append("views")
    return sorted(set(failed))


def test_unmutated_oracle_passes_all_pins():
    assert pins_fail(_load(SRC, "oracle_copy")) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    assert SRC.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutant = _load(SRC.replace(old, new), "oracle_mutant")
    assert pins_fail(mutant), f"mutant '{name}' passed every pin"
