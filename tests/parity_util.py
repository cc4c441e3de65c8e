"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding, run the
oracle on the same seeded inputs, and compare with the stated tolerances.

Tolerances (fixed in the test, not tuned):
  float32 inputs:  max |x - x_ref| <= 1e-5 on O, LSE, dQ, dK, dV;
  bfloat16 inputs: max |x - x_ref| <= 2e-2 on O and LSE, and
                   relative RMS ||x - x_ref||_2 / ||x_ref||_2 <= 5e-3 on O, dQ, dK, dV.
The GPU output is promoted exactly to float64 before comparison.
"""
import math

import torch

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 5e-3


def max_abs(got, ref):
    got = got.double()
    fin = torch.isfinite(ref)
    if not torch.equal(torch.isfinite(got), fin):
        return math.inf
    if not torch.equal(got[~fin], ref[~fin]):
        return math.inf
    if fin.sum() == 0:
        return 0.0
    return float((got[fin] - ref[fin]).abs().max())


ZERO_REF_MAX_ABS = 1e-3  # a reference that is exactly zero (e.g. dQ with one key) is checked by max |x|


def rel_rms(got, ref):
    got = got.double()
    den = float(torch.linalg.vector_norm(ref))
    num = float(torch.linalg.vector_norm(got - ref))
    if den == 0.0:
        return 0.0 if float((got - ref).abs().max()) <= ZERO_REF_MAX_ABS else math.inf
    return num / den


def run_gpu(fa, x, backward=True, dev="cuda"):
    """Forward (and backward) of the HIP path on the inputs dict from workloads.draw* (with
    x["block_mask"], the block-sparse entry points; with x["dropout"] = (p, seed, offset), the dropout ones)."""
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    sl = x.get("seqlens")
    sl = None if sl is None else sl.to(dev)
    bm = x.get("block_mask")
    bm = None if bm is None else bm.to(dev)
    dr = x.get("dropout")  # (p, seed, offset)
    o, lse = fa.forward(q, k, v, x["scale"], x["causal"], sl, block_mask=bm, dropout=dr)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, x["scale"], x["causal"], sl, block_mask=bm, dropout=dr)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def check(name, got, ref, dtype, what, report, abs_scale=1.0):
    """Compare one tensor; append a line to `report`; return a list of failures.

    abs_scale multiplies the max-abs bounds: with dropout the result is the same arithmetic with the
    kept probabilities multiplied by 256/t, so its absolute errors scale by that factor (relative
    errors do not; LSE is undropped and keeps its bound)."""
    fails = []
    ma = max_abs(got, ref)
    rr = rel_rms(got, ref) if what != "lse" else float("nan")
    report.append(f"{name:>4}: max_abs={ma:.3e} rel_rms={rr:.3e}")
    tol_scale = 1.0 if what == "lse" else float(abs_scale)
    if dtype == torch.float32:
        if not ma <= F32_MAX_ABS * tol_scale:
            fails.append(f"{name} max_abs {ma:.3e} > {F32_MAX_ABS * tol_scale}")
    else:
        if what in ("o", "lse") and not ma <= BF16_MAX_ABS * tol_scale:
            fails.append(f"{name} max_abs {ma:.3e} > {BF16_MAX_ABS * tol_scale}")
        if what != "lse" and not rr <= BF16_REL_RMS:
            fails.append(f"{name} rel_rms {rr:.3e} > {BF16_REL_RMS}")
    return fails
