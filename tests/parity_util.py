"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding, run the
oracle on the same seeded inputs, and compare with the stated tolerances.

Tolerances (fixed in the test, not tuned):
  float32 inputs:  max |x - x_ref| <= 1e-5 on LSE, and <= 1e-5 max(1, max |x_ref|) on O, dQ, dK, dV
                   (exactly 1e-5 for the tiny fp32 workload, whose outputs all stay below 0.9 in
                   magnitude; fp32 rounding error grows with the values, so for the larger gradients
                   of longer or sharper edge cases the bound grows with them);
  bfloat16 inputs: max |x - x_ref| <= 2e-2 on O and LSE, and
                   relative RMS ||x - x_ref||_2 / ||x_ref||_2 <= 5e-3 on O, dQ, dK, dV, over the
                   whole tensor and, separately, over every (batch, head) slice of it;
                   every row r (the d values of one query or key) within
                   ||x_r - x_ref,r||_2 <= 0.1 max(||x_ref,r||_2, the RMS row norm of the tensor).
The GPU output is promoted exactly to float64 before comparison.

Why a per-slice and a per-row gate: a whole-tensor norm dilutes a local mistake.  One wholly wrong
row among the 131072 rows of the N=4096 workload moves the tensor's relative RMS by about
sqrt(1/131072) = 2.8e-3, within 5e-3.  A head computed wrong moves its slice's figure to about 1,
and a wrong row moves its own figure to about 1.  The row bound sits between the two: rows of O and
dV (weighted means of V and dO rows) stay within about 2x the tensor's figure, but a row of dQ or
dK is a sum whose weights cancel (every row of dS sums to zero, and in causal rows that see few
keys dP - D nearly cancels too), so the bf16 rounding of dS and of O (through D) is large relative
to what is left: correct rows were measured up to 4.0e-2 (dQ at the GPT-2 shape, causal).  0.1 is
2.5 times that and a tenth of a wrong row's figure.  Rows whose own norm is
small are measured against the typical row norm, so that their relative error does not blow up.
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


BF16_ROW_REL = 0.1


def worst_slice_rel_rms(got, ref):
    """Largest relative RMS over the slices of the leading dimensions ([B, H, N, d]: every (b, h);
    [H, rows, d]: every h)."""
    got = got.double().reshape(-1, ref.shape[-2], ref.shape[-1])
    ref = ref.reshape(-1, ref.shape[-2], ref.shape[-1])
    return max(rel_rms(got[i], ref[i]) for i in range(ref.shape[0]))


def worst_row_error(got, ref):
    """Largest ||x_r - x_ref,r|| / max(||x_ref,r||, RMS row norm) over the rows (last dimension)."""
    got = got.double().reshape(-1, ref.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    norms = torch.linalg.vector_norm(ref, dim=1)
    typical = float(torch.sqrt((norms ** 2).mean()))
    if typical == 0.0:
        return 0.0  # an all-zero reference: the max-abs check decides
    err = torch.linalg.vector_norm(got - ref, dim=1)
    return float((err / torch.clamp(norms, min=typical)).max())


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
    vec = what != "lse" and ref.dim() >= 3 and ref.numel() > 0
    rr = rel_rms(got, ref) if what != "lse" else float("nan")
    hr = worst_slice_rel_rms(got, ref) if vec else float("nan")
    rw = worst_row_error(got, ref) if vec else float("nan")
    if vec:
        report.append(f"{name:>4}: max_abs={ma:.3e} rel_rms={rr:.3e} worst_head_rel_rms={hr:.3e} worst_row={rw:.3e}")
    elif what != "lse":
        report.append(f"{name:>4}: max_abs={ma:.3e} rel_rms={rr:.3e}")
    else:  # (LSE is gated by its absolute error only; rows with no visible key hold -inf on both sides)
        report.append(f"{name:>4}: max_abs={ma:.3e}")
    tol_scale = 1.0 if what == "lse" else float(abs_scale)
    if dtype == torch.float32:
        fin = ref[torch.isfinite(ref)]
        mag = 1.0 if what == "lse" or fin.numel() == 0 else max(1.0, float(fin.abs().max()))
        bound = F32_MAX_ABS * tol_scale * mag
        if not ma <= bound:
            fails.append(f"{name} max_abs {ma:.3e} > {bound:.3e}")
    else:
        if what in ("o", "lse") and not ma <= BF16_MAX_ABS * tol_scale:
            fails.append(f"{name} max_abs {ma:.3e} > {BF16_MAX_ABS * tol_scale}")
        if what != "lse" and not rr <= BF16_REL_RMS:
            fails.append(f"{name} rel_rms {rr:.3e} > {BF16_REL_RMS}")
        if vec and not hr <= BF16_REL_RMS:
            fails.append(f"{name} worst (batch, head) rel_rms {hr:.3e} > {BF16_REL_RMS}")
        if vec and not rw <= BF16_ROW_REL:
            fails.append(f"{name} worst row error {rw:.3e} > {BF16_ROW_REL}")
    return fails
