"""Exact-attention oracle: plain, slow, fp64, CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  The product
(the HIP library and its Python binding) never calls it and shares no code
with it.

What it computes, and where that is defined
-------------------------------------------
* NOTE-005: FlashAttention (anthology-of-the-sota), "Key results", Theorem 1:
  the algorithm returns O = softmax(Q Kᵀ) V.
* "FlashAttention: The IO-Aware Algorithm That Rewrote GPU Training Speed
  Records" (promptingindex.com), section "Why attention is memory-bound, not
  compute-bound": attention is the chain matmul -> scaling -> masking ->
  softmax -> (dropout) -> matmul with V.  Dropout is optional: ``forward`` and
  ``backward`` take an explicit keep mask Z (bool [B, H, N, N]) and the scale s
  of the kept probabilities (oracle/philox.py builds Z from a seed; the kernels
  regenerate the same mask themselves).  The dropped attention is
  O = (P * Z s) V; LSE stays that of the undropped P;
* The same NOTE-005 page, "Method": the forward keeps a running max m and a
  normaliser l per row and the backward recomputes the attention block from
  them.  The quantity stored per row is LSE = m + ln l, the natural-log
  log-sum-exp of the row's scaled, masked scores; P = exp(S - LSE).

Because tiled attention is exact (NOTE-005 "Key insight"; the aicassindra
architecture page, "End-to-end flow"), its result has a plain definition and
this oracle is that definition written out: it materialises the full score
matrix S for one (batch, head) at a time, with no tiling, no online softmax and
no fusion.  Library primitives used as steps: ``torch.matmul``, ``torch.exp``,
``torch.log``, ``torch.amax``, ``torch.sum`` -- all in float64 on the CPU.

Readings where the pages are silent:
* scale: S = scale * Q Kᵀ with the caller's float32 scale promoted to fp64;
* mask: additive 0 / -inf.  Causal keeps key j for query i iff j <= i
  (top-left aligned, Nq = Nk = N).  Key padding keeps key j of batch b iff
  j < L_b with L_b = clamp(seqlens[b], 0, N); both masks combine by AND;
  padded *query* rows are computed normally;
* block-sparse attention (the tiling applied to a sparse pattern: promptingindex
  page, "Benchmark results: speed records without any approximation"; NOTE-005,
  "Key components" and "Limitations", where it is approximate relative to dense
  attention): an optional [B, H, ceil(N/128), ceil(N/128)] block mask; key j is
  visible to query i only if block (i // 128, j // 128) is nonzero.  It combines
  with the other masks by AND, and the result is exact for the masked problem;
* a row with no visible key (L_b = 0, or every block of its row masked out)
  has O = 0, LSE = -inf and contributes no gradient;
* backward of the loss sum(dO * O): dV = Pᵀ dO, dP = dO Vᵀ,
  D_i = sum_j P_ij dP_ij, dS = P * (dP - D), dQ = scale * dS K,
  dK = scale * dSᵀ Q -- the chain rule through the definition above (the pages
  only say that the backward recomputes the block).  With dropout the chain
  passes through P * Z s: dV = (P Z s)ᵀ dO, dP = (dO Vᵀ) Z s, and D_i, dS, dQ, dK
  as above (D_i = sum_j P_ij dP_ij = dO_i . O_i still holds).

Inputs may be any floating dtype; they are promoted exactly to float64, so the
oracle sees the stored (e.g. bfloat16) values themselves.
"""
from __future__ import annotations

import math

import torch

F64 = torch.float64
MASK_BLOCK = 128  # rows and columns of one block of the block-sparse mask


def _f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=F64)


def key_lengths(B: int, N: int, seqlens) -> list[int]:
    """Valid key count L_b per batch entry: clamp(seqlens[b], 0, N), or N when absent."""
    if seqlens is None:
        return [N] * B
    s = torch.as_tensor(seqlens).to("cpu").to(torch.int64).tolist()
    if len(s) != B:
        raise ValueError("seqlens must have one entry per batch element")
    return [min(max(int(x), 0), N) for x in s]


def block_count(N: int) -> int:
    """Blocks per side of the block-sparse mask: ceil(N / 128)."""
    return (N + MASK_BLOCK - 1) // MASK_BLOCK


def visible(N: int, causal: bool, L: int, rows=None, blocks=None) -> torch.Tensor:
    """Boolean visibility vis[i, j] for query rows ``rows`` (default all) and keys 0..N-1.

    Masking step of the attention chain ("Why attention is memory-bound" section
    of the promptingindex page), read as: key j is visible to query i iff
    j < L (key padding) and, when causal, j <= i, and, when ``blocks`` (this
    head's [ceil(N/128), ceil(N/128)] block mask) is given, block
    (i // 128, j // 128) is nonzero.
    """
    i = torch.arange(N, dtype=torch.int64) if rows is None else torch.as_tensor(rows, dtype=torch.int64)
    j = torch.arange(N, dtype=torch.int64)
    vis = (j[None, :] < L).expand(i.numel(), N).clone()
    if causal:
        vis &= j[None, :] <= i[:, None]
    if blocks is not None:
        bm = torch.as_tensor(blocks).to("cpu") != 0
        nb = block_count(N)
        if tuple(bm.shape) != (nb, nb):
            raise ValueError(f"block mask of one head must be [{nb}, {nb}]")
        vis &= bm[(i // MASK_BLOCK)[:, None], (j // MASK_BLOCK)[None, :]]
    return vis


def _head_blocks(block_mask, B: int, H: int, b: int, h: int):
    """The [nb, nb] block mask of head (b, h), or None for dense attention."""
    if block_mask is None:
        return None
    bm = torch.as_tensor(block_mask).to("cpu")
    if bm.dim() != 4 or bm.shape[0] != B or bm.shape[1] != H:
        raise ValueError("block mask must be [B, H, ceil(N/128), ceil(N/128)]")
    return bm[b, h]


def _scores(q, k, scale, vis):
    """S = scale * q kᵀ where visible, -inf elsewhere (fp64)."""
    s = torch.matmul(q, k.transpose(0, 1)) * scale
    return s.masked_fill(~vis, -math.inf)


def _row_lse(s):
    """LSE_i = m_i + ln sum_j exp(S_ij - m_i); -inf for rows with no visible key."""
    m = torch.amax(s, dim=1, keepdim=True)
    empty = torch.isinf(m) & (m < 0)
    m_safe = torch.where(empty, torch.zeros_like(m), m)
    l = torch.sum(torch.exp(s - m_safe), dim=1, keepdim=True)
    lse = m_safe + torch.log(l)
    return torch.where(empty, torch.full_like(lse, -math.inf), lse)[:, 0]


def _probs(s, lse):
    """P_ij = exp(S_ij - LSE_i); rows with LSE = -inf are all zero."""
    empty = torch.isinf(lse) & (lse < 0)
    lse_safe = torch.where(empty, torch.zeros_like(lse), lse)
    p = torch.exp(s - lse_safe[:, None])
    return torch.where(empty[:, None], torch.zeros_like(p), p)


def _keep(keep, b, h):
    return None if keep is None else torch.as_tensor(keep)[b, h].to("cpu")


def forward(q, k, v, scale: float, causal: bool = False, seqlens=None, block_mask=None, keep=None,
            keep_scale: float = 1.0):
    """O and LSE for [B, H, N, d] inputs; returns fp64 tensors O [B,H,N,d] and LSE [B,H,N].

    NOTE-005 "Key results" Theorem 1 (O = softmax(QKᵀ)V) with the scaling and
    masking steps of the promptingindex page; LSE is the per-row statistic the
    forward keeps for the backward (NOTE-005 "Method").
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    L = key_lengths(B, N, seqlens)
    scale = float(scale)
    o = torch.empty(B, H, N, v.shape[-1], dtype=F64)
    lse = torch.empty(B, H, N, dtype=F64)
    for b in range(B):
        vis_b = visible(N, causal, L[b])
        for h in range(H):
            blocks = _head_blocks(block_mask, B, H, b, h)
            vis = vis_b if blocks is None else visible(N, causal, L[b], blocks=blocks)
            s = _scores(q[b, h], k[b, h], scale, vis)
            lse[b, h] = _row_lse(s)
            p = _probs(s, lse[b, h])
            z = _keep(keep, b, h)
            if z is not None:
                p = torch.where(z, p * float(keep_scale), torch.zeros_like(p))
            o[b, h] = torch.matmul(p, v[b, h])
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool = False, seqlens=None, block_mask=None, keep=None,
             keep_scale: float = 1.0):
    """dQ, dK, dV (fp64) of the loss sum(dO * O) through the definition of ``forward``.

    The pages state only that the backward recomputes the attention block from
    the stored statistics (NOTE-005 "Method"; aicassindra page, "The
    architecture: every piece explained").  The formulas are the chain rule:
    dV = Pᵀ dO; dP = dO Vᵀ; D_i = sum_j P_ij dP_ij; dS = P (dP - D);
    dQ = scale dS K; dK = scale dSᵀ Q.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    L = key_lengths(B, N, seqlens)
    scale = float(scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    for b in range(B):
        vis_b = visible(N, causal, L[b])
        for h in range(H):
            blocks = _head_blocks(block_mask, B, H, b, h)
            vis = vis_b if blocks is None else visible(N, causal, L[b], blocks=blocks)
            s = _scores(q[b, h], k[b, h], scale, vis)
            p = _probs(s, _row_lse(s))
            z = _keep(keep, b, h)
            pz = p if z is None else torch.where(z, p * float(keep_scale), torch.zeros_like(p))
            dv[b, h] = torch.matmul(pz.transpose(0, 1), do[b, h])
            dp = torch.matmul(do[b, h], v[b, h].transpose(0, 1))
            if z is not None:
                dp = torch.where(z, dp * float(keep_scale), torch.zeros_like(dp))
            D = torch.sum(p * dp, dim=1, keepdim=True)
            ds = p * (dp - D)
            dq[b, h] = torch.matmul(ds, k[b, h]) * scale
            dk[b, h] = torch.matmul(ds.transpose(0, 1), q[b, h]) * scale
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Row / column views of the same definition, for sequence lengths where a full
# N x N matrix per head does not fit.  Every row is still complete: these only
# choose which rows (or which key columns) are produced.
# ----------------------------------------------------------------------------

def forward_rows(q, k, v, scale: float, causal: bool, seqlens, b: int, h: int, rows, block_mask=None):
    """O[rows] and LSE[rows] of head (b, h), each row over all N keys (same definition as ``forward``)."""
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    N = kh.shape[0]
    rows = torch.as_tensor(rows, dtype=torch.int64)
    L = key_lengths(q.shape[0], N, seqlens)[b]
    blocks = _head_blocks(block_mask, q.shape[0], q.shape[1], b, h)
    s = _scores(qh[rows], kh, float(scale), visible(N, causal, L, rows, blocks))
    lse = _row_lse(s)
    return torch.matmul(_probs(s, lse), vh), lse


def backward_rows(q, k, v, do, scale: float, causal: bool, seqlens, b: int, h: int, rows, block_mask=None):
    """dQ[rows] of head (b, h).  Row i of dQ needs only row i of P, dP and D."""
    qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h])
    N = kh.shape[0]
    rows = torch.as_tensor(rows, dtype=torch.int64)
    L = key_lengths(q.shape[0], N, seqlens)[b]
    blocks = _head_blocks(block_mask, q.shape[0], q.shape[1], b, h)
    s = _scores(qh[rows], kh, float(scale), visible(N, causal, L, rows, blocks))
    p = _probs(s, _row_lse(s))
    dp = torch.matmul(doh[rows], vh.transpose(0, 1))
    D = torch.sum(p * dp, dim=1, keepdim=True)
    return torch.matmul(p * (dp - D), kh) * float(scale)


def row_stats(q, k, v, do, scale: float, causal: bool, seqlens, b: int, h: int, chunk: int = 1024,
              progress=None, block_mask=None):
    """LSE_i and D_i for every row of head (b, h), computed ``chunk`` complete rows at a time.

    D_i = sum_j P_ij dP_ij is evaluated as dO_i . O_i, which equals it because
    dP_ij = dO_i . v_j and O_i = sum_j P_ij v_j (the identity is checked against
    ``backward`` in the oracle's own tests).  ``progress(done_rows, N)`` is
    called after each chunk when given (long passes report that they are alive).
    """
    N = q.shape[2]
    lse = torch.empty(N, dtype=F64)
    D = torch.empty(N, dtype=F64)
    doh = _f64(do[b, h])
    for r0 in range(0, N, chunk):
        rows = torch.arange(r0, min(N, r0 + chunk))
        o_r, lse_r = forward_rows(q, k, v, scale, causal, seqlens, b, h, rows, block_mask)
        lse[rows] = lse_r
        D[rows] = torch.sum(o_r * doh[rows], dim=1)
        if progress is not None:
            progress(int(rows[-1]) + 1, N)
    return lse, D


def backward_keys(q, k, v, do, scale: float, causal: bool, seqlens, b: int, h: int, keys, lse, D,
                  block_mask=None):
    """dK[keys], dV[keys] of head (b, h) from the full-row statistics LSE and D of ``row_stats``.

    Column j of P needs LSE_i of every row i; column j of dS needs D_i of every
    row: dV_j = sum_i P_ij dO_i, dK_j = scale sum_i P_ij (dP_ij - D_i) q_i.
    """
    qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h])
    N = qh.shape[0]
    keys = torch.as_tensor(keys, dtype=torch.int64)
    L = key_lengths(q.shape[0], N, seqlens)[b]
    blocks = _head_blocks(block_mask, q.shape[0], q.shape[1], b, h)
    vis_t = visible(N, causal, L, blocks=blocks)[:, keys]        # [N, |keys|]
    st = (torch.matmul(qh, kh[keys].transpose(0, 1)) * float(scale)).masked_fill(~vis_t, -math.inf)
    lse = _f64(lse)
    empty = torch.isinf(lse) & (lse < 0)
    p = torch.exp(st - torch.where(empty, torch.zeros_like(lse), lse)[:, None])
    p = torch.where(empty[:, None], torch.zeros_like(p), p)      # P[:, keys]
    dp = torch.matmul(doh, vh[keys].transpose(0, 1))              # dP[:, keys]
    ds = p * (dp - _f64(D)[:, None])
    dv = torch.matmul(p.transpose(0, 1), doh)
    dk = torch.matmul(ds.transpose(0, 1), qh) * float(scale)
    return dk, dv
