"""Benchmark of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--workload 4] [--no-cpu-baseline]
                    [--cold]
    python bench.py --all-configs      (every workload, its fraction of the per-config roofline)
    python bench.py --naive-torch      (the materialising attention as plain torch ops; context)

One step = one forward (fa_forward) plus one backward (fa_backward) over one batch of the synthetic
workload, inputs resident in HBM.  The whole-job time (`value`, `ms_per_step`) comes from K steps of
those two public calls with no event between them; a second run of K steps with an event around
every launch (the forward, then fa_backward's two stages, fa_backward_dq_prepare and
fa_backward_dkdv, called separately: the same kernels fa_backward launches for dense bf16) gives each
kernel's average duration (an event recorded between two kernels costs the stream a few
microseconds).  Under
sustained load the GPU's power management needs about a third of a
second to reach its steady state: the clocks ramp up over the first tens of milliseconds, and about
0.27 s in, a one-time throttle stalls the queue for ~60 ms and runs the next ~50 ms at reduced
clocks (measured per 10-step batch over 2 s of this step; no further event followed).  So the step
is first repeated untimed for --settle-ms (default 1000 ms, well past that transient); then W
untimed steps, then the two timed runs of K steps, each bracketed by synchronisation and HIP events
on the stream the kernels run on.

FLOPs are algorithmic: forward 4 d per visible (query, key) pair (QK^T and PV), backward 2.5x
forward (QK^T recomputed, dO V^T, P^T dO, dS^T Q, dS K), of which the dK/dV pass is credited with
the first four products (8 d per pair) and the dQ pass with dS K (2 d per pair; it recomputes
QK^T and dO V^T as well, which counts as overhead, not as work).  Causal pairs per head N(N+1)/2.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (bf16, causal, N=4096 d=128) and % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
PEAK_F32_VALU_TFLOPS = 157.3    # MI355X fp32 vector (the fp32 path runs on the VALU)


def visible_pairs(N: int, causal: bool, key_len: int) -> int:
    """(query, key) pairs with key < key_len and, if causal, key <= query."""
    L = max(0, min(N, key_len))
    if not causal:
        return N * L
    return L * (L + 1) // 2 + (N - L) * L


def workload_flops(w, x):
    lens = [w.N] * w.B if x["seqlens"] is None else [int(s) for s in x["seqlens"]]
    pairs = sum(visible_pairs(w.N, w.causal, L) for L in lens) * w.H
    fwd = 4.0 * w.d * pairs
    return fwd, 2.5 * fwd, 2.0 * fwd, 0.5 * fwd


PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_causal_n4096_d128.md")


def sources_sha256() -> str:
    """sha256 over the library's kernel sources (sorted by name, concatenated)."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "exact_io_aware_66_amd", "csrc")
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(src, "*.hip")) + glob.glob(os.path.join(src, "*.hpp")) +
                    glob.glob(os.path.join(src, "*.cpp"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload_name: str):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE passes, scaled by the copy calibration), or None when there is none for this
    workload or the kernel sources have changed since the counters were taken."""
    import re
    if workload_name != "long-causal-n4096-d128" or not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m = re.search(r"sha256: ([0-9a-f]{64})", text)
    if not m or m.group(1) != sources_sha256():
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0].strip("`").startswith(kernel + "<"):
            return float(cells[5])
    return None


def cpu_baseline(w, x, target_s: float = 12.0):
    """Time the fp64 oracle (forward + backward) on the first heads of batch element 0."""
    import torch

    import oracle
    sl = None if x["seqlens"] is None else x["seqlens"][:1]
    # Without key padding every (batch, head) pair is alike: view them as heads of one batch element.
    flat = {n: (x[n][:1] if sl is not None else x[n].reshape(1, w.B * w.H, w.N, w.d)) for n in ("q", "k", "v", "do")}
    nmax = flat["q"].shape[1]

    def run(nh):
        sub = {n: flat[n][:, :nh].contiguous() for n in ("q", "k", "v", "do")}
        t0 = time.perf_counter()
        oracle.forward(sub["q"], sub["k"], sub["v"], x["scale"], w.causal, sl)
        oracle.backward(sub["q"], sub["k"], sub["v"], sub["do"], x["scale"], w.causal, sl)
        return time.perf_counter() - t0

    t1 = run(1)
    nh = int(max(1, min(nmax, target_s // max(t1, 1e-3))))
    t = run(nh) if nh > 1 else t1
    L = w.N if sl is None else int(sl[0])
    flops = 4.0 * w.d * visible_pairs(w.N, w.causal, L) * nh * 3.5
    # the oracle itself is dense: it materialises every (query, key) pair, forward 4 N^2 d, and its
    # backward 8 N^2 d (it keeps P)
    oracle_flops = 12.0 * w.N * w.N * w.d * nh
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")}
                for i in threadpoolctl.threadpool_info()]
    except Exception:
        pass
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of the first {nh} of the {w.B * w.H} (batch, head) pairs, "
                      f"{t:.1f} s wall; algorithmic FLOPs as for the GPU",
            "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model, "blas": blas,
            "oracle_flops": oracle_flops, "oracle_gflops_per_s": round(oracle_flops / t / 1e9, 2)}


def min_bytes(w):
    """Algorithmic HBM bytes: forward (3 reads + 1 write of [B,H,N,d] + LSE), backward (5 reads +
    3 writes + 12 B of row statistics per row)."""
    es = 2 if w.dtype == "bf16" else 4
    t = w.B * w.H * w.N * w.d * es
    rows = w.B * w.H * w.N
    return 4 * t + 4 * rows, 8 * t + 12 * rows


def dkdv_kernel(w) -> str:
    """The kernel the dK/dV pass of a dense, dropout-free backward runs for this workload: at d = 128
    in bf16 the one with K in LDS and 256 keys per workgroup, otherwise the general one (128 keys)."""
    return "bwd_dkdv_kl_kernel" if (w.d == 128 and w.dtype == "bf16") else "bwd_dkdv_kernel"


def as_tiled_bytes(w, x):
    """HBM bytes per launch of each bf16 kernel if every tile it loads came from HBM (no reuse between
    workgroups in any cache): the Theta(N^2 d^2 / M) term of the pages' IO analysis for the tiles these
    kernels actually use, next to the counters.  Forward: one workgroup per query block of B_r rows
    (256 at d = 128, 128 at d = 64) reads its Q block once and, for every visible 64-key tile, K and V
    (2 d bf16 values per key); O and LSE written once.  dK/dV: one workgroup per 256 keys (d = 128) or
    128 keys (d = 64) reads its K and V once and, for every visible query row, Q, dO (2 d values) and
    the two row statistics (8 B); dK and dV written once.  dQ (with the row statistics formed in it): one workgroup per 256 query
    rows reads its Q, dO and O rows and LSE once and, for every visible 64-key tile, K and V; dQ, D
    and LSE log2(e) written once.  Key padding is ignored in the tile counts (an upper bound)."""
    es = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.H * w.N
    row_b = w.d * es
    lens = [w.N] * w.B if x["seqlens"] is None else [max(0, min(w.N, int(s))) for s in x["seqlens"]]

    def kv_tiles(br, bc=64):
        """(visible keys, rounded up to whole tiles) summed over the query blocks of every head."""
        total = 0
        for L in lens:
            for qb in range(-(-w.N // br)):
                end = min(L, (qb + 1) * br) if w.causal else L
                total += -(-end // bc) * bc
        return total * w.H

    def q_rows_per_key_block(bk):
        total = 0
        for L in lens:
            for kb in range(-(-w.N // bk)):
                if kb * bk >= L:
                    continue
                total += (w.N - kb * bk) if w.causal else w.N
        return total * w.H

    br_f = 256 if w.d == 128 else 128
    fwd = rows * row_b + kv_tiles(br_f) * 2 * row_b + rows * row_b + rows * 4
    kname = dkdv_kernel(w)
    bk = 256 if kname == "bwd_dkdv_kl_kernel" else 128
    dkdv = 2 * rows * row_b + q_rows_per_key_block(bk) * (2 * row_b + 8) + 2 * rows * row_b
    dq = 3 * rows * row_b + rows * 4 + kv_tiles(256) * 2 * row_b + rows * row_b + 8 * rows
    return {"fwd_bf16_kernel": fwd, kname: dkdv, "bwd_dq_kernel": dq}


def naive_torch_forward(w, x, steps: int):
    """The materialising attention (S written, softmax, P V) as plain torch ops, timed on the GPU:
    context for the fused kernels, never a fallback."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    kt = k.transpose(-1, -2).contiguous()
    mask = None
    if w.causal:
        mask = torch.ones(w.N, w.N, dtype=torch.bool, device=dev).triu(1)

    def fwd():
        s = torch.matmul(q, kt) * x["scale"]
        if mask is not None:
            s = s.masked_fill(mask, float("-inf"))
        p = torch.softmax(s.float(), dim=-1).to(q.dtype)
        return torch.matmul(p, v)

    for _ in range(3):
        fwd()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fwd()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def block_pairs(bm, N: int, causal: bool, lens) -> int:
    """Visible (query, key) pairs of a [B, H, nb, nb] block mask combined with the causal mask and
    the key lengths (per batch element)."""
    import torch
    B, H, nb, _ = bm.shape
    blk = 128
    qb = torch.arange(nb)[:, None].expand(nb, nb)
    kb = torch.arange(nb)[None, :].expand(nb, nb)
    total = 0
    for b in range(B):
        L = N if lens is None else max(0, min(N, int(lens[b])))
        r0, r1 = qb * blk, torch.clamp((qb + 1) * blk, max=N)
        k0, k1 = kb * blk, torch.clamp(torch.clamp((kb + 1) * blk, max=N), max=L)
        rows = r1 - r0
        if not causal:
            per = rows * torch.clamp(k1 - k0, min=0)
        else:  # sum over rows i of max(0, min(k1, i + 1) - k0)
            per = torch.zeros(nb, nb, dtype=torch.int64)
            for off in range(blk):
                i = r0 + off
                per += torch.where(i < r1, torch.clamp(torch.minimum(k1, i + 1) - k0, min=0), 0)
        total += int((per * (bm[b] != 0).to(torch.int64)).sum())
    return total


SUB_SETTLE_MS = 200.0


def settle(fn, ms: float = SUB_SETTLE_MS):
    """Repeat fn (untimed) for `ms` of wall time, synchronising every 5 calls: the measurements after
    the dense step follow host-side set-up (quantisation, mask generation) during which the GPU
    idles, and its clocks need tens of milliseconds of load to come back up."""
    import torch
    t = time.perf_counter()
    while (time.perf_counter() - t) * 1e3 < ms:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()


def measure_block_sparse(fa, w, x, pattern: str, steps: int, dense_ms: tuple):
    """Forward and backward of workload w with a block mask (fa_forward_block_sparse,
    fa_backward_block_sparse): time per step, FLOPs over the visible pairs only, speedup over the
    dense steps."""
    import torch

    import workloads
    dev = torch.device("cuda:0")
    bm = workloads.draw_block_mask(w.B, w.H, w.N, pattern, density=0.5, window=1, seed=7)
    pairs = block_pairs(bm, w.N, w.causal, x["seqlens"])
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    sl = None if x["seqlens"] is None else x["seqlens"].to(dev)
    bmd = bm.to(dev)
    o, lse = torch.empty_like(q), torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_size(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def fwd():
        fa.fa_forward_block_sparse(q, k, v, o, lse, x["scale"], w.causal, sl, bmd)

    def bwd():
        fa.fa_backward_block_sparse(q, k, v, o, do, lse, dq, dk, dv, x["scale"], w.causal, sl, bmd, ws)

    settle(lambda: (fwd(), bwd()))
    e[0].record(stream)
    for _ in range(steps):
        fwd()
    e[1].record(stream)
    for _ in range(steps):
        bwd()
    e[2].record(stream)
    torch.cuda.synchronize()
    ms_f, ms_b = e[0].elapsed_time(e[1]) / steps, e[1].elapsed_time(e[2]) / steps
    ff = 4.0 * w.d * pairs
    dense_pairs = workload_flops(w, x)[0] / (4.0 * w.d)
    return {"pattern": pattern, "visible_blocks": int((bm != 0).sum()), "blocks": bm.numel(),
            "visible_pairs_frac_of_dense": round(pairs / dense_pairs, 4),
            "fwd_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
            "fwd_tflops": round(ff / (ms_f * 1e-3) / 1e12, 2), "fwd_bwd_tflops": round(3.5 * ff / ((ms_f + ms_b) * 1e-3) / 1e12, 2),
            "speedup_vs_dense_fwd_bwd": round((dense_ms[0] + dense_ms[1]) / (ms_f + ms_b), 3)}


def measure_dropout(fa, w, x, p: float, steps: int, dense_ms: tuple):
    """Forward and backward of workload w with fused dropout (fa_forward_dropout,
    fa_backward_dropout): time per step, algorithmic FLOPs as for the dense step (every pair is
    still computed; dropout only zeroes some in P V and dP), slowdown against the dense steps."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    sl = None if x["seqlens"] is None else x["seqlens"].to(dev)
    o, lse = torch.empty_like(q), torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_size(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    seed = 0x5EED

    def fwd(i):
        fa.fa_forward_dropout(q, k, v, o, lse, x["scale"], w.causal, sl, p, seed, i)

    def bwd(i):
        fa.fa_backward_dropout(q, k, v, o, do, lse, dq, dk, dv, x["scale"], w.causal, sl, p, seed, i, ws)

    settle(lambda: (fwd(0), bwd(0)))
    e[0].record(stream)
    for i in range(steps):
        fwd(i)
    e[1].record(stream)
    for i in range(steps):
        bwd(i)
    e[2].record(stream)
    torch.cuda.synchronize()
    ms_f, ms_b = e[0].elapsed_time(e[1]) / steps, e[1].elapsed_time(e[2]) / steps
    ff, fb = workload_flops(w, x)[:2]
    return {"p": p, "fwd_ms": round(ms_f, 4), "bwd_ms": round(ms_b, 4),
            "fwd_tflops": round(ff / (ms_f * 1e-3) / 1e12, 2),
            "fwd_bwd_tflops": round((ff + fb) / ((ms_f + ms_b) * 1e-3) / 1e12, 2),
            "time_vs_dense_fwd_bwd": round((ms_f + ms_b) / (dense_ms[0] + dense_ms[1]), 3)}


def kv_outer_model_bytes(B: int, H: int, N: int, d: int, bc: int, br: int) -> int:
    """HBM bytes of the pages' K/V-outer schedule as fa_forward_kv_outer runs it: K and V (bf16) read
    once; O (fp32), m and l initialised; then for every K/V block and every Q block, Q_i (bf16), O_i,
    m_i and l_i read and O_i, m_i, l_i written back (the last K/V block writes O in bf16 and LSE)."""
    tc, tr = -(-N // bc), -(-N // br)
    del tr
    per_head = (2 * N * d * 2                      # K, V
                + N * d * 4 + 2 * N * 4             # initial O, m, l
                + tc * N * (d * 2 + d * 4 + 8)      # Q_i, O_i, m_i, l_i read per K/V block
                + (tc - 1) * N * (d * 4 + 8)        # O_i, m_i, l_i written back
                + N * (d * 2 + 8 + 4))              # last block: O (bf16), m, l, LSE
    return B * H * per_head


def theorem2(fa, lds_list, N: int, d: int, BH: int):
    """One launch of the K/V-outer schedule per LDS budget on seeded inputs; prints one JSON line each."""
    import torch

    import workloads
    x = workloads.draw_custom(1, BH, N, d, dtype="bf16", seed=2)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o, lse = torch.empty_like(q), torch.empty(1, BH, N, dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_forward_kv_outer_workspace_size(1, BH, N, d), dtype=torch.uint8, device="cuda")
    for lds in lds_list:
        m = lds // 4
        bc = -(-m // (4 * d))
        br = min(bc, d)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fa.fa_forward_kv_outer(q, k, v, o, lse, x["scale"], lds, ws)
        b.record()
        torch.cuda.synchronize()
        print(json.dumps({"theorem2": True, "B": 1, "H": BH, "N": N, "d": d, "lds_bytes": lds, "M_elements": m,
                          "Bc": bc, "Br": br, "ms": round(a.elapsed_time(b), 3),
                          "model_bytes": kv_outer_model_bytes(1, BH, N, d, bc, br),
                          "n2d2_over_m": N * N * d * d / m}), flush=True)


def measure_fp8_forward(fa, w, x, steps: int, dense_fwd_ms: float):
    """fa_forward_fp8 on workload w with its inputs quantised to OCP FP8 E4M3 (per-tensor descales):
    time per forward, algorithmic TFLOP/s (4 d per visible pair, as for the bf16 forward)."""
    import torch

    import workloads
    q8, dq = workloads.quantize_fp8(x["q"])
    k8, dk = workloads.quantize_fp8(x["k"])
    v8, dv = workloads.quantize_fp8(x["v"])
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    sl = None if x["seqlens"] is None else x["seqlens"].cuda()
    o = torch.empty(w.B, w.H, w.N, w.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")

    def fwd():
        fa.fa_forward_fp8(q8, k8, v8, dq, dk, dv, o, lse, x["scale"], w.causal, sl)

    settle(fwd)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fwd()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    ff = workload_flops(w, x)[0]
    return {"fwd_ms": round(ms, 4), "fwd_tflops": round(ff / (ms * 1e-3) / 1e12, 2),
            "time_vs_bf16_fwd": round(ms / dense_fwd_ms, 3),
            "note": "S on the FP8 matrix cores (half the forward's flops), P V in bf16"}


def measure(fa, w, x, steps: int, warmup: int, settle_ms: float, cold: bool = False):
    """Time `steps` fwd+bwd steps of workload w (inputs resident on the device): clock settling,
    warm-up, then HIP events around the timed region and around every launch."""
    import statistics

    import torch
    dev = torch.device("cuda:0")
    q, k, v, do = (x[n].to(dev) for n in ("q", "k", "v", "do"))
    sl = None if x["seqlens"] is None else x["seqlens"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_backward_workspace_size(w.B, w.H, w.N, w.d, q.dtype), dtype=torch.uint8, device=dev)
    scale, causal = x["scale"], w.causal
    flops_fwd, flops_bwd, flops_dkdv, flops_dq = workload_flops(w, x)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None

    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(e=None):
        if e is None:  # the public calls
            fa.fa_forward(q, k, v, o, lse, scale, causal, sl)
            fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, scale, causal, sl, ws)
            return
        # fa_backward's two kernels, called as its stages so that an event can separate them
        e[0].record(stream)
        fa.fa_forward(q, k, v, o, lse, scale, causal, sl)
        e[1].record(stream)
        fa.fa_backward_dq_prepare(q, k, v, o, do, lse, dq, scale, causal, sl, ws)
        e[2].record(stream)
        fa.fa_backward_dkdv(q, k, v, do, lse, dk, dv, scale, causal, sl, ws)
        e[3].record(stream)

    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The whole-job time: K steps with nothing but the kernels between two events (an event recorded
    # between kernels costs the stream a few microseconds of its own, so the per-kernel events are
    # kept out of this loop).  Then K more steps with an event around every launch, for the
    # per-kernel durations.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if scratch is None:
        t_start.record(stream)
        for i in range(steps):
            step()
        t_end.record(stream)
        torch.cuda.synchronize()
        ms_step = t_start.elapsed_time(t_end) / steps
    i_start = torch.cuda.Event(enable_timing=True)
    i_end = torch.cuda.Event(enable_timing=True)
    i_start.record(stream)
    for i in range(steps):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        step(ev[i])
    i_end.record(stream)
    torch.cuda.synchronize()
    if scratch is not None:  # cold steps: the scratch writes are outside the kernels, not the job
        ms_step = None
    names = ("fwd", "dq", "dkdv")
    per = {n: [e[j].elapsed_time(e[j + 1]) for e in ev] for j, n in enumerate(names)}
    r = {"ms_step": ms_step, "ms_step_instrumented": i_start.elapsed_time(i_end) / steps,
         "flops_fwd": flops_fwd, "flops_bwd": flops_bwd,
         "flops_dkdv": flops_dkdv, "flops_dq": flops_dq,
         "med": {n: round(statistics.median(v), 4) for n, v in per.items()},
         "min": {n: round(min(v), 4) for n, v in per.items()}}
    for n in names:
        r["ms_" + n] = sum(per[n]) / steps
    r["ms_bwd"] = r["ms_dq"] + r["ms_dkdv"]
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="repeat the step untimed for this long before the warm-up steps (clock ramp and "
                         "the one-time power-management throttle about 0.27 s into sustained load)")
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8-input forward measurement (same workload, inputs quantised to E4M3)")
    ap.add_argument("--no-dropout", action="store_true",
                    help="skip the fused-dropout measurement (same workload, p = 0.1)")
    ap.add_argument("--no-block-sparse", action="store_true",
                    help="skip the block-sparse measurements (same workload, two block masks)")
    ap.add_argument("--cold", action="store_true",
                    help="also time steps with a 512 MiB scratch write between them (cold caches)")
    ap.add_argument("--all-configs", action="store_true",
                    help="only time every workload and print one line each with its per-config roofline fraction")
    ap.add_argument("--naive-torch", action="store_true",
                    help="only time the materialising attention forward as plain torch ops (context)")
    ap.add_argument("--theorem2", action="store_true",
                    help="only run the pages' K/V-outer schedule (fa_forward_kv_outer) once per LDS budget "
                         "(16, 32, 64, 128 KiB) at N=4096, d=128, 64 heads (8 per XCD, so the heads' Q and O overflow "
                         "each XCD's 4 MB L2), for its HBM byte counters")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reads and writes MIB MiB), to scale the HBM "
                         "byte counters of a profiler run, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (got --gpus {args.gpus}); the attention of one "
              f"(batch, head) never crosses GPUs and no multi-GPU path exists", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                          "dispatches": 3}), flush=True)
        return

    import exact_io_aware_66_amd as fa
    import workloads

    fa.load()
    if args.theorem2:
        theorem2(fa, [16 * 1024, 32 * 1024, 64 * 1024, 128 * 1024], 4096, 128, 64)
        return
    if args.all_configs:
        for wid in sorted(workloads.WORKLOADS):
            w = workloads.WORKLOADS[wid]
            x = workloads.draw(w)
            r = measure(fa, w, x, max(3, args.steps // 4), 2, args.settle_ms)
            fb, bb = min_bytes(w)
            ff, fbw = r["flops_fwd"], r["flops_bwd"]
            peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_VALU_TFLOPS
            roof_f = min(peak, ff / fb * PEAK_HBM_GBS / 1e3)
            roof_b = min(peak, fbw / bb * PEAK_HBM_GBS / 1e3)
            tf = ff / (r["ms_fwd"] * 1e-3) / 1e12
            tb = fbw / (r["ms_bwd"] * 1e-3) / 1e12
            print(json.dumps({"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype,
                              "causal": w.causal, "key_padding": w.padded,
                              "fwd_ms": round(r["ms_fwd"], 4), "fwd_tflops": round(tf, 2),
                              "fwd_ai_flop_per_byte": round(ff / fb, 1), "fwd_roofline_tflops": round(roof_f, 1),
                              "fwd_frac_of_roofline": round(tf / roof_f, 4),
                              "bwd_ms": round(r["ms_bwd"], 4), "bwd_tflops": round(tb, 2),
                              "bwd_ai_flop_per_byte": round(fbw / bb, 1), "bwd_roofline_tflops": round(roof_b, 1),
                              "bwd_frac_of_roofline": round(tb / roof_b, 4)}), flush=True)
        return

    w = workloads.WORKLOADS[args.workload]
    x = workloads.draw(w)
    if args.naive_torch:
        ms = naive_torch_forward(w, x, args.steps)
        ff = workload_flops(w, x)[0]
        es = 2 if w.dtype == "bf16" else 4
        print(json.dumps({"workload": w.name, "naive_torch_fwd_ms": round(ms, 4),
                          "naive_torch_fwd_tflops": round(ff / (ms * 1e-3) / 1e12, 2),
                          "materialised_score_bytes": w.B * w.H * w.N * w.N * es,
                          "note": "S = q k^T scale, masked_fill, softmax in fp32, P V: plain torch ops; context only"}),
              flush=True)
        return
    r = measure(fa, w, x, args.steps, args.warmup, args.settle_ms)
    ms_step, ms_fwd, ms_dkdv, ms_dq = r["ms_step"], r["ms_fwd"], r["ms_dkdv"], r["ms_dq"]
    ms_bwd = r["ms_bwd"]
    flops_fwd, flops_bwd, flops_dkdv, flops_dq = r["flops_fwd"], r["flops_bwd"], r["flops_dkdv"], r["flops_dq"]
    value = (flops_fwd + flops_bwd) / (ms_step * 1e-3) / 1e12
    kernels = {"fwd_bf16_kernel": (ms_fwd, flops_fwd), dkdv_kernel(w): (ms_dkdv, flops_dkdv),
               "bwd_dq_kernel": (ms_dq, flops_dq)}
    dom = max(kernels, key=lambda n: kernels[n][0])
    dom_ms, dom_flops = kernels[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_kernel_events": round(r["ms_step_instrumented"], 4), "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "key_padding": w.padded, "q_std": w.q_std, "parallelism": "single GPU"},
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(ms_fwd, 4), "ms_median": r["med"]["fwd"], "ms_min": r["min"]["fwd"],
                "tflops": round(flops_fwd / (ms_fwd * 1e-3) / 1e12, 2),
                "pct_of_mfma_peak": round(100 * flops_fwd / (ms_fwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "bwd": {"ms": round(ms_bwd, 4), "ms_dq": round(ms_dq, 4), "ms_dkdv": round(ms_dkdv, 4),
                "dq_includes_prepare": True,
                "ms_median": {k: r["med"][k] for k in ("dq", "dkdv")},
                "ms_min": {k: r["min"][k] for k in ("dq", "dkdv")},
                "tflops": round(flops_bwd / (ms_bwd * 1e-3) / 1e12, 2)},
        "flops": {"fwd": flops_fwd, "bwd": flops_bwd},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom, w.name), "traffic_unit": "bytes per launch",
                     "ms_per_launch": round(dom_ms, 4)},
        "bytes_per_launch": {"as_tiled_no_reuse": as_tiled_bytes(w, x),
                             "counters": {kn: measured_traffic(kn, w.name) for kn in kernels},
                             "minimum_fwd_bwd": min_bytes(w)},
    }
    if not args.no_fp8 and w.d == 128:
        out["fp8_forward"] = measure_fp8_forward(fa, w, x, args.steps, ms_fwd)
    if not args.no_dropout:
        out["dropout"] = measure_dropout(fa, w, x, 0.1, args.steps, (ms_fwd, ms_bwd))
    if not args.no_block_sparse:
        out["block_sparse"] = [measure_block_sparse(fa, w, x, pat, args.steps, (ms_fwd, ms_bwd))
                               for pat in ("local+global", "random")]
    if args.cold:
        rc = measure(fa, w, x, args.steps, args.warmup, 0.0, cold=True)
        out["cold"] = {"note": "512 MiB scratch written between steps (outside the timed kernels)",
                       "ms_fwd": round(rc["ms_fwd"], 4), "ms_bwd": round(rc["ms_bwd"], 4)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
