"""Host-side helpers of bench.py (no GPU): the visible-pair counts behind the FLOP figures agree
with the oracle's visibility matrix counted element by element."""
import pytest

import bench
import oracle
import workloads


@pytest.mark.parametrize("N,causal,lens", [(300, True, None), (300, False, [250, 129]), (1000, True, [700]),
                                           (520, True, [520, 301]), (129, False, None)])
def test_block_pairs_match_element_count(N, causal, lens):
    B = 1 if lens is None else len(lens)
    bm = workloads.draw_block_mask(B, 2, N, "random", density=0.5, seed=3)
    want = 0
    for b in range(B):
        L = N if lens is None else lens[b]
        for h in range(2):
            want += int(oracle.visible(N, causal, L, blocks=bm[b, h]).sum())
    assert bench.block_pairs(bm, N, causal, lens) == want


@pytest.mark.parametrize("N,causal,L", [(4096, True, 4096), (512, False, 300), (1000, True, 611), (7, True, 0)])
def test_visible_pairs_match_element_count(N, causal, L):
    assert bench.visible_pairs(N, causal, L) == int(oracle.visible(N, causal, L).sum())


def _brute_kv_tiles(N, causal, L, br, bc=64):
    """Key tiles with at least one visible (query, key) pair, counted pair by pair per query block."""
    n = 0
    for q0 in range(0, N, br):
        for k0 in range(0, N, bc):
            if any((k < L) and (not causal or k <= q) for q in range(q0, min(N, q0 + br)) for k in range(k0, min(N, k0 + bc))):
                n += 1
    return n


def test_as_tiled_bytes_matches_a_brute_force_tile_count():
    import bench
    import workloads
    for N, d, causal in ((512, 128, True), (300, 64, False), (640, 64, True)):
        x = workloads.draw_custom(2, 3, N, d, dtype="bf16", causal=causal, seed=1)
        w = workloads.Workload(0, "t", 2, 3, N, d, "bf16", causal, False)
        got = bench.as_tiled_bytes(w, x)
        rows, rb = 2 * 3 * N, 2 * d
        br = 256 if d == 128 else 128
        kv = _brute_kv_tiles(N, causal, N, br) * 64 * 2 * rb * 6
        assert got["fwd_bf16_kernel"] == 2 * rows * rb + 4 * rows + kv
        kvq = _brute_kv_tiles(N, causal, N, 256) * 64 * 2 * rb * 6
        assert got["bwd_dq_kernel"] == 4 * rows * rb + 12 * rows + kvq
        bk = 256 if d == 128 else 128  # keys per workgroup of the dK/dV kernel that runs
        name = "bwd_dkdv_kl_kernel" if d == 128 else "bwd_dkdv_kernel"
        assert bench.dkdv_kernel(w) == name
        qrows = sum(sum(1 for q in range(N) if not causal or q >= k0) for k0 in range(0, N, bk)) * 6
        assert got[name] == 4 * rows * rb + qrows * (2 * rb + 8)
