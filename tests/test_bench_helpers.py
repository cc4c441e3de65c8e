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
