"""The parity gates themselves, on the CPU: a bf16-rounded oracle result passes, and the local
mistakes a whole-tensor relative RMS would dilute -- one wrong row, one head slightly off -- fail."""
import torch

import oracle
import workloads
from parity_util import BF16_REL_RMS, check, rel_rms, worst_row_error, worst_slice_rel_rms


def _reference():
    x = workloads.draw_custom(2, 4, 256, 64, dtype="bf16", causal=True, q_std=2.0, seed=31)
    return oracle.backward(x["q"], x["k"], x["v"], x["do"], x["scale"], True, None)[1]  # dK, fp64


def test_rounded_reference_passes():
    ref = _reference()
    got = ref.to(torch.bfloat16)
    assert check("dk", got, ref, torch.bfloat16, "dk", []) == []


def test_one_wrong_row_fails():
    # (at 131072 rows, as in the N = 4096 workload, the same loss moves the tensor's relative RMS by
    # only about sqrt(1/131072) = 2.8e-3; the row figure does not depend on the row count)
    ref = _reference()
    got = ref.to(torch.bfloat16).clone()
    got[1, 2, 177] = 0  # one key row of 2048 lost
    assert worst_row_error(got, ref) > 0.1  # measured against the typical row norm when its own is smaller
    assert check("dk", got, ref, torch.bfloat16, "dk", []) != []


def test_one_element_of_a_row_wrong_fails():
    ref = _reference()
    got = ref.to(torch.bfloat16).clone()
    r = ref[0, 1, 100]
    got[0, 1, 100, 5] = (r[5] + 0.5 * torch.linalg.vector_norm(r)).to(torch.bfloat16)
    assert check("dk", got, ref, torch.bfloat16, "dk", []) != []


def test_one_head_slightly_off_fails_per_head_only():
    ref = _reference()
    got = ref.clone()
    got[1, 3] *= 1.012  # 1.2 % on one head of eight
    got = got.to(torch.bfloat16)
    assert rel_rms(got, ref) < BF16_REL_RMS  # diluted over eight heads
    assert worst_slice_rel_rms(got, ref) > BF16_REL_RMS
    fails = check("dk", got, ref, torch.bfloat16, "dk", [])
    assert any("head" in f for f in fails), fails
