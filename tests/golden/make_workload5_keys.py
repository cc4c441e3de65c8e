"""Write tests/golden/workload5_keys.npz: the fp64 oracle's dK and dV on the sampled key rows of every
head of the N = 65536 workload (B=1, H=8, d=64, bf16 inputs, no mask), from its seeded inputs.

Column j of dK and dV needs the log-sum-exp LSE_i and D_i = sum_c dO_ic O_ic of every one of the
65536 query rows, i.e. one complete pass of the oracle over each head (about a minute per head on
eight host cores), so it is computed once here and stored.  Only oracle/ and the seeded input
generator are called.  The file also records a SHA-256 digest of the inputs, which the GPU test
checks before it compares anything.

    python tests/golden/make_workload5_keys.py
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload5_keys.npz")


def input_digest(x) -> str:
    """SHA-256 over the bytes of q, k, v, dO (as drawn, bf16) and the sampled key indices."""
    h = hashlib.sha256()
    for name in ("q", "k", "v", "do"):
        h.update(x[name].contiguous().view(-1).view(dtype=__import__("torch").int16).numpy().tobytes())
    h.update(x["keys"].numpy().astype(np.int64).tobytes())
    return h.hexdigest()


def main():
    w = workloads.WORKLOADS[5]
    x = workloads.draw(w)
    dk_all, dv_all = [], []
    for h in range(w.H):
        t0 = time.time()
        lse, D = oracle.row_stats(x["q"], x["k"], x["v"], x["do"], x["scale"], False, None, 0, h, chunk=2048)
        dk, dv = oracle.backward_keys(x["q"], x["k"], x["v"], x["do"], x["scale"], False, None, 0, h, x["keys"][h],
                                      lse, D)
        dk_all.append(dk.numpy())
        dv_all.append(dv.numpy())
        print(f"head {h}: {time.time() - t0:.1f} s", flush=True)
    np.savez(OUT, dk=np.stack(dk_all), dv=np.stack(dv_all), keys=x["keys"].numpy().astype(np.int64),
             digest=np.array(input_digest(x)))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
