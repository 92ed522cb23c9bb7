"""Write the oracle's expected values for the full-size workloads.

Calls only the CPU oracle (oracle/) and the seeded input generator.  For each
workload it stores, in tests/golden/workload<k>_oracle.npz:
  logp_sum  float64 [rows]   exact per-row sums of completion log-probs
  lse       float64 [N_c]    log-sum-exp over the vocabulary at each completion
                             position, in row-major position order
  n_tokens  int64 [rows]     completion positions per row
  digest    str              sha256 of the generated input bytes, so a test can
                             tell that it regenerated the same inputs
The full forward at these sizes costs 2*N_c*H*V flops in float64 (about
1.5e13 for workload 2), so the values are computed once here rather than in
every test run.

usage: python tests/golden/make_large_golden.py 2 4 5 [3]
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import dpo_oracle as O  # noqa: E402
from preference_alignment_amd import workloads as W  # noqa: E402


def input_digest(x) -> str:
    h = hashlib.sha256()
    for a in (x.hidden, x.w_vocab, x.logits, x.targets, x.mask):
        if a is not None:
            h.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1)[: 1 << 30].tobytes())
            h.update(str(a.shape).encode())
    return h.hexdigest()


def main(ks):
    for k in ks:
        t0 = time.time()
        x = W.make_workload(k)
        dig = input_digest(x)
        if x.logits is not None:
            out = O.logits_seq_logps(x.logits, x.targets, x.mask, chunk=256)
        else:
            out = O.seq_logps(x.hidden, x.w_vocab, x.targets, x.mask, chunk=256)
        lse_c = out["lse"].reshape(-1)[out["idx"]]
        path = os.path.join(HERE, f"workload{k}_oracle.npz")
        np.savez_compressed(path, logp_sum=out["logp_sum"], lse=lse_c, n_tokens=out["n_tokens"],
                            digest=np.array(dig))
        print(f"workload {k}: N_c={lse_c.size} sums={out['logp_sum']} ({time.time() - t0:.0f} s) -> {path}",
              flush=True)


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [2, 4, 5])
