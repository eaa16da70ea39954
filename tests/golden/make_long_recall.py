"""Writes long_recall.json: the CPU oracle's recall of the planted bindings of
the long-context workload (one sequence of 131072 tokens, 2^20 slots, 64
bindings each planted 16 times), after 1, 2, 3 and 4 passes from the same
initial state.

Only the oracle computes here (fp64 C, OpenMP; no GPU code is imported).  A
pass p of a 4-pass run is pass p of a p-pass run (each pass restarts at
token 0 with the state carried, and the last token of a pass has no
target), so one run of four single-pass calls gives every pass count.  The
inputs are the workload's seeded tokens and its state drawn on the CPU; the
file records their digests so a reader can tell it was made from the same
bits.  Takes about ten minutes on eight cores:

    python tests/golden/make_long_recall.py
"""
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from sparse_weight_memory_sub_amd.workloads import WORKLOADS, make_state, make_tokens, planted_recall  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_recall.json")


def digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()[:16]


def main():
    wl = WORKLOADS["long"]
    cfg, T = wl.cfg, wl.T
    q, v, g, extra = make_tokens(cfg, 1, T, wl.seed, wl.kind)
    K1, K2, V = make_state(cfg, 1, wl.seed)
    pv, pos = extra["plant_v"], extra["plant_pos"]
    first, last = pos.min(1).values, pos.max(1).values
    res = {"workload": wl.description, "seed": wl.seed, "T": T, "n_bind": int(pv.shape[0]), "reps": int(pos.shape[1]),
           "digest_tokens": digest(q, v, g), "digest_state": digest(K1, K2, V),
           "threads": oracle.num_threads(), "passes": {}}
    state = (K1, K2, V)
    for p in range(1, 5):
        t0 = time.time()
        out = oracle.forward_seq(cfg, q, v, g, *state, passes=1)
        state = (out["K1"], out["K2"], out["V"])
        vh = torch.from_numpy(out["vhat"][0])
        rf, af, mf = planted_recall(vh[first], pv)
        rl, al, ml = planted_recall(vh[last], pv)
        res["passes"][str(p)] = {"recall_first": rf, "recall_last": rl, "argmax_first": af, "argmax_last": al,
                                 "margin_first": [round(x, 6) for x in mf], "margin_last": [round(x, 6) for x in ml],
                                 "oracle_s": round(time.time() - t0, 1)}
        print(f"pass {p}: recall first {rf:.4f} last {rl:.4f} ({time.time() - t0:.0f} s)", flush=True)
        del out, vh
    with open(OUT, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
