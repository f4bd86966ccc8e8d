"""Write the oracle regression fixture `oracle_small_seed11.json`.

Calls only the seeded input generator and the CPU oracle. Re-run it only when
a change to the oracle's arithmetic is justified by a passage of the source
pages, and name that passage in the commit.
Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import ds_oracle as O  # noqa: E402
from sparse_attention_decode_04_amd import inputs as I  # noqa: E402

KV_LEN = [5, 300, 1100]
SEED = 11
SAMPLE = [(0, 0), (0, 511), (17, 100), (33, 0), (63, 511)]


def build():
    inp = I.small_rows(SEED, KV_LEN)
    res = O.decode_rows(inp)
    rows = []
    for r in res:
        rows.append(dict(
            indices=r["indices"].tolist(),
            score_sum=float(np.where(np.isfinite(r["scores"]), r["scores"], 0).astype(np.float64).sum()),
            out_sample=[float(r["out"][h, d]) for h, d in SAMPLE],
            out_abs_sum=float(np.abs(r["out"].astype(np.float64)).sum()),
        ))
    return dict(seed=SEED, kv_len=KV_LEN, sample=SAMPLE, rows=rows,
                note="written by tests/golden/make_golden.py from the CPU oracle")


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_seed11.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
