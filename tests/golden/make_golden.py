"""Writes tests/golden/tiny_fp32.json from the CPU oracle.

Run from the repository root:  python tests/golden/make_golden.py
The values come from ``oracle/`` alone (inputs from the seeded generator in
``sparse_rank_attention_rope3d_amd/synth.py``); no GPU result is ever
stored here. The layer is the tiny fp32 check layer: B=1, 2 heads, D=64,
grid 4x8x8, blocks of 32, keep 2 of 8, rank 8 with the rotation after phi.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sparse_rank_attention_rope3d_amd import synth  # noqa: E402

# token rows and columns whose outputs are stored verbatim
PROBE_ROWS = [0, 31, 32, 100, 200, 255]
PROBE_COLS = [0, 7, 31, 63]


def main():
    cfg = synth.tiny()
    p = synth.lowrank_params(cfg)
    heads = []
    for h in range(cfg.H):
        q, k, v = synth.qkv_slice(cfg, 0, h)
        res = oracle.layer_slice(cfg, q, k, v, p["wq"][h], p["wk"][h], p["gate"][h])
        out = res["out"].reshape(-1, cfg.D)[:cfg.L]
        o_lr = res["o_lr"].reshape(-1, cfg.D)[:cfg.L]
        heads.append({
            "head": h,
            "idx": res["idx_ref"].tolist(),
            "kth_score": res["thr"].tolist(),
            "next_score": [float(x) for x in res["next"]],
            "out_fro": float(np.linalg.norm(out)),
            "o_lr_fro": float(np.linalg.norm(o_lr)),
            "S_fro": float(np.linalg.norm(res["S"])),
            "z": res["z"].tolist(),
            "out_probe": [[float(out[r, c]) for c in PROBE_COLS] for r in PROBE_ROWS],
        })
    doc = {
        "source": "oracle/ (fp64 CPU definition) on the tiny fp32 check layer; written by "
                  "tests/golden/make_golden.py",
        "probe_rows": PROBE_ROWS,
        "probe_cols": PROBE_COLS,
        "heads": heads,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_fp32.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
