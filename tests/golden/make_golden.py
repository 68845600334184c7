"""Writes tests/golden/tiny_layer.json from the oracle alone (never from the HIP path).

The pages print no per-layer values, so this fixture only freezes the oracle's own
output on a tiny seeded workload: a later change to the oracle's arithmetic must either
reproduce it or regenerate it in a commit that names the passage justifying the change.
Run:  python tests/golden/make_golden.py"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import layer  # noqa: E402
from synth import custom_config, make_workload  # noqa: E402

CFG = dict(num_nodes=5, block=6, hidden=64, n_q=2, n_kv=1, head_dim=64, ffn=64, prefix=7,
           graph="dag", reveal=(1, 2), seed=99)
TAU = 0.05


def compute():
    cfg = custom_config(**CFG)
    w = make_workload(cfg)
    pk, pv = w.prefix_kv(0)
    out = layer(w.weights[0], w.H, w.fold_src, TAU, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv,
                eps=cfg.rms_eps)
    return dict(config=CFG, tau=TAU, fold_src=w.fold_src.tolist(),
                recompute=out["recompute"].astype(int).tolist(), src=out["src"].tolist(),
                slot_row=out["slot_row"].tolist(), K=int(out["K"]),
                y_row_sums=[[float(v) for v in r] for r in out["y"].sum(axis=2)],
                y_first8=[float(v) for v in out["y"][-1, -1, :8]])


if __name__ == "__main__":
    with open(os.path.join(HERE, "tiny_layer.json"), "w") as f:
        json.dump(compute(), f, indent=1)
