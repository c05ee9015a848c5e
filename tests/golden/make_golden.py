"""Writes tests/golden/tiny_chain.json from the CPU oracle only.

The pages print no worked numerical example, so this fixture freezes the
oracle's own output on the tiny workload (B=4, D=16, N=4, T=8 -> L=10, f32 io,
seed 0) for the chain that one stage entry runs:
  pad (aux head/tail = patch mean; "Seeing Both Ways, Running One Way" 3.2)
  -> boundary-masked depthwise conv (techloop walkthrough, conv-boundary section)
  -> selective scan (same page 3.1, folded with the reset of 3.3)
  -> aux swap (3.2).
Any later change to the oracle's arithmetic shows up as a mismatch here and
must name the passage that justifies it.

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from selective_scan_segmented_amd import synth  # noqa: E402


def main():
    w = synth.WORKLOADS["tiny"]
    li = synth.make_layer(w, seed=0)
    xp = oracle.aux_pad(li.as_f64("x"), "f32")
    u = oracle.round_io(oracle.dwconv1d(xp, li.as_f64("conv_w"), None, pad_left=1), "f32")
    y = oracle.selective_scan(u, li.as_f64("delta"), li.as_f64("A"), li.as_f64("Bm"), li.as_f64("Cm"),
                              li.as_f64("Dskip"), li.as_f64("delta_bias"), softplus=True)
    ys = oracle.aux_swap(y)
    doc = {
        "what": "oracle output on the tiny workload, seed 0: pad -> conv(K=4, pad_left=1) -> "
                "round to f32 -> scan (softplus, D skip) -> swap",
        "citation": "Seeing Both Ways, Running One Way: 3.1 recurrence, 3.2 aux tokens and swap, "
                    "3.3 folding with periodic reset; techloop walkthrough, conv-boundary section",
        "workload": {"B": w.B, "D": w.D, "N": w.N, "T": w.T, "L": w.L, "io": w.io, "seed": 0},
        "padded_x": [float(v) for v in xp.ravel()],
        "y_swapped": [repr(float(v)) for v in ys.ravel()],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_chain.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
    print("wrote", path)


if __name__ == "__main__":
    main()
