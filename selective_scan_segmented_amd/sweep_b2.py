"""Build the adaptive-B1 lookup table by timing the folded scan on this GPU.

The pages describe B1 as picked from an offline table keyed by batch size,
sequence length, model dimension and state size (techloop walkthrough,
"还有一个工程补充：Adaptive B1"; "Seeing Both Ways, Running One Way" 8.1 item 6),
without printing the table.  This script fills it for MI355X: for every
workload key (B, L, D, N) it times ``sfm_selective_scan_fwd_ex`` (aux pad +
conv + scan + swap in one launch, as the bench runs it) at every candidate
fold ratio B2 that divides B, over rotating input sets larger than the 256 MB
Infinity Cache, and keeps the fastest B2.

    python -m selective_scan_segmented_amd.sweep_b2 [--workloads stage4,stage3,...]
        [--write-table]   # rewrite csrc/b1_table.inc (then rebuild the library)
        [--json out.json]

Needs a GPU and the built library.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "b1_table.inc")


def _time_scan(w, B2: int, steps: int, warmup: int, min_bytes: int = 2 << 30) -> float:
    import numpy as np
    import torch

    import selective_scan_segmented_amd as sfm
    from selective_scan_segmented_amd import synth

    li = synth.make_layer(w, seed=synth.WORKLOAD_ORDER.index(w.name) if w.name in synth.WORKLOAD_ORDER else 0)
    dev = torch.device("cuda:0")

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base = dict(x=t(li.x), d=t(li.delta), B=t(li.Bm), C=t(li.Cm))
    prm = {k: torch.from_numpy(getattr(li, k)).to(dev) for k in ("A", "Dskip", "delta_bias", "conv_w")}
    eb = 2 if w.io == "bf16" else 4
    set_bytes = sum(v.numel() * v.element_size() for v in base.values()) + w.B * w.D * w.L * eb
    nsets = max(2, math.ceil(min_bytes / set_bytes))
    sets = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["y"] = torch.empty((w.B, w.D, w.L), dtype=base["x"].dtype, device=dev)
        sets.append(s)

    # The call arguments are marshalled once per set and the C entry point is
    # called directly, so host-side Python work does not floor short launches.
    lib = sfm.load_library()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    io = sfm.SFM_BF16 if w.io == "bf16" else sfm.SFM_F32
    K = prm["conv_w"].shape[1]
    calls = []
    for s in sets:
        calls.append((vp(s["x"].data_ptr()), vp(s["d"].data_ptr()), vp(prm["A"].data_ptr()), vp(s["B"].data_ptr()),
                      vp(s["C"].data_ptr()), vp(prm["Dskip"].data_ptr()), vp(prm["delta_bias"].data_ptr()), 1,
                      vp(prm["conv_w"].data_ptr()), None, K, 1, 0, vp(s["y"].data_ptr()),
                      w.B // B2, B2, w.D, w.N, w.L, io, sfm.SFM_FUSE_PAD | sfm.SFM_FUSE_SWAP, stream))
    fn = lib.sfm_selective_scan_fwd_ex

    def run(i):
        rc = fn(*calls[i % nsets])
        if rc != 0:
            raise sfm.SFMError(f"sfm_selective_scan_fwd_ex returned {rc}: {lib.sfm_last_error().decode()}")

    # untimed launches for 100 ms first: the chip's clocks ramp up under load
    # (a cold stage-4 launch takes ~10 % longer than a warm one)
    import time
    i = 0
    t_end = time.time() + 0.1
    while i < warmup or time.time() < t_end:
        run(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup = i
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del sets
    torch.cuda.empty_cache()
    return ms * 1000.0


def sweep(names, steps=50, warmup=5, reps=3):
    """Per workload, every candidate B2 timed `reps` times, the candidates
    interleaved within each repetition (so drift of the clock or of the box hits
    them alike); the median decides, the spread is kept beside it."""
    from selective_scan_segmented_amd import synth
    rows = []
    for name in names:
        w = synth.WORKLOADS[name]
        cands = [b for b in sorted(set(w.B2_list) | {1}) if w.B % b == 0]
        runs = {b2: [] for b2 in cands}
        for rep in range(reps):
            for b2 in cands:
                runs[b2].append(_time_scan(w, b2, steps, warmup))
                print(json.dumps({"workload": name, "rep": rep, "B2": b2, "us": round(runs[b2][-1], 3)}), flush=True)
        times = {b2: sorted(v)[len(v) // 2] for b2, v in runs.items()}
        spread = {b2: (max(v) - min(v)) / times[b2] for b2, v in runs.items()}
        best = min(times, key=times.get)
        rows.append({"workload": name, "B": w.B, "L": w.L, "D": w.D, "N": w.N, "times_us": times,
                     "runs_us": runs, "rel_spread": spread, "best_B2": best,
                     "speedup_best_vs_B2_1": times[1] / times[best]})
    return rows


def write_table(rows, path=TABLE):
    lines = ["// b1_table.inc -- adaptive-B1 lookup table: key (B, L, D, N) -> fold ratio B2.",
             "// Written by selective_scan_segmented_amd/sweep_b2.py from timings of",
             "// sfm_selective_scan_fwd_ex (pad + conv + scan + swap, one launch) on MI355X;",
             "// each entry keeps the fastest B2 (median of the repetitions).  Timings (us",
             "// per launch) per candidate B2:"]
    for r in rows:
        t = ", ".join(f"B2={b}: {v:.1f}" for b, v in sorted(r["times_us"].items()))
        lines.append(f"//   {r['workload']} (B={r['B']} L={r['L']} D={r['D']} N={r['N']}): {t}")
    lines.append("static const B1Entry kB1Table[] = {")
    for r in rows:
        lines.append(f"    {{{r['B']}, {r['L']}, {r['D']}, {r['N']}, {r['best_B2']}}},")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workloads", default="stage4,stage3,base_stage3,long")
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--write-table", action="store_true")
    ap.add_argument("--json", default="")
    a = ap.parse_args()
    rows = sweep(a.workloads.split(","), a.steps, a.warmup, a.reps)
    for r in rows:
        print(json.dumps({k: v for k, v in r.items() if k not in ("times_us", "runs_us")}), flush=True)
    if a.json:
        with open(a.json, "w") as f:
            json.dump(rows, f, indent=1)
    if a.write_table:
        write_table(rows)
        print(f"wrote {TABLE}; rebuild libsfm.so to use it")
    return 0


if __name__ == "__main__":
    sys.exit(main())
