#!/usr/bin/env python3
"""Throughput of the folded, segmented selective-scan hot path on one MI355X.

One step = the whole hot path over one batch of synthetic stage-shaped input:
  adaptive-B1 pick (host table) -> aux pad (stage entry, T -> T+2)
  -> fused boundary-masked depthwise conv + folded segmented selective scan
  -> aux head/tail swap (in place, ready for the next layer).
Inputs are resident in HBM before the timed region; the steps cycle through
enough independent input sets (>= 2 GiB) that no set is still in the 256 MB
Infinity Cache when it comes round again.

Prints ONE JSON line.  `value` is token*channels per second (token*channels =
B * D * (T + 2), aux tokens included).  The `roofline` object is for the scan
kernel, timed live with HIP events around each of its launches on the stream
it runs on; the `hbm` object gives the same kernel's algorithmic bytes against
the HBM peak; `cpu_baseline` times the CPU oracle on the same workload.

    python bench.py [--steps K] [--warmup W] [--workload stage4] [--b2 B2]
    python bench.py --mode copy    # plain 1 GiB copy, used to calibrate HBM counters
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# fp32 VALU issue rate of MI355X: 256 CUs x 4 SIMDs x 32 lanes/clock x 2.4 GHz
VALU_PEAK_TSLOT = 256 * 4 * 32 * 2.4e9 / 1e12
TRANS_SLOTS = 4  # v_exp_f32 / v_log_f32 issue at a quarter of the fp32 rate


class Hip:
    """The few HIP runtime calls the timing needs, called directly."""

    def __init__(self):
        import torch  # noqa: F401  (loads the same libamdhip64 torch uses)
        self.lib = None
        for name in ("libamdhip64.so", "libamdhip64.so.7", "libamdhip64.so.6"):
            try:
                self.lib = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if self.lib is None:
            raise RuntimeError("libamdhip64 not found")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e

    def record(self, e, stream):
        self.lib.hipEventRecord(e, stream)

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        self.lib.hipEventSynchronize(b)
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)


def scan_source_hash() -> str:
    """Hash of the code (comments and whitespace removed) of the files that
    define the channel-first scan kernel: counters taken on one version of that
    code stay valid across comment-only edits and no longer apply after any
    other change."""
    h = hashlib.sha256()
    for f in ("scan.hip", "scan_kernel.h", "sfm_device.h", "sfm_internal.h"):
        with open(os.path.join(ROOT, "selective_scan_segmented_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, b2: int):
    """HBM bytes per scan launch from the committed rocprofv3 counter summary,
    only if it was taken on the current scan source and the same launch."""
    path = os.path.join(ROOT, "profiles", f"scan_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = {k: re.search(rf"^{k}:\s*(\S+)", text, re.M) for k in ("source_hash", "b2", "bytes_per_launch")}
    if not all(m.values()):
        return None
    if m["source_hash"].group(1) != scan_source_hash() or int(m["b2"].group(1)) != b2:
        return None
    return float(m["bytes_per_launch"].group(1))


def alg_scan_bytes(w, io_bytes: int, fused_pad: bool) -> int:
    """Algorithmic HBM bytes of one scan launch: the conv input (T tokens per row
    when the aux pad is fused, else L), delta and y once each, B and C once per
    sample, and the per-channel parameters."""
    xrow = w.T if fused_pad else w.L
    return (w.B * w.D * (xrow + 2 * w.L) * io_bytes + 2 * w.B * w.N * w.L * io_bytes
            + w.D * (w.N + 3 + w.K) * 4)


def alg_scan_slots(w) -> int:
    """Algorithmic VALU work of the fused conv+scan, in fp32 issue slots:
    per (token, channel) N exp (quarter rate) and 4N mul/fma for the N states,
    softplus (exp + log, 6 fp32 ops), K conv FMAs, bias add, Delta*u, D*u."""
    per_tc = w.N * (TRANS_SLOTS + 4) + 2 * TRANS_SLOTS + 6 + w.K + 3
    return w.B * w.D * w.L * per_tc


def cpu_baseline(w, li, seconds: float):
    import numpy as np

    import oracle
    threads = oracle.threads(max(1, min(16, os.cpu_count() or 1)))
    x = li.as_f64("x")
    args = [li.as_f64(k) for k in ("delta", "A", "Bm", "Cm", "Dskip", "delta_bias", "conv_w")]
    # bounded sample: whole samples taken from the front of the batch, sized so
    # one pass of the oracle chain takes on the order of a second or two
    nb = max(1, min(w.B, int(round(w.B * 0.25))))
    xs = x[:nb]
    d, A, Bm, Cm, Dk, bias, cw = args
    d, Bm, Cm = d[:nb], Bm[:nb], Cm[:nb]
    t0 = time.perf_counter()
    passes = 0
    while True:
        xp = oracle.aux_pad(xs, w.io)
        y = oracle.layer(xp, d, A, Bm, Cm, Dk, bias, cw, pad_left=1, nthreads=threads)
        oracle.aux_swap(oracle.round_io(y, w.io))
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds or passes >= 1000:
            break
    tcs = passes * nb * w.D * w.L / el
    del np
    return {"value": tcs, "unit": "token*channels/s", "cores": threads, "kind": "oracle",
            "sample": f"{nb} of {w.B} samples (all {w.D} channels, L={w.L}) x {passes} passes of the fp64 oracle "
                      f"chain pad->conv->scan->swap, {el:.1f} s wall on {threads} threads"}


def alg_bwd_slots(w) -> int:
    """Algorithmic VALU work of the backward of the fused conv+scan, in fp32 issue
    slots: one forward (alg_scan_slots) plus the reverse step -- per state the
    gradient carry, dC, dB, du, dDelta and dA terms (10 fp32 ops) and the decay
    exp (4 slots) -- and per position the softplus and conv derivatives (~20)."""
    return alg_scan_slots(w) + w.B * w.D * w.L * (w.N * (10 + 4) + 20)


def alg_bwd_bytes(w, io_bytes: int) -> int:
    """Algorithmic HBM bytes of the backward: x (T tokens), delta, dy read and
    du (L), ddelta written in io; B and C read once per sample; dB and dC
    (float32) written once per sample; per-channel parameters and gradients."""
    return (w.B * w.D * (w.T + 4 * w.L) * io_bytes + 2 * w.B * w.N * w.L * io_bytes
            + 2 * w.B * w.N * w.L * 4 + 2 * w.D * (w.N + 3 + w.K) * 4)


def run_bwd(a, w, li, sets, prm, lib, io, io_bytes, b2, hip, sp, dev, dev_io):
    import numpy as np
    import torch
    import selective_scan_segmented_amd as sfm
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    rng = np.random.default_rng(7)
    dy32 = rng.standard_normal((w.B, w.D, w.L)).astype(np.float32)
    from selective_scan_segmented_amd import synth
    dy = dev_io(synth.f32_to_bf16_bits(dy32) if w.io == "bf16" else dy32)
    cl = a.layout == "bld"
    if cl:
        dy = dy.transpose(1, 2).contiguous()
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(dA=torch.empty((w.D, w.N), **f32), dBm=torch.empty((w.B, w.N * w.L), **f32),
             dCm=torch.empty((w.B, w.N * w.L), **f32), dDskip=torch.empty(w.D, **f32),
             ddelta_bias=torch.empty(w.D, **f32), dconv_w=torch.empty((w.D, w.K), **f32))
    flags = 3 | (sfm.SFM_LAYOUT_BLD if cl else 0)
    need = sfm.sfm_selective_scan_bwd_workspace_size(w.B // b2, b2, w.D, w.N, w.L, w.K, w.io, flags)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    calls = []
    for s in sets:
        # du / ddelta reuse the set's padded-x and y buffers ([B, D, L] io)
        calls.append((vp(s["x"]), vp(s["delta"]), vp(prm["A"]), vp(s["Bm"]), vp(s["Cm"]), vp(prm["Dskip"]),
                      vp(prm["delta_bias"]), 1, vp(prm["conv_w"]), None, w.K, 1, 0, vp(dy),
                      vp(s["xp"]), vp(s["y"]), vp(g["dA"]), vp(g["dBm"]), vp(g["dCm"]), vp(g["dDskip"]),
                      vp(g["ddelta_bias"]), vp(g["dconv_w"]), None, w.B // b2, b2, w.D, w.N, w.L, io, flags,
                      vp(ws), need, sp))
    fn = lib.sfm_selective_scan_bwd

    def step(i):
        rc = fn(*calls[i % len(calls)])
        if rc:
            raise RuntimeError(f"bwd failed: {lib.sfm_last_error().decode()}")

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    K = a.steps
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for i in range(K):
        step(a.warmup + i)
    hip.record(t1, sp)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(t0, t1) / K
    tc = w.B * w.D * w.L
    slots = alg_bwd_slots(w)
    nbytes = alg_bwd_bytes(w, io_bytes)
    alu = slots / (ms * 1e-3) / 1e12
    hbm = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "backward of the fused folded selective scan, token*channels/s (T+2 aux tokens counted)",
        "value": tc / (ms * 1e-3), "unit": "token*channels/s", "n_gpus": 1, "steps": K, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "dtype": w.io, "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} D={w.D} N={w.N} T={w.T} L={w.L} K={w.K}", "B2": b2,
                   "mode": "bwd", "input_sets": len(sets), "workspace_bytes": need,
                   "layout": "channel-last [B, L, D]" if cl else "channel-first [B, D, L]",
                   "step": "sfm_selective_scan_bwd: the backward launch (with rows split along L: "
                           "token sums, carry pass, main pass and seam launches) + the fixed-order "
                           "reduce launch of the float32 sums (pad and swap fused)"},
        "roofline": {"bound": "alu" if alu / VALU_PEAK_TSLOT >= hbm / HBM_PEAK_GBPS else "hbm",
                     "alu_achieved": round(alu, 3), "alu_peak": round(VALU_PEAK_TSLOT, 3),
                     "alu_frac": round(alu / VALU_PEAK_TSLOT, 4), "hbm_GBps": round(hbm, 1),
                     "hbm_frac": round(hbm / HBM_PEAK_GBPS, 4), "alg_valu_slots": slots, "alg_bytes": nbytes},
    }))


def run_block(a, w, hip, sp, dev):
    """Mixer-block forward (random-weight projection GEMMs around the channel-last
    scan launch) at several fold ratios B2: block time, the scan's share of it."""
    import torch

    import selective_scan_segmented_amd as sfm
    from selective_scan_segmented_amd import block, synth
    C = w.D // 2                   # model width: expand factor 2 to the scan's D channels
    R = math.ceil(C / 16)          # rank of the step projection
    bi = synth.make_block(B=w.B, T=w.T, C=C, D=w.D, N=w.N, K=w.K, R=R, io=w.io, seed=11)
    blk = block.MixerBlock(bi, device=dev)
    pick = w.B // sfm.sfm_pick_b1(w.B, w.L, w.D, w.N)
    b2s = [pick] + [b for b in (1, 2, 4, 8, 16) if b != pick and w.B % b == 0]
    rows = []
    for b2 in b2s:
        for _ in range(a.warmup):
            blk.forward(B2=b2)
        torch.cuda.synchronize()
        K = a.steps
        sev = [(hip.event(), hip.event()) for _ in range(K)]
        t0, t1 = hip.event(), hip.event()
        hip.record(t0, sp)
        for i in range(K):
            blk.forward(B2=b2, scan_events=(lambda e=sev[i][0]: hip.record(e, sp),
                                            lambda e=sev[i][1]: hip.record(e, sp)))
        hip.record(t1, sp)
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(t0, t1) / K
        scan_ms = sum(hip.elapsed_ms(e0, e1) for e0, e1 in sev) / K
        rows.append({"B2": b2, "ms_per_block": round(ms, 5), "scan_ms": round(scan_ms, 5),
                     "scan_share": round(scan_ms / ms, 3)})
    base = next(r for r in rows if r["B2"] == 1)
    for r in rows:
        r["speedup_vs_B2_1"] = round(base["ms_per_block"] / r["ms_per_block"], 3)
    top = rows[0]
    tc = w.B * w.L * w.D
    flops = block.gemm_flops(bi)
    print(json.dumps({
        "metric": "mixer-block forward, token*channels/s (scan channels, T+2 aux tokens counted)",
        "value": tc / (top["ms_per_block"] * 1e-3), "unit": "token*channels/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": top["ms_per_block"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.io, "data": "synthetic (seeded random weights and tokens)",
        "config": {"workload": f"{w.name} mixer block: B={w.B} L={w.L} C={C} D={w.D} N={w.N} K={w.K} R={R}",
                   "mode": "block", "B2": top["B2"], "layout": "channel-last [B, L, D]",
                   "step": "6 projection GEMMs + one fused conv/scan launch + silu gate + out-projection GEMM"},
        "gemm_flops_per_block": flops,
        "gemm_TFLOPs_outside_scan": round(flops / ((top["ms_per_block"] - top["scan_ms"]) * 1e-3) / 1e12, 1),
        "b2_sweep": rows,
    }))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stage4")
    ap.add_argument("--b2", type=int, default=0, help="fold ratio; 0 = adaptive-B1 table")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets; 0 = enough for 2 GiB")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["step", "copy", "scan", "bwd", "block"], default="step",
                    help="step: the whole hot path (default); scan: the scan launch alone; "
                         "bwd: the backward of the fused step (one sfm_selective_scan_bwd call); "
                         "block: a random-weight mixer block around the channel-last scan, per fold ratio; "
                         "copy: a plain 1 GiB copy (counter calibration)")
    ap.add_argument("--unfused", action="store_true",
                    help="run the step as three launches (pad, conv+scan, swap) instead of one")
    ap.add_argument("--fwd-ws", action="store_true",
                    help="run the fused step through sfm_selective_scan_fwd_ws (rows split along L across the "
                         "GPU, with a device workspace, where the plan splits them)")
    ap.add_argument("--layout", choices=["bdl", "bld"], default="bdl",
                    help="bdl: channel-first [B, D, L] (default); bld: channel-last [B, L, D] activations and "
                         "[B, L, N] B/C (fused step only)")
    a = ap.parse_args()
    if a.layout == "bld" and (a.mode not in ("step", "bwd") or a.unfused):
        raise SystemExit("--layout bld times the fused step or its backward only")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only; the hot path shards by sample "
                                   "(no collectives), so N GPUs would run N independent copies of this "
                                   "bench -- run it with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import selective_scan_segmented_amd as sfm
    from selective_scan_segmented_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    hip = Hip()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    if a.mode == "copy":
        n = 1 << 29  # 1 GiB of bf16
        src = torch.empty(n, dtype=torch.bfloat16, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sp)
        reps = 10
        for _ in range(reps):
            dst.copy_(src)
        hip.record(e1, sp)
        ms = hip.elapsed_ms(e0, e1) / reps
        print(json.dumps({"mode": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n, "ms": ms,
                          "GBps": 4 * n / ms / 1e6}))
        return

    w = synth.WORKLOADS[a.workload]
    if a.mode == "block":
        run_block(a, w, hip, sp, dev)
        return
    io_bytes = 4 if w.io == "f32" else 2
    B1 = sfm.sfm_pick_b1(w.B, w.L, w.D, w.N)
    b2 = a.b2 if a.b2 > 0 else w.B // B1
    if w.B % b2:
        raise SystemExit(f"B2={b2} must divide B={w.B}")
    li = synth.make_layer(w, seed=synth.WORKLOAD_ORDER.index(a.workload))

    def dev_io(arr):
        if arr.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)

    base = {"x": dev_io(li.x), "delta": dev_io(li.delta), "Bm": dev_io(li.Bm), "Cm": dev_io(li.Cm)}
    cl = a.layout == "bld"
    if cl:  # channel-last copies of the same values (outside the timed region)
        base = {k: v.transpose(1, 2).contiguous() for k, v in base.items()}
    prm = {k: torch.from_numpy(getattr(li, k)).to(dev) for k in ("A", "Dskip", "delta_bias", "conv_w")}
    set_bytes = sum(t.numel() * t.element_size() for t in base.values()) + 2 * w.B * w.D * w.L * io_bytes
    nsets = a.sets if a.sets > 0 else max(2, math.ceil((2 << 30) / set_bytes))
    sets = []
    for _ in range(nsets):
        s = {k: v.clone() for k, v in base.items()}
        s["xp"] = torch.empty((w.B, w.L, w.D) if cl else (w.B, w.D, w.L), dtype=base["x"].dtype, device=dev)
        s["y"] = torch.empty_like(s["xp"])
        sets.append(s)
    torch.cuda.synchronize()

    lib = sfm.load_library()
    io = 0 if w.io == "f32" else 1
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    if a.mode == "bwd":
        run_bwd(a, w, li, sets, prm, lib, io, io_bytes, b2, hip, sp, dev, dev_io)
        return
    # fused (default): one launch does pad + conv + scan + swap from the unpadded x
    fused = a.mode == "step" and not a.unfused
    calls = []
    for s in sets:
        pad_args = (vp(s["x"]), vp(s["xp"]), w.B, w.D, w.T, 0, io, sp)
        scan_in = s["x"] if fused else s["xp"]
        scan_args = (vp(scan_in), vp(s["delta"]), vp(prm["A"]), vp(s["Bm"]), vp(s["Cm"]), vp(prm["Dskip"]),
                     vp(prm["delta_bias"]), 1, vp(prm["conv_w"]), None, w.K, 1, 0, vp(s["y"]),
                     w.B // b2, b2, w.D, w.N, w.L, io, (3 | (4 if cl else 0)) if fused else 0, sp)
        swap_args = (vp(s["y"]), vp(s["y"]), w.B, w.D, w.L - 2, 1, io, sp)
        calls.append((pad_args, scan_args, swap_args))
    b1_out = ctypes.c_int64()
    ws_t = None
    if a.fwd_ws:
        if not fused or cl:
            raise SystemExit("--fwd-ws times the fused channel-first step")
        need = sfm.sfm_selective_scan_fwd_ws_size(w.B // b2, b2, w.D, w.N, w.L, w.K, w.io, 3)
        ws_t = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        pad_args, scan_args, swap_args = calls[i % nsets]
        if a.mode == "step":
            lib.sfm_pick_b1(w.B, w.L, w.D, w.N, ctypes.byref(b1_out))
        if a.mode == "step" and not fused:
            rc = lib.sfm_aux_pad_swap(*pad_args)
            if rc:
                raise RuntimeError(f"pad failed: {lib.sfm_last_error().decode()}")
        if ev is not None:
            hip.record(ev[0], sp)
        if ws_t is not None:
            rc = lib.sfm_selective_scan_fwd_ws(*scan_args[:-1], vp(ws_t), ws_t.numel(), sp)
        else:
            rc = lib.sfm_selective_scan_fwd_ex(*scan_args)
        if ev is not None:
            hip.record(ev[1], sp)
        if rc:
            raise RuntimeError(f"scan failed: {lib.sfm_last_error().decode()}")
        if a.mode == "step" and not fused:
            rc = lib.sfm_aux_pad_swap(*swap_args)
            if rc:
                raise RuntimeError(f"swap failed: {lib.sfm_last_error().decode()}")

    if a.mode == "scan":  # inputs of the scan must exist
        for s in sets:
            sfm.sfm_aux_pad_swap(s["x"], out=s["xp"], mode="pad")
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()

    K = a.steps
    # A step with one launch (the fused step, scan only) is timed by the two
    # events around the K back-to-back launches, which also give the kernel's
    # average duration (gaps between launches included); an event pair around
    # every launch would add markers to the stream and stretch each step (by
    # about 7 us at stage-4).  Steps with several launches (pad, scan, swap)
    # bracket the scan launch with its own events.
    single = fused or a.mode == "scan"
    kev = None if single else [(hip.event(), hip.event()) for _ in range(K)]
    t_start, t_end = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(t_start, sp)
    h0 = time.perf_counter()
    for i in range(K):
        step(a.warmup + i, None if single else kev[i])
    host_s = time.perf_counter() - h0
    hip.record(t_end, sp)
    torch.cuda.synchronize()
    total_ms = hip.elapsed_ms(t_start, t_end)
    if single:
        scan_avg = scan_med = total_ms / K
    else:
        scan_ms = sorted(hip.elapsed_ms(e0, e1) for e0, e1 in kev)
        scan_avg = sum(scan_ms) / K
        scan_med = scan_ms[K // 2]

    tc = w.B * w.D * w.L
    ms_per_step = total_ms / K
    value = tc / (ms_per_step * 1e-3)
    sbytes = alg_scan_bytes(w, io_bytes, fused)
    slots = alg_scan_slots(w)
    hbm_gbps = sbytes / (scan_avg * 1e-3) / 1e9
    alu = slots / (scan_avg * 1e-3) / 1e12
    hbm_frac = hbm_gbps / HBM_PEAK_GBPS
    alu_frac = alu / VALU_PEAK_TSLOT
    traffic = read_traffic(a.workload, b2)
    if alu_frac >= hbm_frac:
        roof = {"bound": "alu", "achieved": round(alu, 3), "peak": round(VALU_PEAK_TSLOT, 3),
                "unit": "T VALU-slot/s", "frac": round(alu_frac, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(hbm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(hbm_frac, 4)}
    roof["traffic"] = None if cl else traffic
    roof["kernel"] = ("sfm scan_kernel (aux pad + boundary-masked conv + folded segmented scan + aux swap, "
                      "one launch)" if fused else "sfm scan_kernel (conv + folded segmented scan)")
    if cl:
        roof["kernel"] = "sfm scan_cl_kernel (channel-last; aux pad + conv + folded segmented scan + aux swap)"
    roof["plan"] = sfm.sfm_scan_plan_string(w.B // b2, b2, w.D, w.N, w.L, w.K, w.io,
                                            (3 | (4 if cl else 0)) if fused else 0)
    roof["kernel_ms_avg"] = round(scan_avg, 5)
    roof["kernel_ms_median"] = None if single else round(scan_med, 5)
    roof["kernel_timing"] = ("HIP events around the K back-to-back launches (one launch per step)" if single else
                             "HIP events around each scan launch")
    roof["alg_bytes_per_launch"] = sbytes
    roof["alg_valu_slots_per_launch"] = slots
    out = {
        "metric": "folded selective-scan token*channels/s (T+2 aux tokens counted), % HBM peak",
        "value": value,
        "unit": "token*channels/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.io,
        "data": "synthetic (seeded SplitMix64 + Box-Muller, stage-shaped)",
        "config": {"workload": f"{w.name}: B={w.B} D={w.D} N={w.N} T={w.T} L={w.L} K={w.K}",
                   "B2": b2, "B1": w.B // b2, "mode": a.mode, "input_sets": nsets,
                   "layout": "channel-last [B, L, D]" if cl else "channel-first [B, D, L]",
                   "step": ("pick_b1 + sfm_selective_scan_fwd_ws (token sums, carry pass, output pass where "
                            "rows are split)" if ws_t is not None else
                            "pick_b1 + one launch of pad/conv/scan/swap" if fused else
                            "pick_b1 + pad + conv/scan + swap (3 launches)") if a.mode == "step" else "scan only"},
        "roofline": roof,
        "hbm": {"scan_alg_GBps": round(hbm_gbps, 1), "frac_of_8TBps": round(hbm_frac, 4)},
        "token_channels_T_only_per_s": w.B * w.D * w.T / (ms_per_step * 1e-3),
        "host_ms_per_step": host_s * 1e3 / K,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, li, a.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
