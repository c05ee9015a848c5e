"""Mixer-block timing harness: random-weight projections around the scan launch.

The pages report model-level throughput for SF-Mamba ("Seeing Both Ways,
Running One Way" 8.2; techloop walkthrough, experiments part) without the
weights or data to reproduce it.  This harness connects the kernel to that
level: one Mamba-style mixer block on channel-last tokens,

    x, z   = X W_x, X W_z                (in-projection, two GEMMs)
    B, C   = X W_b, X W_c                (state input / readout projections)
    delta  = (X W_dt1) W_dt2             (low-rank step projection)
    y      = scan(silu(conv(x)); delta, A, B, C, D, bias)   one libsfm launch, folded by B2
    out    = (y * silu(z)) W_out         (gate, out-projection GEMM)

with random weights (selective_scan_segmented_amd.synth.make_block).  The GEMMs
and the gate are PyTorch (hipBLASLt GEMMs on ROCm); the conv + scan is the C-ABI
channel-last launch (sfm_selective_scan_fwd_ex with SFM_LAYOUT_BLD).  B, C and
the step are projected from the block input rather than from the conv output,
which keeps the conv fused into the scan launch; the GEMM shapes are those of
the block.  X is the stage's already padded token sequence (the aux pad runs
once per stage, not per block).
"""
from __future__ import annotations

import numpy as np

from . import synth


class MixerBlock:
    """Device copy of a synth.BlockInputs and its forward pass."""

    def __init__(self, bi: synth.BlockInputs, device="cuda"):
        import torch
        self.bi = bi
        self.io = bi.io
        dt = torch.bfloat16 if bi.io == "bf16" else torch.float32

        def dev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        self.dtype = dt
        self.X = dev(bi.X)
        self.W = {k: dev(getattr(bi, k)) for k in ("W_x", "W_z", "W_b", "W_c", "W_dt1", "W_dt2", "W_out")}
        self.A = dev(bi.A)
        self.Dskip = dev(bi.Dskip)
        self.delta_bias = dev(bi.delta_bias)
        self.conv_w = dev(bi.conv_w)
        B, L, C, D, N, R = bi.B, bi.L, bi.C, bi.D, bi.N, bi.R
        e = lambda *s: torch.empty(s, dtype=dt, device=device)
        # activations, allocated once (the timed forward allocates nothing)
        self.buf = dict(x=e(B * L, D), z=e(B * L, D), Bm=e(B * L, N), Cm=e(B * L, N), r=e(B * L, R),
                        delta=e(B * L, D), y=e(B, L, D), s=e(B * L, D), g=e(B * L, D), out=e(B * L, C))

    def forward(self, B2: int = 1, X=None, scan_events=None):
        """One block forward on the current stream; returns out [B, L, C].
        scan_events: optional (start, end) HIP events recorded around the scan launch."""
        import torch

        import selective_scan_segmented_amd as sfm
        bi, W, b = self.bi, self.W, self.buf
        B, L, C, D, N = bi.B, bi.L, bi.C, bi.D, bi.N
        Xf = (self.X if X is None else X).view(B * L, C)
        torch.mm(Xf, W["W_x"], out=b["x"])
        torch.mm(Xf, W["W_z"], out=b["z"])
        torch.mm(Xf, W["W_b"], out=b["Bm"])
        torch.mm(Xf, W["W_c"], out=b["Cm"])
        torch.mm(Xf, W["W_dt1"], out=b["r"])
        torch.mm(b["r"], W["W_dt2"], out=b["delta"])
        if scan_events is not None:
            scan_events[0]()
        sfm.sfm_selective_scan_fwd_ex(b["x"].view(B, L, D), b["delta"].view(B, L, D), self.A,
                                      b["Bm"].view(B, L, N), b["Cm"].view(B, L, N), self.Dskip, self.delta_bias,
                                      True, self.conv_w, None, 1, "silu", y=b["y"], B2=B2,
                                      flags=sfm.SFM_LAYOUT_BLD)
        if scan_events is not None:
            scan_events[1]()
        torch.ops.aten.silu.out(b["z"], out=b["s"])
        torch.mul(b["y"].view(B * L, D), b["s"], out=b["g"])
        torch.mm(b["g"], W["W_out"], out=b["out"])
        return b["out"].view(B, L, C)


def gemm_flops(bi: synth.BlockInputs) -> int:
    """Multiply-add flops (2 per MAC) of the block's projections."""
    M = bi.B * bi.L
    return 2 * M * (bi.C * (2 * bi.D + 2 * bi.N + bi.R) + bi.R * bi.D + bi.D * bi.C)
