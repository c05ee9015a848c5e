"""Mixer-block harness: random-weight projections around the channel-last scan launch.

Reference: float64 numpy GEMMs and the oracle's conv + scan on the same seeded
inputs, with every intermediate the GPU stores (each GEMM output, the scan
output, silu(z), the gated product, the block output) rounded to the io type as
the GPU rounds it.  Bars: 2e-2 (bf16 io) and 1e-4 (f32 io; float32 GEMM
accumulation order differs from float64) under the forward's rule
|g - r| <= rtol (|r| + rms r).  Folding (B2) must not change a single bit.
"""
import numpy as np
import pytest

import oracle
from selective_scan_segmented_amd import block, synth

from helpers import from_dev

pytestmark = pytest.mark.gpu
RTOL = {"bf16": 2e-2, "f32": 1e-4}


def reference(bi):
    up = lambda a: synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    rnd = lambda a: oracle.round_io(a, bi.io)
    B, L, C, D, N = bi.B, bi.L, bi.C, bi.D, bi.N
    Xf = up(bi.X).reshape(B * L, C)
    x, z = rnd(Xf @ up(bi.W_x)), rnd(Xf @ up(bi.W_z))
    Bm, Cm = rnd(Xf @ up(bi.W_b)), rnd(Xf @ up(bi.W_c))
    delta = rnd(rnd(Xf @ up(bi.W_dt1)) @ up(bi.W_dt2))
    cf = lambda a, n: a.reshape(B, L, n).transpose(0, 2, 1).copy()  # channel-first for the oracle
    y = oracle.layer(cf(x, D), cf(delta, D), bi.A.astype(np.float64), cf(Bm, N), cf(Cm, N),
                     bi.Dskip.astype(np.float64), bi.delta_bias.astype(np.float64), bi.conv_w.astype(np.float64),
                     None, pad_left=1, act=1)
    y = rnd(y.transpose(0, 2, 1).reshape(B * L, D))
    s = rnd(z / (1.0 + np.exp(-z)))
    g = rnd(y * s)
    return rnd(g @ up(bi.W_out)).reshape(B, L, C)


def check(got, want, io):
    rms = float(np.sqrt(np.mean(want * want)))
    err = np.abs(got - want)
    bad = err > RTOL[io] * (np.abs(want) + rms)
    assert not bad.any(), (f"{int(bad.sum())}/{want.size} outside rtol {RTOL[io]}; worst "
                           f"{float(np.max(err / (RTOL[io] * (np.abs(want) + rms)))):.3g}")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_block_against_reference(io):
    import torch
    bi = synth.make_block(B=4, T=8, C=16, D=64, N=4, K=4, R=4, io=io, seed=3)
    blk = block.MixerBlock(bi)
    out = from_dev(blk.forward(B2=1))
    torch.cuda.synchronize()
    check(out, reference(bi), io)


def test_block_stage4_shape_and_folding():
    """The stage-4 block (C=320 -> D=640, N=8, 49 + 2 tokens, batch 16 of 256): every
    fold gives the same bits; sampled samples against the reference."""
    import torch
    bi = synth.make_block(B=16, T=49, C=320, D=640, N=8, K=4, R=20, io="bf16", seed=4)
    blk = block.MixerBlock(bi)
    ref = from_dev(blk.forward(B2=1)).copy()
    for B2 in (2, 4, 16):
        got = from_dev(blk.forward(B2=B2))
        torch.cuda.synchronize()
        assert np.array_equal(got, ref), f"B2={B2} changed the block output"
    check(ref, reference(bi), "bf16")
