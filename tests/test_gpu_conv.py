"""The standalone boundary-masked depthwise conv (sfm_dwconv1d_fold) on rows of
16 or more positions, where it walks the [B*D, L] rows as one flat array (8
elements per thread, coalesced 16-byte loads and stores, the halo from the
neighbouring lanes): against the float64 oracle for every conv width and
pad_left up to K = 8, SiLU and bias, f32 and bf16, ragged totals (B*D*L not a
multiple of 8), one channel, folded rows; bit-identical to the per-row kernel
(SFM_CONV_FLAT=0) on finite inputs; and no tap ever reads another sample
(non-finite values in one sample leave the others bit-identical)."""
import os
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(B, D, L, K, io, bias, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, D, L)).astype(np.float32)
    if io == "bf16":
        x = synth.f32_to_bf16_bits(x)
    w = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32)
    bv = r.standard_normal(D).astype(np.float32) if bias else None
    return x, w, bv


def _conv(x, w, bv, P, act, B2, flat=True):
    import torch
    old = os.environ.get("SFM_CONV_FLAT")
    if not flat:
        os.environ["SFM_CONV_FLAT"] = "0"
    try:
        out = sfm.sfm_dwconv1d_fold(to_dev(x), torch.from_numpy(w).cuda(),
                                    None if bv is None else torch.from_numpy(bv).cuda(), pad_left=P, act=act, B2=B2)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("SFM_CONV_FLAT", None)
        if old is not None:
            os.environ["SFM_CONV_FLAT"] = old
    return from_dev(out)


CASES = [
    # B, D, L, K, P, act, bias, io, B2
    (4, 64, 51, 4, 1, None, False, "bf16", 1),     # stage-4 row length
    (4, 64, 51, 4, 3, "silu", True, "bf16", 4),    # causal, folded rows
    (3, 5, 17, 3, 0, None, True, "f32", 1),        # ragged total (255 elements), right halo
    (2, 1, 16, 8, 7, "silu", False, "f32", 2),     # one channel, L = 16: the widest window, causal
    (2, 7, 16, 8, 0, None, True, "bf16", 1),       # L = 16, anti-causal widest window
    (2, 9, 198, 5, 2, None, False, "bf16", 2),     # stage-3 row length, K = 5 (8-tap window)
    (2, 3, 4002, 4, 1, None, True, "bf16", 1),     # long rows
    (1, 3, 33, 1, 0, None, False, "f32", 1),       # K = 1
    (2, 6, 40, 6, 5, "silu", True, "f32", 1),      # K = 6, causal
    (3, 11, 23, 2, 1, None, False, "bf16", 3),     # odd L, folded, ragged total
]


@pytest.mark.parametrize("B,D,L,K,P,act,bias,io,B2", CASES)
def test_flat_conv_against_oracle(B, D, L, K, P, act, bias, io, B2):
    say(f"conv B={B} D={D} L={L} K={K} P={P} act={act} bias={bias} io={io} B2={B2}")
    x, w, bv = _inputs(B, D, L, K, io, bias, seed=B * 100 + D * 10 + L + K + P)
    got = _conv(x, w, bv, P, act, B2)
    xo = synth.bf16_bits_to_f64(x) if io == "bf16" else x.astype(np.float64)
    want = oracle.dwconv1d(xo, w, bv, pad_left=P, act=1 if act == "silu" else 0)
    assert_close(got, want, io, "flat conv")


@pytest.mark.parametrize("B,D,L,K,P,act,bias,io,B2", CASES[:6])
def test_flat_conv_matches_per_row_kernel(B, D, L, K, P, act, bias, io, B2):
    x, w, bv = _inputs(B, D, L, K, io, bias, seed=7 + L + K)
    assert np.array_equal(_conv(x, w, bv, P, act, B2), _conv(x, w, bv, P, act, B2, flat=False))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_flat_conv_never_mixes_samples(io):
    import torch
    B, D, L, K, P = 5, 6, 21, 4, 2
    x, w, _ = _inputs(B, D, L, K, io, False, seed=3)
    clean = _conv(x, w, None, P, None, 1)
    for poison in (np.nan, np.inf, 1e30):
        xq = x.copy()
        xq[2] = synth.f32_to_bf16_bits(np.full((D, L), poison, np.float32)) if io == "bf16" else poison
        got = _conv(xq, w, None, P, None, 1)
        assert np.array_equal(got[[0, 1, 3, 4]], clean[[0, 1, 3, 4]]), f"poison {poison} leaked"
