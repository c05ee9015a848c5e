"""The flat forms of the standalone aux pad and aux swap: the pad's shifted
copy over the whole [rows, L] output plus one lane per row for the float64
index-order mean (rows of 64 or more tokens, or forced with SFM_PAD_FLAT=1),
and the 16-byte swap copy.  Bit-exact against the oracle and against the staged
pad kernel (SFM_PAD_FLAT=0), f32 and bf16, ragged totals, single rows, rows
shorter than a 16-byte group."""
import os
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class env:
    def __init__(self, **kv):
        self.kv = kv

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kv}
        for k, v in self.kv.items():
            os.environ[k] = str(v)

    def __exit__(self, *a):
        for k, v in self.old.items():
            os.environ.pop(k, None)
            if v is not None:
                os.environ[k] = v


def _x(B, D, T, io, seed):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((B, D, T)) * np.exp2(r.integers(-6, 6, (B, D, T)))).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if io == "bf16" else x


def _up(a):
    return synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


PAD_CASES = [
    # B, D, T, io, flat
    (3, 5, 64, "bf16", -1),    # the shortest rows the flat form takes by default
    (2, 7, 196, "bf16", -1),   # stage-3 rows
    (2, 3, 4000, "bf16", -1),  # long rows: 16-byte loads for the sums
    (3, 5, 65, "f32", -1),     # odd row length (f32 rows start on words)
    (2, 3, 130, "f32", -1),    # f32 with 16-byte unit rows plus a tail
    (1, 1, 70, "bf16", -1),    # a single row
    (4, 3, 2, "bf16", 1),      # forced on rows shorter than a 16-byte group (L = 4)
    (3, 3, 7, "f32", 1),       # forced, ragged total
    (2, 5, 46, "bf16", 1),     # forced, even L below the default threshold
]


@pytest.mark.parametrize("B,D,T,io,flat", PAD_CASES)
def test_flat_pad_bit_exact(B, D, T, io, flat):
    say(f"pad flat B={B} D={D} T={T} io={io}")
    x = _x(B, D, T, io, seed=B + D + T)
    want = oracle.aux_pad(_up(x), io)
    with env(SFM_PAD_FLAT=flat):
        got = from_dev(sfm.sfm_aux_pad_swap(to_dev(x), mode="pad"))
    with env(SFM_PAD_FLAT=0):
        staged = from_dev(sfm.sfm_aux_pad_swap(to_dev(x), mode="pad"))
    assert np.array_equal(got, want)
    assert np.array_equal(got, staged)


@pytest.mark.parametrize("B,D,L,io", [(3, 5, 51, "bf16"), (2, 3, 3, "bf16"), (4, 2, 2, "f32"), (3, 7, 17, "f32"),
                                      (2, 9, 198, "bf16"), (1, 1, 1, "f32")])
def test_swap_copy_bit_exact(B, D, L, io):
    say(f"swap copy B={B} D={D} L={L} io={io}")
    y = _x(B, D, L, io, seed=L)
    got = from_dev(sfm.sfm_aux_pad_swap(to_dev(y), mode="swap"))
    assert np.array_equal(got, oracle.aux_swap(_up(y)))
