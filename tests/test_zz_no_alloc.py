"""sfm_selective_scan_fwd_noalloc -- the fused forward for callers that cannot
allocate device memory -- through the C ABI, against the existing workspace
entry point sfm_selective_scan_fwd_ws on the same inputs: bit-identical (same
kernels, the static scratch standing in for the workspace), on two calls in a
row, the second with smaller rows (the scratch keeps the first call's
contents), plus a shape the plan does not split (the regular forward) and the
rejection of rows that need more scratch than the static array holds."""
import sys

import numpy as np
import pytest

import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def layer(B, D, N, T, io, seed):
    import torch
    w = synth.Workload("noalloc", B=B, D=D, N=N, T=T, io=io, B2_list=(1,), K=4)
    li = synth.make_layer(w, seed=seed)
    f = lambda a: torch.from_numpy(a).cuda()
    return (to_dev(li.x), to_dev(li.delta), f(li.A), to_dev(li.Bm), to_dev(li.Cm), f(li.Dskip),
            f(li.delta_bias)), dict(conv_w=f(li.conv_w), conv_pad_left=1, flags=3)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_noalloc_matches_fwd_ws_on_two_calls(io):
    import torch
    for B, D, N, T in [(4, 128, 8, 4000), (2, 64, 8, 2000)]:  # the second call is smaller
        need = sfm.sfm_selective_scan_fwd_ws_size(B, 1, D, N, T + 2, 4, io, 3)
        say(f"noalloc B={B} D={D} N={N} T={T} io={io} scratch={need}")
        assert 0 < need <= sfm.SFM_NOALLOC_SCRATCH_BYTES
        args, kw = layer(B, D, N, T, io, seed=B + T)
        ref = sfm.sfm_selective_scan_fwd_ws(*args, **kw)
        y = torch.full_like(ref, float("nan"))
        got = sfm.sfm_selective_scan_fwd_noalloc(*args, y=y, **kw)
        torch.cuda.synchronize()
        assert got is y
        assert np.array_equal(from_dev(got), from_dev(ref))


def test_noalloc_unsplit_rows_run_the_regular_forward():
    import torch
    B, D, N, T = 8, 128, 8, 49
    assert sfm.sfm_selective_scan_fwd_ws_size(B, 1, D, N, T + 2, 4, "bf16", 3) == 0
    args, kw = layer(B, D, N, T, "bf16", seed=3)
    ref = sfm.sfm_selective_scan_fwd_ex(*args, **kw)
    got = sfm.sfm_selective_scan_fwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(got), from_dev(ref))


def test_noalloc_rejects_rows_beyond_the_scratch(monkeypatch):
    import torch
    monkeypatch.setenv("SFM_BWD_SEGMENTS", "64")  # more segments, more carries than the array holds
    B, D, N, T = 16, 320, 16, 4000
    need = sfm.sfm_selective_scan_fwd_ws_size(B, 1, D, N, T + 2, 4, "bf16", 3)
    assert need > sfm.SFM_NOALLOC_SCRATCH_BYTES
    args, kw = layer(B, D, N, T, "bf16", seed=1)
    y = torch.full((B, D, T + 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        sfm.sfm_selective_scan_fwd_noalloc(*args, y=y, **kw)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()  # nothing was launched
