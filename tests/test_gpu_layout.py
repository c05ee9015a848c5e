"""Channel-last layout ([B, L, D] activations, [B, L, N] B/C) of the fused forward.

The pages pick channel-first or channel-last per model, whichever runs faster;
the layout is a permutation of the same values, so every case here checks the
channel-last launch (a) bit for bit against the one-lane-per-channel
channel-first kernel (SFM_SCAN_SPLIT=0; its per-position arithmetic is the one
the channel-last kernel runs, while the lane-split kernel sums C.h in another
order) on the transposed tensors and (b) against the float64 oracle (computed
channel-first and transposed) with the forward's tolerance.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import selective_scan_segmented_amd as sfm
from selective_scan_segmented_amd import synth

from helpers import assert_close, from_dev, host_threads, to_dev

pytestmark = pytest.mark.gpu
CL = sfm.SFM_LAYOUT_BLD
NT = host_threads()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tr(t):
    """[B, a, b] -> [B, b, a], contiguous (device)."""
    return t.transpose(1, 2).contiguous()


def run(x, delta, A, Bm, Cm, Dk, db, cw, P, act, softplus, B2, flags, io, oracle_samples=None, cf_whole_samples=False):
    """x [B, D, T or L], delta [B, D, L], Bm/Cm [B, N, L] as numpy (f32 or bf16 bits).
    cf_whole_samples: plan the channel-first reference with one piece per folded
    row (no carried state), the layout the channel-last kernel runs, so that the
    two are comparable bit for bit (a carry adds in another order)."""
    import torch
    T_ = lambda a: torch.from_numpy(a).cuda() if a is not None else None
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    kw = dict(delta_softplus=softplus, conv_w=T_(cw), conv_pad_left=P, conv_act="silu" if act else None, B2=B2)
    saved = {k: os.environ.pop(k, None) for k in ("SFM_SCAN_WAVES", "SFM_SCAN_SPLIT")}
    try:
        os.environ["SFM_SCAN_SPLIT"] = "0"
        if cf_whole_samples:
            os.environ["SFM_SCAN_WAVES"] = "1"
        ref = sfm.sfm_selective_scan_fwd_ex(xd, dd, T_(A), Bd, Cd, T_(Dk), T_(db), flags=flags, **kw)
    finally:
        for k, v in saved.items():
            os.environ.pop(k, None)
            if v is not None:
                os.environ[k] = v
    got = sfm.sfm_selective_scan_fwd_ex(tr(xd), tr(dd), T_(A), tr(Bd), tr(Cd), T_(Dk), T_(db), flags=flags | CL,
                                        **kw)
    torch.cuda.synchronize()
    g = from_dev(tr(got))
    r = from_dev(ref)
    up = lambda a: synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    sel = slice(None) if oracle_samples is None else oracle_samples
    xo = up(x)[sel]
    if flags & sfm.SFM_FUSE_PAD:
        xo = oracle.aux_pad(xo, io)
    f64 = lambda a: a.astype(np.float64) if a is not None else None
    if cw is not None:
        want = oracle.layer(xo, up(delta)[sel], f64(A), up(Bm)[sel], up(Cm)[sel], f64(Dk), f64(db), f64(cw), None,
                            pad_left=P, act=act, softplus=softplus, nthreads=NT)
    else:
        want = oracle.selective_scan(xo, up(delta)[sel], f64(A), up(Bm)[sel], up(Cm)[sel], f64(Dk), f64(db),
                                     softplus=softplus, nthreads=NT)
    if flags & sfm.SFM_FUSE_SWAP:
        want = oracle.aux_swap(want)
    assert_close(g[sel], want, io, "channel-last vs oracle")
    if not np.array_equal(g, r):
        bad = np.argwhere(g != r)
        raise AssertionError(f"channel-last differs from channel-first at {len(bad)} of {g.size}; first "
                             f"{bad[:4].tolist()}: {[float(g[tuple(i)]) for i in bad[:4]]} vs "
                             f"{[float(r[tuple(i)]) for i in bad[:4]]}")


def random_case(B, D, N, T, K, io, seed, pad=True):
    r = np.random.default_rng(seed)
    L = T + 2
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    x = f(B, D, T if pad else L)
    delta, Bm, Cm = f(B, D, L), f(B, N, L), f(B, N, L)
    if io == "bf16":
        x, delta, Bm, Cm = map(synth.f32_to_bf16_bits, (x, delta, Bm, Cm))
    A = (-r.uniform(0.5, 4.0, (D, N))).astype(np.float32)
    Dk, db = f(D), r.uniform(-4, -1, D).astype(np.float32)
    cw = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32) if K else None
    return x, delta, A, Bm, Cm, Dk, db, cw


@pytest.mark.parametrize("B2", [1, 2])
@pytest.mark.parametrize("flags", [0, 1, 3])
def test_layout_tiny_f32(B2, flags):
    """The tiny shape (B=4 D=16 N=4 T=8), f32."""
    x, delta, A, Bm, Cm, Dk, db, cw = random_case(4, 16, 4, 8, 4, "f32", seed=flags * 3 + B2, pad=bool(flags & 1))
    run(x, delta, A, Bm, Cm, Dk, db, cw, 1, 0, True, B2, flags, "f32")


def test_layout_stage4_bf16():
    """The bench's stage-4 shape, pad and swap fused, every element against the oracle."""
    say("layout stage4")
    li = synth.make_layer(synth.WORKLOADS["stage4"], seed=1)
    run(li.x, li.delta, li.A, li.Bm, li.Cm, li.Dskip, li.delta_bias, li.conv_w, 1, 0, True, 1, 3, "bf16")


def test_layout_stage3_two_chunks():
    """L = 198 is staged in two chunks (conv halo across the cut, mean from global memory)."""
    say("layout stage3")
    li = synth.make_layer(synth.WORKLOADS["stage3"], seed=2)
    run(li.x, li.delta, li.A, li.Bm, li.Cm, li.Dskip, li.delta_bias, li.conv_w, 1, 0, True, 4, 3, "bf16",
        oracle_samples=np.array([0, 77, 255]))


@pytest.mark.parametrize("B,D,N,T,B2,K,P,act,sp,flags,io", [
    (3, 72, 5, 49, 3, 3, 0, 0, True, 3, "bf16"),     # partial tile of 8 channels, N padded to 8
    (2, 20, 16, 13, 2, 4, 3, 1, True, 3, "f32"),     # partial tile of 20 channels, causal SiLU conv
    (2, 64, 4, 30, 1, 8, 4, 0, True, 1, "bf16"),     # widest conv, pad only
    (3, 16, 8, 9, 3, 0, 0, 0, True, 2, "f32"),       # no conv, swap only
    (2, 24, 4, 11, 1, 4, 1, 0, False, 0, "f32"),     # no softplus
])
def test_layout_edges(B, D, N, T, B2, K, P, act, sp, flags, io):
    x, delta, A, Bm, Cm, Dk, db, cw = random_case(B, D, N, T, K, io, seed=B * 31 + T, pad=bool(flags & 1))
    if not sp:
        delta = np.abs(delta) * 0.05 if io == "f32" else delta
        db = None
    run(x, delta, A, Bm, Cm, Dk, db, cw, P, act, sp, B2, flags, io)


@pytest.mark.parametrize("chunk", [7, 16])
def test_layout_small_chunks(chunk, monkeypatch):
    """Ragged chunking of every sample: halo rows, the pad mean from global memory, last chunk short."""
    monkeypatch.setenv("SFM_CL_CHUNK", str(chunk))
    x, delta, A, Bm, Cm, Dk, db, cw = random_case(3, 72, 8, 38, 4, "bf16", seed=chunk)
    run(x, delta, A, Bm, Cm, Dk, db, cw, 1, 0, True, 3, 3, "bf16")


def test_layout_long_rows():
    """The long workload (L = 4002, one sample per row) in chunks."""
    say("layout long")
    li = synth.make_layer(synth.WORKLOADS["long"], seed=4)
    run(li.x, li.delta, li.A, li.Bm, li.Cm, li.Dskip, li.delta_bias, li.conv_w, 1, 0, True, 1, 3, "bf16",
        oracle_samples=np.array([0, 15]), cf_whole_samples=True)


def test_layout_rejects_unaligned_rows():
    import torch
    B, D, N, L = 2, 70, 4, 10  # 70 bf16 channels = 140 bytes: not whole 16-byte units
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sfm.SFMError):
        sfm.sfm_selective_scan_fwd_ex(z(B, L, D), z(B, L, D), torch.zeros((D, N), device="cuda"), z(B, L, N),
                                      z(B, L, N), flags=CL)
