"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Every input comes from selective_scan_segmented_amd.synth; the oracle receives
the same bytes upcast to float64.  Bars: bit-exact for pad, swap and the
integer / identity scans; |g - r| <= rtol (|r| + rms r) for floating point
(rtol 1e-5 with f32 io, 2e-2 with bf16 io and float32 state).
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

NT = host_threads()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_cache = {}


def layer_inputs(name, seed=None, layer=0, a_mode="structured"):
    key = (name, seed, layer, a_mode)
    if key not in _cache:
        w = synth.WORKLOADS[name]
        _cache[key] = synth.make_layer(w, seed=synth.WORKLOAD_ORDER.index(name) if seed is None else seed,
                                       layer=layer, a_mode=a_mode)
    return _cache[key]


def dev_params(li):
    import torch
    return dict(A=torch.from_numpy(li.A).cuda(), Dskip=torch.from_numpy(li.Dskip).cuda(),
                delta_bias=torch.from_numpy(li.delta_bias).cuda(), conv_w=torch.from_numpy(li.conv_w).cuda())


def sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------------- aux pad

@pytest.mark.parametrize("name", ["tiny", "stage4", "stage3", "base_stage3", "long"])
def test_pad_bit_exact(name):
    say(f"pad {name}")
    li = layer_inputs(name)
    x = to_dev(li.x)
    out = sfm.sfm_aux_pad_swap(x, mode="pad")
    sync()
    got = from_dev(out)
    want = oracle.aux_pad(li.as_f64("x"), li.io)
    assert np.array_equal(got, want)


def test_pad_tie_rounding_bf16():
    import torch
    x = torch.tensor([[[1.0, 1.0, 1.0, 1.0 + 4 * 2**-8], [1.0, 1.0, 1.0, 1.0 + 12 * 2**-8]]],
                     dtype=torch.float64).to(torch.bfloat16).cuda()
    out = from_dev(sfm.sfm_aux_pad_swap(x, mode="pad"))
    assert out[0, 0, 0] == 1.0 and out[0, 1, 0] == 1 + 2**-6
    assert np.array_equal(out, oracle.aux_pad(from_dev(x), "bf16"))


# ------------------------------------------------------------------ aux swap

@pytest.mark.parametrize("name", ["tiny", "stage4"])
def test_swap_bit_exact(name):
    say(f"swap {name}")
    li = layer_inputs(name)
    y = to_dev(li.delta)
    want = oracle.aux_swap(li.as_f64("delta"))
    out = sfm.sfm_aux_pad_swap(y, mode="swap")          # out of place
    sync()
    assert np.array_equal(from_dev(out), want)
    sfm.sfm_aux_pad_swap(y, out=y, mode="swap")          # in place
    sync()
    assert np.array_equal(from_dev(y), want)
    sfm.sfm_aux_pad_swap(y, out=y, mode="swap")          # involution
    sync()
    assert np.array_equal(from_dev(y), li.as_f64("delta"))


# ----------------------------------------------------------------------- conv

@pytest.mark.parametrize("K,P,act,bias", [(4, 1, None, False), (4, 3, None, True), (4, 0, "silu", True),
                                          (3, 1, "silu", False), (1, 0, None, True), (8, 3, None, False),
                                          (5, 4, None, True)])
@pytest.mark.parametrize("B2", [1, 2])
def test_conv_tiny(K, P, act, bias, B2):
    import torch
    r = np.random.default_rng(K * 10 + P)
    B, D, L = 4, 16, 10
    x = r.standard_normal((B, D, L)).astype(np.float32)
    w = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32)
    bv = r.standard_normal(D).astype(np.float32) if bias else None
    out = sfm.sfm_dwconv1d_fold(to_dev(x), torch.from_numpy(w).cuda(),
                                None if bv is None else torch.from_numpy(bv).cuda(), pad_left=P, act=act, B2=B2)
    sync()
    want = oracle.dwconv1d(x, w, bv, pad_left=P, act=1 if act == "silu" else 0)
    assert_close(from_dev(out), want, "f32", "conv")


@pytest.mark.parametrize("B2", [1, 4, 32])
def test_conv_stage4(B2):
    say(f"conv stage4 B2={B2}")
    li = layer_inputs("stage4")
    xp = oracle.aux_pad(li.as_f64("x"), "bf16")
    import torch
    xp_dev = sfm.sfm_aux_pad_swap(to_dev(li.x), mode="pad")
    out = sfm.sfm_dwconv1d_fold(xp_dev, torch.from_numpy(li.conv_w).cuda(), pad_left=1, B2=B2)
    sync()
    want = oracle.dwconv1d(xp, li.as_f64("conv_w"), None, pad_left=1, nthreads=NT)
    assert_close(from_dev(out), want, "bf16", "conv stage4")


def test_conv_never_mixes_samples():
    import torch
    li = layer_inputs("tiny")
    xp = sfm.sfm_aux_pad_swap(to_dev(li.x), mode="pad")
    w = torch.from_numpy(li.conv_w).cuda()
    clean = from_dev(sfm.sfm_dwconv1d_fold(xp, w, pad_left=1, B2=4))
    for poison in (float("nan"), float("inf"), 1e30):
        xq = xp.clone()
        xq[2] = poison
        got = from_dev(sfm.sfm_dwconv1d_fold(xq, w, pad_left=1, B2=4))
        assert np.array_equal(got[[0, 1, 3]], clean[[0, 1, 3]])


# ----------------------------------------------------------------------- scan

def run_scan(li, B2, fused=True, u_dev=None, softplus=True, waves=None, **extra):
    import torch
    prm = dev_params(li)
    if u_dev is None:
        u_dev = sfm.sfm_aux_pad_swap(to_dev(li.x), mode="pad")
    old = os.environ.get("SFM_SCAN_WAVES")
    if waves is not None:
        os.environ["SFM_SCAN_WAVES"] = str(waves)
    try:
        y = sfm.sfm_selective_scan_fwd(u_dev, to_dev(li.delta), prm["A"], to_dev(li.Bm), to_dev(li.Cm),
                                       prm["Dskip"], prm["delta_bias"], delta_softplus=softplus,
                                       conv_w=prm["conv_w"] if fused else None, conv_pad_left=1, B2=B2, **extra)
        sync()
    finally:
        if waves is not None:
            if old is None:
                del os.environ["SFM_SCAN_WAVES"]
            else:
                os.environ["SFM_SCAN_WAVES"] = old
    return from_dev(y)


def oracle_layer(li, samples=None, softplus=True):
    xp = oracle.aux_pad(li.as_f64("x"), li.io)
    sel = slice(None) if samples is None else samples
    return oracle.layer(xp[sel], li.as_f64("delta")[sel], li.as_f64("A"), li.as_f64("Bm")[sel],
                        li.as_f64("Cm")[sel], li.as_f64("Dskip"), li.as_f64("delta_bias"), li.as_f64("conv_w"),
                        pad_left=1, softplus=softplus, nthreads=NT)


@pytest.mark.parametrize("B2", [1, 2, 4])
@pytest.mark.parametrize("waves", [None, 3])
def test_scan_tiny_f32(B2, waves):
    li = layer_inputs("tiny")
    got = run_scan(li, B2, waves=waves)
    assert_close(got, oracle_layer(li), "f32", f"tiny B2={B2}")


def test_scan_tiny_unfused_no_softplus():
    li = layer_inputs("tiny")
    xp = oracle.aux_pad(li.as_f64("x"), "f32")
    u = np.asarray(xp, dtype=np.float32)
    delta = np.abs(li.delta)  # positive steps without softplus
    li2 = synth.LayerInputs(io="f32", x=li.x, delta=delta.astype(np.float32), Bm=li.Bm, Cm=li.Cm, A=li.A,
                            Dskip=li.Dskip, delta_bias=np.zeros_like(li.delta_bias), conv_w=li.conv_w)
    got = run_scan(li2, 2, fused=False, u_dev=to_dev(u), softplus=False)
    want = oracle.selective_scan(xp, delta.astype(np.float64), li.as_f64("A"), li.as_f64("Bm"), li.as_f64("Cm"),
                                 li.as_f64("Dskip"), np.zeros(16), softplus=False)
    assert_close(got, want, "f32", "tiny unfused")


@pytest.mark.parametrize("B2", [1, 2, 4, 8, 16, 32])
def test_scan_stage4_every_fold(B2):
    say(f"scan stage4 B2={B2}")
    li = layer_inputs("stage4")
    got = run_scan(li, B2)
    want = _cache.setdefault(("oracle", "stage4"), None)
    if want is None:
        want = oracle_layer(li)
        _cache[("oracle", "stage4")] = want
    assert_close(got, want, "bf16", f"stage4 B2={B2}")


def test_scan_stage4_random_A_control():
    say("scan stage4 random A")
    li = layer_inputs("stage4", a_mode="random")
    samples = np.array([0, 1, 63, 64, 127, 200, 255])
    got = run_scan(li, 8)[samples]
    assert_close(got, oracle_layer(li, samples), "bf16", "stage4 random A")


@pytest.mark.parametrize("B2", [1, 2, 4, 8])
def test_chain_stage3_two_layers_with_swap(B2):
    """pad -> (conv+scan) -> swap -> (conv+scan), layers with independent draws."""
    say(f"chain stage3 B2={B2}")
    import torch
    l1, l2 = layer_inputs("stage3", layer=0), layer_inputs("stage3", layer=1)
    xp = sfm.sfm_aux_pad_swap(to_dev(l1.x), mode="pad")
    p1, p2 = dev_params(l1), dev_params(l2)
    y1 = sfm.sfm_selective_scan_fwd(xp, to_dev(l1.delta), p1["A"], to_dev(l1.Bm), to_dev(l1.Cm), p1["Dskip"],
                                    p1["delta_bias"], conv_w=p1["conv_w"], conv_pad_left=1, B2=B2)
    sfm.sfm_aux_pad_swap(y1, out=y1, mode="swap")
    y2 = sfm.sfm_selective_scan_fwd(y1, to_dev(l2.delta), p2["A"], to_dev(l2.Bm), to_dev(l2.Cm), p2["Dskip"],
                                    p2["delta_bias"], conv_w=p2["conv_w"], conv_pad_left=1, B2=B2)
    sync()
    key = ("oracle", "stage3-chain")
    if key not in _cache:
        o1 = oracle_layer(l1)
        o1s = oracle.aux_swap(oracle.round_io(o1, "bf16"))  # the layer output is stored as bf16
        o2 = oracle.layer(o1s, l2.as_f64("delta"), l2.as_f64("A"), l2.as_f64("Bm"), l2.as_f64("Cm"),
                          l2.as_f64("Dskip"), l2.as_f64("delta_bias"), l2.as_f64("conv_w"), pad_left=1, nthreads=NT)
        _cache[key] = (o1s, o2)
    o1s, o2 = _cache[key]
    assert_close(from_dev(y1), o1s, "bf16", f"stage3 layer 1 B2={B2}")
    assert_close(from_dev(y2), o2, "bf16", f"stage3 layer 2 B2={B2}")


@pytest.mark.parametrize("B2", ["lut", 1, 64])
def test_scan_base_stage3_sampled(B2):
    li = layer_inputs("base_stage3")
    w = synth.WORKLOADS["base_stage3"]
    if B2 == "lut":
        B2 = w.B // sfm.sfm_pick_b1(w.B, w.L, w.D, w.N)
    say(f"scan base_stage3 B2={B2}")
    samples = np.array([0, 1, 63, 64, 255, 256, 510, 511])
    got = run_scan(li, B2)[samples]
    assert_close(got, oracle_layer(li, samples), "bf16", f"base_stage3 B2={B2}")


@pytest.mark.parametrize("waves", [None, 1, 5])
def test_scan_long_sampled(waves):
    say(f"scan long waves={waves}")
    li = layer_inputs("long")
    samples = np.array([0, 7, 15])
    got = run_scan(li, 1, waves=waves)[samples]
    assert_close(got, oracle_layer(li, samples), "bf16", f"long waves={waves}")


# ----------------------------------------------------------- exact invariants

def _int_inputs(B, D, L, N, a_val, u=None):
    import torch
    dev = "cuda"
    u = torch.ones((B, D, L), device=dev) if u is None else u
    return dict(u=u, delta=torch.ones((B, D, L), device=dev), A=torch.full((D, N), a_val, device=dev),
                Bm=torch.ones((B, N, L), device=dev), Cm=torch.ones((B, N, L), device=dev),
                Dskip=torch.zeros(D, device=dev), delta_bias=torch.zeros(D, device=dev))


@pytest.mark.parametrize("B2,waves", [(1, None), (2, None), (4, None), (8, None), (8, 3), (8, 5), (2, 7)])
def test_integer_scan_counts_positions(B2, waves):
    """A = 0, Delta = 1, N = 1, B = C = 1, D = 0, u = 1  =>  y[b,d,t] = t + 1 exactly."""
    B, D, L = 8, 70, 37
    a = _int_inputs(B, D, L, 1, 0.0)
    old = os.environ.pop("SFM_SCAN_WAVES", None)
    if waves:
        os.environ["SFM_SCAN_WAVES"] = str(waves)
    try:
        y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=B2)
        sync()
    finally:
        os.environ.pop("SFM_SCAN_WAVES", None)
        if old is not None:
            os.environ["SFM_SCAN_WAVES"] = old
    want = np.broadcast_to(np.arange(1, L + 1, dtype=np.float64), (B, D, L))
    assert np.array_equal(from_dev(y), want)


@pytest.mark.parametrize("B2", [1, 4])
def test_identity_scan(B2):
    """A = -inf (Abar = 0), same otherwise, u unique integers < 2^24  =>  y = u exactly."""
    import torch
    B, D, L = 4, 70, 23
    u = torch.arange(B * D * L, dtype=torch.float32, device="cuda").reshape(B, D, L) + 1
    a = _int_inputs(B, D, L, 1, float("-inf"), u=u)
    y = sfm.sfm_selective_scan_fwd(**a, delta_softplus=False, B2=B2)
    sync()
    assert np.array_equal(from_dev(y), from_dev(u))


@pytest.mark.parametrize("B2,waves", [(1, None), (4, None), (4, 3)])
def test_reset_isolates_poisoned_sample(B2, waves):
    li = layer_inputs("tiny")
    clean = run_scan(li, B2, waves=waves)
    for poison in (np.nan, np.inf, 1e30):
        x = li.x.copy()
        x[1] = poison
        d = li.delta.copy()
        d[1] = poison
        lp = synth.LayerInputs(io=li.io, x=x, delta=d, Bm=li.Bm, Cm=li.Cm, A=li.A, Dskip=li.Dskip,
                               delta_bias=li.delta_bias, conv_w=li.conv_w)
        got = run_scan(lp, B2, waves=waves)
        assert np.array_equal(got[[0, 2, 3]], clean[[0, 2, 3]]), f"poison {poison} leaked"


def test_deterministic_and_every_element_written():
    import torch
    li = layer_inputs("stage4")
    prm = dev_params(li)
    xp = sfm.sfm_aux_pad_swap(to_dev(li.x), mode="pad")
    args = (xp, to_dev(li.delta), prm["A"], to_dev(li.Bm), to_dev(li.Cm), prm["Dskip"], prm["delta_bias"])
    outs = []
    for _ in range(2):
        y = torch.full_like(xp, float("nan"))
        sfm.sfm_selective_scan_fwd(*args, conv_w=prm["conv_w"], conv_pad_left=1, y=y, B2=4)
        sync()
        outs.append(from_dev(y))
    assert not np.isnan(outs[0]).any()
    assert np.array_equal(outs[0], outs[1])


# -------------------------------------------------------------- edge shapes

@pytest.mark.parametrize("B,D,N,T,B2,K,P,act", [
    (3, 70, 1, 5, 3, 4, 1, None),     # ragged channel tile, N padded to 4
    (2, 33, 3, 1, 1, 2, 0, "silu"),   # L = 3
    (4, 64, 5, 30, 2, 8, 3, None),    # N padded to 8, widest conv
    (2, 130, 12, 40, 2, 5, 4, "silu"),  # N padded to 16, right-only halo
    (6, 16, 16, 20, 6, 1, 0, None),   # B2 = B: a single folded row
    (3, 72, 8, 49, 3, 4, 1, None),    # whole-row staging with a partial 8-row tile
    (2, 8, 7, 300, 1, 3, 2, None),    # L > 256: chunked rows, carry across waves
])
def test_edge_shapes(B, D, N, T, B2, K, P, act):
    import torch
    r = np.random.default_rng(B * 1000 + D)
    L = T + 2
    x = r.standard_normal((B, D, T)).astype(np.float32)
    delta = r.standard_normal((B, D, L)).astype(np.float32)
    Bm = r.standard_normal((B, N, L)).astype(np.float32)
    Cm = r.standard_normal((B, N, L)).astype(np.float32)
    A = (-r.uniform(0.5, 4.0, (D, N))).astype(np.float32)
    Dk = r.standard_normal(D).astype(np.float32)
    db = r.uniform(-4, -1, D).astype(np.float32)
    cw = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32)
    cb = r.standard_normal(D).astype(np.float32)
    xp = sfm.sfm_aux_pad_swap(to_dev(x), mode="pad")
    T_ = lambda a: torch.from_numpy(a).cuda()
    y = sfm.sfm_selective_scan_fwd(xp, to_dev(delta), T_(A), to_dev(Bm), to_dev(Cm), T_(Dk), T_(db),
                                   conv_w=T_(cw), conv_b=T_(cb), conv_pad_left=P, conv_act=act, B2=B2)
    sync()
    xpo = oracle.aux_pad(x, "f32")
    assert np.array_equal(from_dev(xp), xpo)
    want = oracle.layer(xpo, delta, A, Bm, Cm, Dk, db, cw, cb, pad_left=P, act=1 if act == "silu" else 0)
    assert_close(from_dev(y), want, "f32", f"edge {B},{D},{N},{T}")


def test_L1_scan():
    import torch
    r = np.random.default_rng(3)
    B, D, N, L = 4, 20, 4, 1
    arrs = [r.standard_normal(s).astype(np.float32) for s in [(B, D, L), (B, D, L), (B, N, L), (B, N, L)]]
    A = -np.ones((D, N), np.float32)
    y = sfm.sfm_selective_scan_fwd(*[to_dev(a) for a in arrs[:2]], torch.from_numpy(A).cuda(),
                                   *[to_dev(a) for a in arrs[2:]], B2=2)
    sync()
    want = oracle.selective_scan(arrs[0], arrs[1], A, arrs[2], arrs[3])
    assert_close(from_dev(y), want, "f32", "L=1")


# ------------------------------------------------- fused aux pad / aux swap

FUSE_CASES = [
    # name, B2   (tiny: f32 whole rows; stage4: whole rows; stage3/base/long: chunked rows)
    ("tiny", 1), ("tiny", 2), ("stage4", 1), ("stage4", 4), ("stage3", 1), ("stage3", 8),
]


@pytest.mark.parametrize("name,B2", FUSE_CASES)
@pytest.mark.parametrize("flags", [1, 2, 3])
def test_fused_pad_swap_matches_unfused_chain(name, B2, flags):
    """sfm_selective_scan_fwd_ex(flags) is bit-identical to pad -> scan -> swap."""
    say(f"fused {name} B2={B2} flags={flags}")
    li = layer_inputs(name)
    prm = dev_params(li)
    x = to_dev(li.x)
    d, Bm, Cm = to_dev(li.delta), to_dev(li.Bm), to_dev(li.Cm)
    xp = sfm.sfm_aux_pad_swap(x, mode="pad")
    ref = sfm.sfm_selective_scan_fwd(xp, d, prm["A"], Bm, Cm, prm["Dskip"], prm["delta_bias"],
                                     conv_w=prm["conv_w"], conv_pad_left=1, B2=B2)
    if flags & 2:
        sfm.sfm_aux_pad_swap(ref, out=ref, mode="swap")
    u_in = x if flags & 1 else xp
    got = sfm.sfm_selective_scan_fwd_ex(u_in, d, prm["A"], Bm, Cm, prm["Dskip"], prm["delta_bias"],
                                        conv_w=prm["conv_w"], conv_pad_left=1, B2=B2, flags=flags)
    sync()
    assert np.array_equal(from_dev(got), from_dev(ref))


def test_fused_stage4_against_oracle():
    li = layer_inputs("stage4")
    prm = dev_params(li)
    got = sfm.sfm_selective_scan_fwd_ex(to_dev(li.x), to_dev(li.delta), prm["A"], to_dev(li.Bm), to_dev(li.Cm),
                                        prm["Dskip"], prm["delta_bias"], conv_w=prm["conv_w"], conv_pad_left=1,
                                        B2=1, flags=3)
    sync()
    key = ("oracle", "stage4")
    if key not in _cache:
        _cache[key] = oracle_layer(li)
    assert_close(from_dev(got), oracle.aux_swap(_cache[key]), "bf16", "fused stage4")


@pytest.mark.parametrize("name", ["base_stage3", "long"])
def test_fused_sampled_against_oracle(name):
    say(f"fused sampled {name}")
    li = layer_inputs(name)
    prm = dev_params(li)
    w = synth.WORKLOADS[name]
    B2 = w.B // sfm.sfm_pick_b1(w.B, w.L, w.D, w.N)
    got = sfm.sfm_selective_scan_fwd_ex(to_dev(li.x), to_dev(li.delta), prm["A"], to_dev(li.Bm), to_dev(li.Cm),
                                        prm["Dskip"], prm["delta_bias"], conv_w=prm["conv_w"], conv_pad_left=1,
                                        B2=B2, flags=3)
    sync()
    samples = np.array([0, w.B // 2, w.B - 1])
    want = oracle.aux_swap(oracle_layer(li, samples))
    assert_close(from_dev(got)[samples], want, "bf16", f"fused {name}")


@pytest.mark.parametrize("B,D,N,T,B2,K,P,io", [
    (3, 70, 5, 49, 3, 4, 1, "bf16"),    # ragged tile, odd L, whole rows
    (3, 72, 8, 49, 1, 4, 1, "bf16"),    # whole-row staging with a partial 8-row tile
    (2, 40, 8, 299, 1, 4, 2, "bf16"),   # odd L > 256: element staging, chunked mean
    (2, 72, 16, 300, 2, 3, 0, "f32"),   # chunked tiles in f32
    (4, 8, 4, 1, 2, 2, 1, "f32"),       # T = 1: mean of a single token
])
def test_fused_edge_shapes(B, D, N, T, B2, K, P, io):
    import torch
    r = np.random.default_rng(T * 7 + D)
    L = T + 2
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    x, delta, Bm, Cm = f(B, D, T), f(B, D, L), f(B, N, L), f(B, N, L)
    if io == "bf16":
        cast = lambda a: synth.f32_to_bf16_bits(a)
    else:
        cast = lambda a: a
    x, delta, Bm, Cm = map(cast, (x, delta, Bm, Cm))
    A = (-r.uniform(0.5, 4.0, (D, N))).astype(np.float32)
    Dk, db = f(D), r.uniform(-4, -1, D).astype(np.float32)
    cw = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32)
    T_ = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    xp = sfm.sfm_aux_pad_swap(xd, mode="pad")
    ref = sfm.sfm_selective_scan_fwd(xp, dd, T_(A), Bd, Cd, T_(Dk), T_(db), conv_w=T_(cw), conv_pad_left=P, B2=B2)
    sfm.sfm_aux_pad_swap(ref, out=ref, mode="swap")
    got = sfm.sfm_selective_scan_fwd_ex(xd, dd, T_(A), Bd, Cd, T_(Dk), T_(db), conv_w=T_(cw), conv_pad_left=P,
                                        B2=B2, flags=3)
    sync()
    assert np.array_equal(from_dev(got), from_dev(ref))
    up = lambda a: synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    want = oracle.aux_swap(oracle.layer(oracle.aux_pad(up(x), io), up(delta), A, up(Bm), up(Cm), Dk, db, cw,
                                        pad_left=P))
    assert_close(from_dev(got), want, io, "fused edge")


def test_fused_pad_rejects_short_rows():
    import torch
    u = torch.zeros((2, 4, 1), device="cuda")  # L - 2 = 1 -> L = 3 is fine; L = 2 is not expressible here
    A = torch.zeros((4, 2), device="cuda")
    BC = torch.zeros((2, 2, 3), device="cuda")
    sfm.sfm_selective_scan_fwd_ex(u, torch.zeros((2, 4, 3), device="cuda"), A, BC, BC, flags=1)
    lib = sfm.load_library()
    rc = lib.sfm_selective_scan_fwd_ex(u.data_ptr(), u.data_ptr(), A.data_ptr(), BC.data_ptr(), BC.data_ptr(),
                                       None, None, 1, None, None, 0, 0, 0, A.data_ptr(), 2, 1, 4, 2, 2, 0, 1, None)
    assert rc == 2  # SFM_ERR_SHAPE: SFM_FUSE_PAD needs L >= 3


# --------------------------------------------- double-buffered chunk staging

@pytest.mark.parametrize("stages", [1, 2])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("ch", [6, 7, 16])
def test_chunk_pipeline_against_oracle(ch, io, stages):
    """Tile staging with forced chunk sizes (odd ones start chunks mid-word in
    bf16) and one or two LDS stages per wave: fused pad/swap with two samples
    per wave (B2 = 16 over 8 pieces), unfused with pieces that cut samples
    (carries), a partial channel tile."""
    import torch
    say(f"chunk pipeline ch={ch} io={io} stages={stages}")
    B, D, N, T, K, P = 16, 72, 8, 58, 4, 1
    L = T + 2
    r = np.random.default_rng(ch * 31 + len(io))
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    x, delta, Bm, Cm = f(B, D, T), f(B, D, L), f(B, N, L), f(B, N, L)
    cast = synth.f32_to_bf16_bits if io == "bf16" else (lambda a: a)
    x, delta, Bm, Cm = map(cast, (x, delta, Bm, Cm))
    A = (-r.uniform(0.5, 4.0, (D, N))).astype(np.float32)
    Dk, db = f(D), r.uniform(-4, -1, D).astype(np.float32)
    cw = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32)
    T_ = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    up = lambda a: synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    xp64 = oracle.aux_pad(up(x), io)
    want = oracle.layer(xp64, up(delta), A, up(Bm), up(Cm), Dk, db, cw, pad_left=P)
    saved = {k: os.environ.pop(k, None) for k in ("SFM_SCAN_CHUNK", "SFM_SCAN_WAVES", "SFM_SCAN_STAGES")}
    try:
        os.environ["SFM_SCAN_CHUNK"] = str(ch)
        os.environ["SFM_SCAN_STAGES"] = str(stages)
        plan = sfm.sfm_scan_plan_string(1, B, D, N, L, K, io, 3)
        assert "mode=1" in plan and f"stages={stages}" in plan
        fused = sfm.sfm_selective_scan_fwd_ex(xd, dd, T_(A), Bd, Cd, T_(Dk), T_(db), conv_w=T_(cw),
                                              conv_pad_left=P, B2=B, flags=3)
        xp = sfm.sfm_aux_pad_swap(xd, mode="pad")
        sync()
        assert np.array_equal(from_dev(xp), xp64)
        os.environ["SFM_SCAN_WAVES"] = "3"
        assert "carry=1" in sfm.sfm_scan_plan_string(1, B, D, N, L, K, io, 0)
        carried = sfm.sfm_selective_scan_fwd(xp, dd, T_(A), Bd, Cd, T_(Dk), T_(db), conv_w=T_(cw),
                                             conv_pad_left=P, B2=B)
        sync()
    finally:
        for k, v in saved.items():
            os.environ.pop(k, None)
            if v is not None:
                os.environ[k] = v
    assert_close(from_dev(fused), oracle.aux_swap(want), io, f"fused ch={ch}")
    assert_close(from_dev(carried), want, io, f"carried ch={ch}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("waves,ch", [(3, 16), (5, 7), (8, 32)])
def test_fused_pad_swap_with_carries(waves, ch, io):
    """Fused pad/swap on tile-staged rows whose pieces cut samples (carried
    state): the pieces holding a sample's ends take the row mean and write the
    swapped ends themselves.  Bit-identical to pad -> scan -> swap with the same
    pieces, and within tolerance of the oracle."""
    import torch
    say(f"fused carries waves={waves} ch={ch} io={io}")
    B, D, N, T, K, P = 3, 72, 8, 298, 4, 1
    L = T + 2
    r = np.random.default_rng(waves * 13 + ch + len(io))
    f = lambda *s: r.standard_normal(s).astype(np.float32)
    x, delta, Bm, Cm = f(B, D, T), f(B, D, L), f(B, N, L), f(B, N, L)
    cast = synth.f32_to_bf16_bits if io == "bf16" else (lambda a: a)
    x, delta, Bm, Cm = map(cast, (x, delta, Bm, Cm))
    A = (-r.uniform(0.5, 4.0, (D, N))).astype(np.float32)
    Dk, db = f(D), r.uniform(-4, -1, D).astype(np.float32)
    cw = r.uniform(-0.5, 0.5, (D, K)).astype(np.float32)
    T_ = lambda a: torch.from_numpy(a).cuda()
    xd, dd, Bd, Cd = map(to_dev, (x, delta, Bm, Cm))
    up = lambda a: synth.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
    want = oracle.aux_swap(oracle.layer(oracle.aux_pad(up(x), io), up(delta), A, up(Bm), up(Cm), Dk, db, cw,
                                        pad_left=P))
    saved = {k: os.environ.pop(k, None) for k in ("SFM_SCAN_CHUNK", "SFM_SCAN_WAVES", "SFM_SCAN_STAGES")}
    try:
        os.environ["SFM_SCAN_WAVES"] = str(waves)
        os.environ["SFM_SCAN_CHUNK"] = str(ch)
        plan = sfm.sfm_scan_plan_string(B, 1, D, N, L, K, io, 3)
        assert "mode=1" in plan and "carry=1" in plan, plan
        got = sfm.sfm_selective_scan_fwd_ex(xd, dd, T_(A), Bd, Cd, T_(Dk), T_(db), conv_w=T_(cw),
                                            conv_pad_left=P, B2=1, flags=3)
        xp = sfm.sfm_aux_pad_swap(xd, mode="pad")
        ref = sfm.sfm_selective_scan_fwd(xp, dd, T_(A), Bd, Cd, T_(Dk), T_(db), conv_w=T_(cw),
                                         conv_pad_left=P, B2=1)
        sfm.sfm_aux_pad_swap(ref, out=ref, mode="swap")
        sync()
    finally:
        for k, v in saved.items():
            os.environ.pop(k, None)
            if v is not None:
                os.environ[k] = v
    assert np.array_equal(from_dev(got), from_dev(ref))
    assert_close(from_dev(got), want, io, f"fused carries waves={waves}")
