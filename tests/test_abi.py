"""The C-ABI library loads, exports every symbol include/sfm.h declares, and
rejects invalid arguments before any launch (host-only paths; no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_scan_segmented_amd as sfm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sfm.h")

OK, NULL, SHAPE, DTYPE, UNSUP, HIP, ALIAS, ALIGN = range(8)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sfm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sfm.library_path()):
        from selective_scan_segmented_amd import build
        build.build(verbose=False)
    return sfm.load_library()


def test_every_declared_symbol_is_exported(lib):
    syms = declared_symbols()
    assert {"sfm_selective_scan_fwd", "sfm_dwconv1d_fold", "sfm_aux_pad_swap", "sfm_pick_b1"} <= set(syms)
    out = subprocess.run(["nm", "-D", "--defined-only", sfm.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (sfm_[a-z0-9_]+)\b", out))
    missing = [s for s in syms if s not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for s in syms:
        assert hasattr(lib, s)


def test_status_strings_and_version(lib):
    assert lib.sfm_status_string(0) == b"ok"
    assert b"null" in lib.sfm_status_string(1)
    assert sfm.sfm_version() >= 100


P = 0x10000  # fake, never dereferenced: every call below fails validation first


def scan(lib, **kw):
    a = dict(u=P, delta=2 * P, A=3 * P, Bm=4 * P, Cm=5 * P, Dskip=None, dbias=None, sp=1, cw=None, cb=None,
             k=4, pad=1, act=0, y=6 * P, B1=2, B2=2, D=4, N=4, L=10, io=0, stream=None)
    a.update(kw)
    return lib.sfm_selective_scan_fwd(a["u"], a["delta"], a["A"], a["Bm"], a["Cm"], a["Dskip"], a["dbias"], a["sp"],
                                      a["cw"], a["cb"], a["k"], a["pad"], a["act"], a["y"], a["B1"], a["B2"],
                                      a["D"], a["N"], a["L"], a["io"], a["stream"])


def test_scan_validation(lib):
    assert scan(lib, u=None) == NULL
    assert scan(lib, y=None) == NULL
    assert scan(lib, io=7) == DTYPE
    assert scan(lib, N=0) == SHAPE
    assert scan(lib, N=17) == SHAPE
    assert scan(lib, L=0) == SHAPE
    assert scan(lib, B1=0) == SHAPE
    assert scan(lib, B2=0) == SHAPE
    assert scan(lib, D=0) == SHAPE
    assert scan(lib, sp=2) == SHAPE
    assert scan(lib, cw=7 * P, k=0) == SHAPE
    assert scan(lib, cw=7 * P, k=9) == SHAPE
    assert scan(lib, cw=7 * P, k=4, pad=4) == SHAPE
    assert scan(lib, cw=7 * P, k=4, pad=-1) == SHAPE
    assert scan(lib, cw=7 * P, act=3) == SHAPE
    assert scan(lib, u=P + 2) == ALIGN
    assert scan(lib, y=P) == ALIAS            # y on top of u
    assert scan(lib, y=5 * P + 16) == ALIAS   # y inside Cm
    assert b"overlaps" in lib.sfm_last_error()


def test_conv_validation(lib):
    f = lib.sfm_dwconv1d_fold
    assert f(None, P, None, 2 * P, 1, 1, 4, 10, 4, 1, 0, 0, None) == NULL
    assert f(P, P, None, 2 * P, 1, 1, 4, 10, 0, 0, 0, 0, None) == SHAPE
    assert f(P, P, None, 2 * P, 1, 1, 4, 10, 4, 4, 0, 0, None) == SHAPE
    assert f(P, P, None, 2 * P, 1, 1, 4, 10, 4, 1, 2, 0, None) == SHAPE
    assert f(P, P, None, 2 * P, 1, 1, 4, 10, 4, 1, 0, 5, None) == DTYPE
    assert f(P, P, None, P + 16, 1, 1, 4, 10, 4, 1, 0, 0, None) == ALIAS
    assert f(P + 4, P, None, 2 * P, 1, 1, 4, 10, 4, 1, 0, 0, None) == ALIGN


def test_aux_validation(lib):
    f = lib.sfm_aux_pad_swap
    assert f(None, P, 2, 3, 4, 0, 0, None) == NULL
    assert f(P, 2 * P, 2, 3, 0, 0, 0, None) == SHAPE      # PAD needs T >= 1
    assert f(P, 2 * P, 2, 3, 4, 2, 0, None) == SHAPE      # bad mode
    assert f(P, 2 * P, 2, 3, 4, 0, 3, None) == DTYPE
    assert f(P, P + 16, 2, 3, 4, 0, 0, None) == ALIAS     # PAD out overlaps in
    assert f(P, P + 8, 2, 3, 4, 0, 0, None) == ALIGN
    assert f(P, P + 16, 2, 3, 4, 1, 0, None) == ALIAS     # SWAP partial overlap


def test_pick_b1_returns_divisor(lib):
    for B, L, D, N in [(256, 51, 640, 8), (256, 198, 320, 8), (512, 198, 512, 16), (16, 4002, 320, 16),
                       (7, 51, 640, 8), (1, 10, 16, 4), (96, 100, 256, 8)]:
        b1 = sfm.sfm_pick_b1(B, L, D, N)
        assert 1 <= b1 <= B and B % b1 == 0
    with pytest.raises(sfm.SFMError):
        sfm.sfm_pick_b1(0, 51, 640, 8)
    assert lib.sfm_pick_b1(4, 10, 16, 4, None) == NULL


def test_pick_b1_env_table_overrides(lib, tmp_path, monkeypatch):
    t = tmp_path / "table.txt"
    t.write_text("# B L D N B2\n256 51 640 8 8\n")
    monkeypatch.setenv("SFM_B1_TABLE", str(t))
    assert sfm.sfm_pick_b1(256, 51, 640, 8) == 32
    # nearest key, then the largest divisor of B not above the table's B2
    assert sfm.sfm_pick_b1(12, 51, 640, 8) == 2


def bwd(lib, **kw):
    a = dict(u=P, delta=2 * P, A=3 * P, Bm=4 * P, Cm=5 * P, Dskip=None, dbias=None, sp=1, cw=None, cb=None, k=4,
             pad=1, act=0, dy=6 * P, du=7 * P, ddelta=8 * P, dA=9 * P, dBm=10 * P, dCm=11 * P, dD=None, db=None,
             dcw=None, dcb=None, B1=2, B2=2, D=4, N=4, L=10, io=0, flags=0, ws=12 * P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.sfm_selective_scan_bwd(
        a["u"], a["delta"], a["A"], a["Bm"], a["Cm"], a["Dskip"], a["dbias"], a["sp"], a["cw"], a["cb"], a["k"],
        a["pad"], a["act"], a["dy"], a["du"], a["ddelta"], a["dA"], a["dBm"], a["dCm"], a["dD"], a["db"], a["dcw"],
        a["dcb"], a["B1"], a["B2"], a["D"], a["N"], a["L"], a["io"], a["flags"], a["ws"], a["wsb"], a["stream"])


def test_bwd_validation(lib):
    assert bwd(lib, dy=None) == NULL
    assert bwd(lib, du=None) == NULL
    assert bwd(lib, dCm=None) == NULL
    assert bwd(lib, cw=13 * P, dcw=None) == NULL      # conv weights need their gradient
    assert bwd(lib, io=2) == DTYPE
    assert bwd(lib, N=17) == SHAPE
    assert bwd(lib, flags=8) == SHAPE                  # unknown flag
    assert bwd(lib, flags=4, D=6, io=1) == SHAPE       # channel-last rows of 6 bf16 channels: not whole 16-byte units
    assert bwd(lib, flags=1, L=2) == SHAPE             # fused pad needs L >= 3
    assert bwd(lib, cw=13 * P, dcw=14 * P, k=4, pad=4) == SHAPE
    assert bwd(lib, sp=3) == SHAPE
    assert bwd(lib, du=7 * P + 4) == ALIGN
    assert bwd(lib, du=P) == ALIAS                     # du on top of u
    assert bwd(lib, dA=8 * P + 8) == ALIAS             # dA inside ddelta
    assert bwd(lib, dD=3 * P) == ALIAS                 # dDskip on top of A
    assert bwd(lib, ws=10 * P) == ALIAS                # workspace on top of dBm
    assert bwd(lib, ws=None) == SHAPE                  # no workspace
    assert bwd(lib, wsb=16) == SHAPE                   # too small
    assert b"workspace" in lib.sfm_last_error()


def ws_expect(B1, B2, D, N, L, K):
    """Workspace floats, each region rounded up to 64: state checkpoints per (sample,
    channel tile, chunk of 32/Np positions, state, lane); partial dB/dC per (tile, sample,
    position, B|C, state); per-channel partial sums per (sample, row, channel) with
    rows dA (N), dD, dbias and, with the conv, dconv_b and dconv_w (K).  The backward
    runs unfolded, so only B = B1*B2 matters."""
    ns = 4 if N <= 4 else (8 if N <= 8 else 16)
    tiles, q = (D + 63) // 64, 32 // ns
    up = lambda v: (v + 63) // 64 * 64
    kc = N + 2 + (1 + K if K else 0)
    B = B1 * B2
    return 4 * (up(B * tiles * ((L + q - 1) // q) * ns * 64) + up(tiles * B * L * 2 * ns) + up(B * kc * D))


def test_bwd_workspace_size(lib):
    out = ctypes.c_int64(0)
    f = lib.sfm_selective_scan_bwd_workspace_size
    assert f(2, 2, 4, 4, 10, 4, 0, 0, ctypes.byref(out)) == OK
    assert out.value == ws_expect(2, 2, 4, 4, 10, 4)
    assert f(2, 2, 4, 4, 10, 0, 0, 0, ctypes.byref(out)) == OK
    assert out.value == ws_expect(2, 2, 4, 4, 10, 0)
    assert f(2, 2, 4, 4, 10, 4, 0, 0, None) == NULL
    assert f(2, 2, 4, 0, 10, 4, 0, 0, ctypes.byref(out)) == SHAPE
    assert f(2, 2, 4, 4, 10, 4, 9, 0, ctypes.byref(out)) == DTYPE
    assert sfm.sfm_selective_scan_bwd_workspace_size(256, 1, 640, 8, 51, 4, "bf16", 3) == \
        ws_expect(256, 1, 640, 8, 51, 4)
    assert sfm.sfm_selective_scan_bwd_workspace_size(64, 4, 640, 8, 51, 4, "bf16", 3) == \
        ws_expect(256, 1, 640, 8, 51, 4)


def ws_expect_split(B, D, N, L, K, segs, cps, kw):
    """Workspace floats with rows split into `segs` segments of `cps` chunks: the
    checkpoints per segment wave, the dB/dC partials, per-channel partials per
    (sample, segment), then the carries per segment wave (state, output gradient,
    two step sums), the float64 token sums per segment wave (for the fused pad's
    row mean) and the boundary partials [2][kw - 1][64]."""
    ns = 4 if N <= 4 else (8 if N <= 8 else 16)
    tiles = (D + 63) // 64
    up = lambda v: (v + 63) // 64 * 64
    kc = N + 2 + (1 + K if K else 0)
    waves = B * tiles * segs
    return 4 * (up(waves * cps * ns * 64) + up(tiles * B * L * 2 * ns) + up(B * segs * kc * D) +
                up(waves * (2 * ns + 2) * 64) + up(waves * 64 * 2) + up(waves * 2 * (kw - 1) * 64))


def test_bwd_workspace_size_channel_last_long_rows():
    """Channel-last rows too long for the whole-sample kernel run channel-first on
    transposed copies: that plan's workspace, then x, delta, dy, B, C transposed,
    then du, ddelta (io) and dB, dC (float32), each region on 256 bytes."""
    up = lambda v: (v + 255) // 256 * 256
    B, D, N, L, XL = 1, 64, 16, 4002, 4000
    cf = ws_expect_split(B, D, N, L, 4, 63, 32, 4)
    assert sfm.sfm_selective_scan_bwd_workspace_size(B, 1, D, N, L, 4, "bf16", 3) == cf
    want = up(cf) + up(B * D * XL * 2) + 4 * up(B * D * L * 2) + 2 * up(B * N * L * 2) + 2 * up(B * N * L * 4)
    assert sfm.sfm_selective_scan_bwd_workspace_size(B, 1, D, N, L, 4, "bf16", 3 | sfm.SFM_LAYOUT_BLD) == want


def test_bwd_workspace_size_split_rows():
    """Few samples x tiles (here 1 x 1) on long rows: the chunked plan splits each
    row into segments of 64 positions or more; the reported size is that layout."""
    # N = 16: chunks of 2 positions, 2001 chunks; about 8192 waves wanted, capped at
    # 64 segments of 32 chunks -> 63 segments, the last of 34 positions
    assert sfm.sfm_selective_scan_bwd_workspace_size(1, 1, 64, 16, 4002, 4, "bf16", 3) == \
        ws_expect_split(1, 64, 16, 4002, 4, 63, 32, 4)
    # 8 samples x 5 tiles = 40 waves: 205 segments wanted, capped at 64; 1001 chunks of
    # 4 positions (N = 8), 16 a segment (the 64-position floor) -> 63, the last of 34
    assert sfm.sfm_selective_scan_bwd_workspace_size(8, 1, 320, 8, 4002, 0, "bf16", 0) == \
        ws_expect_split(8, 320, 8, 4002, 0, 63, 16, 1)
    # 2 samples x 1 tile, 1001 chunks: 20 chunks for 52 wanted segments would leave a
    # last segment of 2 positions (under the window of 4), so 21 chunks -> 48
    import os
    os.environ["SFM_BWD_SEGMENTS"] = "52"
    try:
        got = sfm.sfm_selective_scan_bwd_workspace_size(2, 1, 64, 8, 4002, 4, "bf16", 0)
    finally:
        del os.environ["SFM_BWD_SEGMENTS"]
    assert got == ws_expect_split(2, 64, 8, 4002, 4, 48, 21, 4)


def test_aux_pad_bwd_validation(lib):
    fx = lib.sfm_aux_pad_bwd_ex
    assert fx(P, 2 * P, 2, 3, 4, 0, 2, None) == SHAPE     # unknown flag
    assert fx(None, P, 2, 3, 4, 0, 4, None) == NULL
    f = lib.sfm_aux_pad_bwd
    assert f(None, P, 2, 3, 4, 0, None) == NULL
    assert f(P, 2 * P, 2, 3, 0, 0, None) == SHAPE
    assert f(P, 2 * P, 2, 3, 4, 5, None) == DTYPE
    assert f(P, P + 16, 2, 3, 4, 0, None) == ALIAS
    assert f(P, P + 8, 2, 3, 4, 0, None) == ALIGN


def test_build_scratch_guard_parses_resource_remarks():
    """The build rejects forward kernels that keep state in scratch memory."""
    from selective_scan_segmented_amd import build as b
    ok = ("x.hip:1:1: remark: Function Name: k_ok [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]\n")
    bad = ("x.hip:9:1: remark: Function Name: k_bad [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 512 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:9:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:12:1: remark: Function Name: k_dyn [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:12:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:12:1: remark:     Dynamic Stack: True [-Rpass-analysis=kernel-resource-usage]\n")
    assert b.scratch_users(ok) == []
    assert b.scratch_users(ok + bad) == ["k_bad (512 bytes/lane)", "k_dyn (dynamic stack)"]
    assert "bwd.hip" in b.SPILL_OK and "scan_bf16_n8.hip" not in b.SPILL_OK


def test_fwd_ws_size():
    """The workspace-taking forward: zero (the regular forward runs) where rows are not
    split, are channel-last, or are streamed by the regular forward (the long
    workload's rows of 16 states); long rows of 8 states are split into one round
    of resident waves (21 segments for 16 samples x 5 tiles) with only the carries
    [waves][2 Np + 2][64] f32 and the float64 token sums [waves][64]."""
    assert sfm.sfm_selective_scan_fwd_ws_size(256, 1, 640, 8, 51, 4, "bf16", 3) == 0
    assert sfm.sfm_selective_scan_fwd_ws_size(16, 1, 320, 16, 4002, 4, "bf16", 3) == 0
    up = lambda v: (v + 63) // 64 * 64
    waves = 16 * 5 * 21
    assert sfm.sfm_selective_scan_fwd_ws_size(16, 1, 320, 8, 4002, 4, "bf16", 3) == \
        4 * (up(waves * 18 * 64) + up(waves * 64 * 2))
    assert sfm.sfm_selective_scan_fwd_ws_size(16, 1, 320, 8, 4002, 4, "bf16", 3 | sfm.SFM_LAYOUT_BLD) == 0


def test_plans_of_the_benchmark_workloads():
    """Host-only planner (no GPU: the device's 256 compute units are assumed, as
    on MI355X).  The launch plans the timed steps rely on: stage-4 rows whole
    on the two-lane kernel with the staggered start of its resident rounds;
    stage-3 rows whole on the four-lane kernel, the stagger also covering the
    two resident rounds of a grid larger than one round; the base model's
    stage-3 rows chunked on the two-lane kernel; the long rows streamed (16
    lanes per channel); stage-4 folded pairs on the two-lane kernel, folded
    fours on the one-lane kernel (one piece per sample)."""
    plan = lambda *a: sfm.sfm_scan_plan_string(*a)
    assert plan(256, 1, 640, 8, 51, 4, "bf16", 3) == \
        "split=2 chunk=0 ns=8 wpg=4 lds=31008 grid=1280 block=256 stagger=107/256"
    assert plan(256, 1, 320, 8, 198, 4, "bf16", 3) == \
        "split=4 chunk=0 ns=8 wpg=4 lds=69696 grid=1280 block=256 stagger=223/256"
    assert plan(512, 1, 512, 16, 198, 4, "bf16", 3).startswith("split=2 chunk=64 ns=16 ")
    assert plan(16, 1, 320, 16, 4002, 4, "bf16", 3).startswith("split=16 chunk=240 ns=16 wpg=8 ")
    assert plan(128, 2, 640, 8, 51, 4, "bf16", 3).startswith("split=2 chunk=0 ")
    assert plan(64, 4, 640, 8, 51, 4, "bf16", 3).startswith("mode=0 ch=51 pieces=4 ")
    # SFM_SCAN_STAGGER=0 turns the staggered start off
    import os
    os.environ["SFM_SCAN_STAGGER"] = "0"
    try:
        assert plan(256, 1, 320, 8, 198, 4, "bf16", 3).endswith("stagger=0/0")
    finally:
        del os.environ["SFM_SCAN_STAGGER"]
