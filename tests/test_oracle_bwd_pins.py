"""Pins for the oracle's backward (test infrastructure checking test infrastructure).

The pages define the forward only; the backward oracle is the chain rule of
that definition.  It is pinned here by things other than itself:
  * central finite differences of the oracle's own forward (pad -> conv ->
    scan -> swap, float64) for every entry of every input, on tiny shapes;
  * reverse-mode autodiff (torch, float64, CPU) of an independent forward
    written below with plain torch ops;
  * structural facts: the softplus threshold, the reset cutting all gradient
    flow between samples, linearity in the upstream gradient.
"""
import numpy as np
import pytest

import oracle


def _case(seed, B=2, D=3, N=4, T=4, K=4, bias_scale=0.5):
    r = np.random.default_rng(seed)
    L = T + 2
    c = dict(
        x=r.standard_normal((B, D, L)),
        delta=r.standard_normal((B, D, L)),
        A=-np.exp(0.5 * r.standard_normal((D, N))),
        Bm=r.standard_normal((B, N, L)),
        Cm=r.standard_normal((B, N, L)),
        Dskip=r.standard_normal(D),
        delta_bias=bias_scale * r.standard_normal(D),
        conv_w=r.standard_normal((D, K)) * 0.5,
        conv_b=r.standard_normal(D) * 0.1,
        dy=r.standard_normal((B, D, L)),
    )
    return c


def _forward(c, conv, P, act, softplus, pad, swap):
    x = c["x"]
    if pad:
        x = oracle.aux_pad(x[:, :, 1:-1], "f64")  # the unpadded input is x[..., 1:-1]
    if conv:
        u = oracle.dwconv1d(x, c["conv_w"], c["conv_b"], pad_left=P, act=act)
    else:
        u = x
    y = oracle.selective_scan(u, c["delta"], c["A"], c["Bm"], c["Cm"], c["Dskip"], c["delta_bias"], softplus)
    if swap:
        y = oracle.aux_swap(y)
    return y


def _loss(c, **kw):
    return float(np.sum(c["dy"] * _forward(c, **kw)))


def _grads(c, conv, P, act, softplus, pad, swap):
    x = c["x"][:, :, 1:-1] if pad else c["x"]
    return oracle.layer_bwd(x, c["delta"], c["A"], c["Bm"], c["Cm"], c["Dskip"], c["delta_bias"], c["dy"],
                            c["conv_w"] if conv else None, c["conv_b"] if conv else None, P, act, softplus,
                            fuse_pad=pad, fuse_swap=swap)


NAMES = {"x": "dx", "delta": "ddelta", "A": "dA", "Bm": "dBm", "Cm": "dCm", "Dskip": "dDskip",
         "delta_bias": "ddelta_bias", "conv_w": "dconv_w", "conv_b": "dconv_b"}


@pytest.mark.parametrize("conv,P,act,softplus,pad,swap", [
    (True, 1, 0, True, False, False),
    (True, 2, 1, True, False, False),     # SiLU, right-heavy halo
    (True, 0, 0, False, False, False),    # no softplus
    (False, 0, 0, True, False, False),    # scan only
    (True, 1, 1, True, True, True),       # the fused stage chain pad -> conv -> scan -> swap
])
def test_bwd_matches_finite_differences(conv, P, act, softplus, pad, swap):
    c = _case(7 + P + 3 * act)
    kw = dict(conv=conv, P=P, act=act, softplus=softplus, pad=pad, swap=swap)
    g = _grads(c, **kw)
    eps = 1e-6
    for name, gname in NAMES.items():
        if not conv and name in ("conv_w", "conv_b"):
            continue
        arr = c[name]
        want = g[gname]
        if name == "x" and pad:
            arr_view = arr[:, :, 1:-1]          # only the unpadded tokens are inputs
        else:
            arr_view = arr
        fd = np.zeros(arr_view.shape)
        for idx in np.ndindex(arr_view.shape):
            full = idx if not (name == "x" and pad) else (idx[0], idx[1], idx[2] + 1)
            old = arr[full]
            arr[full] = old + eps
            lp = _loss(c, **kw)
            arr[full] = old - eps
            lm = _loss(c, **kw)
            arr[full] = old
            fd[idx] = (lp - lm) / (2 * eps)
        scale = np.abs(fd).max() + 1e-12
        err = np.abs(fd - want).max() / scale
        assert err < 2e-6, f"{gname}: rel err {err:.2e}"


def _torch_forward(t, x, delta, A, Bm, Cm, Dskip, bias, w, cb, P, act, softplus):
    """Independent forward with plain torch ops (float64): conv via explicit
    zero-padded taps, scan as an explicit loop over positions."""
    B, D, L = x.shape
    K = w.shape[1]
    xp = t.nn.functional.pad(x, (P, K - 1 - P))
    z = cb[None, :, None] + sum(w[None, :, j, None] * xp[:, :, j:j + L] for j in range(K))
    u = t.nn.functional.silu(z) if act == 1 else z
    v = delta + bias[None, :, None]
    dt = t.nn.functional.softplus(v) if softplus else v
    h = t.zeros(B, D, A.shape[1], dtype=x.dtype)
    ys = []
    for i in range(L):
        bx = dt[:, :, i, None] * Bm[:, None, :, i] * u[:, :, i, None]
        if i == 0:
            h = bx
        else:
            h = t.exp(dt[:, :, i, None] * A[None]) * h + bx
        ys.append((h * Cm[:, None, :, i]).sum(-1) + Dskip[None, :] * u[:, :, i])
    return t.stack(ys, dim=-1)


@pytest.mark.parametrize("act,softplus", [(0, True), (1, True), (1, False)])
def test_bwd_matches_torch_autograd(act, softplus):
    import torch
    c = _case(21 + act, B=3, D=4, N=5, T=7)
    P = 1
    names = ["x", "delta", "A", "Bm", "Cm", "Dskip", "delta_bias", "conv_w", "conv_b"]
    ts = {k: torch.tensor(c[k], dtype=torch.float64, requires_grad=True) for k in names}
    y = _torch_forward(torch, ts["x"], ts["delta"], ts["A"], ts["Bm"], ts["Cm"], ts["Dskip"], ts["delta_bias"],
                       ts["conv_w"], ts["conv_b"], P, act, softplus)
    (y * torch.tensor(c["dy"])).sum().backward()
    g = _grads(c, conv=True, P=P, act=act, softplus=softplus, pad=False, swap=False)
    for k in names:
        want = ts[k].grad.numpy()
        got = g[NAMES[k]]
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12, err_msg=k)


def test_softplus_threshold_derivative_is_one():
    # v = delta + bias > 20 everywhere: Delta = v exactly, so dDelta/dv = 1 exactly
    c = _case(3, bias_scale=0.0)
    c["delta"] = 25.0 + np.abs(c["delta"])
    c["A"] = -np.full_like(c["A"], 1e-3)
    g_sp = _grads(c, conv=True, P=1, act=0, softplus=True, pad=False, swap=False)
    g_id = _grads(c, conv=True, P=1, act=0, softplus=False, pad=False, swap=False)
    for k in g_sp:
        np.testing.assert_array_equal(g_sp[k], g_id[k], err_msg=k)


def test_reset_isolates_samples():
    # upstream gradient only on sample 1: every gradient of sample 0's inputs is zero
    c = _case(5, B=2)
    c["dy"][0] = 0.0
    g = _grads(c, conv=True, P=1, act=1, softplus=True, pad=False, swap=False)
    assert np.all(g["dx"][0] == 0) and np.all(g["ddelta"][0] == 0)
    assert np.all(g["dBm"][0] == 0) and np.all(g["dCm"][0] == 0)
    # and sample 1's gradients do not depend on sample 0's inputs
    c2 = {k: v.copy() for k, v in c.items()}
    for k in ("x", "delta", "Bm", "Cm"):
        c2[k][0] = 123.0
    g2 = _grads(c2, conv=True, P=1, act=1, softplus=True, pad=False, swap=False)
    for k in ("dx", "ddelta", "dBm", "dCm"):
        np.testing.assert_array_equal(g[k][1], g2[k][1], err_msg=k)


def test_bwd_is_linear_in_dy():
    c = _case(11)
    kw = dict(conv=True, P=1, act=1, softplus=True, pad=True, swap=True)
    dy1, dy2 = c["dy"], np.random.default_rng(12).standard_normal(c["dy"].shape)
    c["dy"] = dy1
    g1 = _grads(c, **kw)
    c["dy"] = dy2
    g2 = _grads(c, **kw)
    c["dy"] = dy1 + dy2
    g12 = _grads(c, **kw)
    for k in g1:
        np.testing.assert_allclose(g12[k], g1[k] + g2[k], rtol=1e-9, atol=1e-11, err_msg=k)
