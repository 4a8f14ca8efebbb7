"""Pins for the oracle's backward pass (CPU only): every gradient equals a
central finite difference of the oracle's own (pinned) forward pass.

The loss is L = sum(dy * y) + sum(dlast * last_state) for random dy, dlast,
so dL/dx is exactly the vector-Jacobian product the backward computes.  The
forward reads float32 inputs, so each perturbed input is rounded to float32
first and the difference quotient divides by the rounded step: only the
O(eps^2) truncation error remains.

Sources: [EXPLAINED] "Mamba CUDA 实现解析" eqs. (5)-(7) (the recurrence being
differentiated); [SPEC] "ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Реализовать selective scan
(Mamba)" Stage 1 (softplus, D skip, silu gate) and its backward-pass stage.
"""
import numpy as np
import pytest

import oracle


def inputs(seed, batch=2, dim=3, dstate=4, seqlen=12, gate=True, bias=True):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(u=f(batch, dim, seqlen), delta=(0.5 * f(batch, dim, seqlen)).astype(np.float32),
                A=(-np.abs(f(dim, dstate)) - 0.2).astype(np.float32),
                B=f(batch, dstate, seqlen), C=f(batch, dstate, seqlen), D=f(dim),
                z=f(batch, dim, seqlen) if gate else None,
                delta_bias=(0.3 * f(dim)).astype(np.float32) if bias else None)


def loss(x, softplus, h0, dy, dlast):
    y, st = oracle.selective_scan(**x, delta_softplus=softplus, h0=h0, nthreads=1)
    b, d, L = x["u"].shape
    return float(np.sum(dy.reshape(b * d, L) * y) + np.sum(dlast.reshape(b * d, -1) * st))


def fd_grad(x, name, softplus, h0, dy, dlast, eps=5e-4):
    base = x[name]
    g = np.zeros(base.shape, np.float64)
    for idx in np.ndindex(base.shape):
        xp, xm = dict(x), dict(x)
        vp, vm = base.copy(), base.copy()
        vp[idx] = np.float32(base[idx] + eps * max(1.0, abs(float(base[idx]))))
        vm[idx] = np.float32(base[idx] - eps * max(1.0, abs(float(base[idx]))))
        xp[name], xm[name] = vp, vm
        g[idx] = (loss(xp, softplus, h0, dy, dlast) - loss(xm, softplus, h0, dy, dlast)) / (
            float(vp[idx]) - float(vm[idx]))
    return g


def fd_grad_h0(x, softplus, h0, dy, dlast, eps=1e-3):
    g = np.zeros(h0.shape)
    for idx in np.ndindex(h0.shape):
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += eps
        hm[idx] -= eps
        g[idx] = (loss(x, softplus, hp, dy, dlast) - loss(x, softplus, hm, dy, dlast)) / (2 * eps)
    return g


@pytest.mark.parametrize("softplus,gate,bias", [(True, True, True), (False, False, False),
                                                (True, False, True)])
def test_backward_equals_finite_differences(softplus, gate, bias):
    x = inputs(5, gate=gate, bias=bias)
    if not softplus:
        x["delta"] = np.abs(x["delta"]).astype(np.float32)
    rng = np.random.default_rng(9)
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    h0 = rng.standard_normal((b, d, n))
    dy = rng.standard_normal((b, d, L))
    dlast = rng.standard_normal((b, d, n))
    g = oracle.selective_scan_bwd(**x, dy=dy, delta_softplus=softplus, h0=h0, dlast=dlast,
                                  nthreads=1)
    names = [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
             ("D", "dD")]
    if gate:
        names.append(("z", "dz"))
    if bias:
        names.append(("delta_bias", "ddelta_bias"))
    for name, gname in names:
        want = fd_grad(x, name, softplus, h0, dy, dlast)
        np.testing.assert_allclose(g[gname], want, rtol=2e-5, atol=2e-6, err_msg=gname)
    np.testing.assert_allclose(g["dh0"], fd_grad_h0(x, softplus, h0, dy, dlast), rtol=2e-5,
                               atol=2e-6, err_msg="dh0")
    if not gate:
        assert g["dz"] is None


def test_backward_threads_do_not_change_results():
    x = inputs(6, batch=3, dim=5, seqlen=20)
    rng = np.random.default_rng(2)
    dy = rng.standard_normal((3, 5, 20))
    g1 = oracle.selective_scan_bwd(**x, dy=dy, nthreads=1)
    g4 = oracle.selective_scan_bwd(**x, dy=dy, nthreads=4)
    for k in g1:
        if g1[k] is not None:
            np.testing.assert_allclose(g1[k], g4[k], rtol=1e-13, atol=1e-13, err_msg=k)


def test_grouped_backward_equals_finite_differences():
    """B and C per group of channels ([batch, ngroups, dstate, seqlen], channel
    d in group d // (dim // ngroups)): every gradient, dB and dC per group
    included, equals a central difference of the oracle's grouped forward."""
    rng = np.random.default_rng(21)
    b, d, n, L, g = 2, 4, 3, 10, 2
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    x = dict(u=f(b, d, L), delta=(0.5 * f(b, d, L)).astype(np.float32),
             A=(-np.abs(f(d, n)) - 0.2).astype(np.float32), B=f(b, g, n, L), C=f(b, g, n, L),
             D=f(d), z=f(b, d, L), delta_bias=(0.3 * f(d)).astype(np.float32))
    h0 = rng.standard_normal((b, d, n))
    dy = rng.standard_normal((b, d, L))
    dlast = rng.standard_normal((b, d, n))
    got = oracle.selective_scan_bwd(**x, dy=dy, delta_softplus=True, h0=h0, dlast=dlast,
                                    nthreads=2)
    assert got["dB"].shape == (b, g, n, L)
    for name, gname in [("B", "dB"), ("C", "dC"), ("u", "du"), ("delta", "ddelta"),
                        ("A", "dA"), ("z", "dz")]:
        want = fd_grad(x, name, True, h0, dy, dlast)
        np.testing.assert_allclose(got[gname], want, rtol=2e-5, atol=2e-6, err_msg=gname)


def test_per_channel_groups_split_the_one_group_gradient():
    """With B, C repeated into every group, the per-group dB, dC add up over
    the groups to the one-group gradient (the groups' channels partition the
    sum over channels); the other gradients are unchanged."""
    x = inputs(8, batch=2, dim=6, dstate=3, seqlen=9)
    rng = np.random.default_rng(3)
    dy = rng.standard_normal((2, 6, 9))
    one = oracle.selective_scan_bwd(**x, dy=dy, nthreads=1)
    xg = dict(x, B=np.repeat(x["B"][:, None], 3, axis=1), C=np.repeat(x["C"][:, None], 3, axis=1))
    grp = oracle.selective_scan_bwd(**xg, dy=dy, nthreads=3)
    np.testing.assert_allclose(grp["dB"].sum(axis=1), one["dB"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(grp["dC"].sum(axis=1), one["dC"], rtol=1e-12, atol=1e-12)
    for k in ("du", "ddelta", "dA", "dD", "dz", "ddelta_bias"):
        np.testing.assert_allclose(grp[k], one[k], rtol=1e-12, atol=1e-12, err_msg=k)
