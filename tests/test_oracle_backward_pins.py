"""Pins of the gradient oracle (oracle/backward.py) to facts outside itself: central
finite differences of the forward oracle, torch.autograd in float64, closed forms, the
zero row-sum invariant, masking and the fused chain rule against exact rationals.
Planted mistakes check that each pin bites."""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.backward as OB
from entropy_rlk_logprob_amd import synthetic as S


def pin_finite_differences():
    """d(g_lp lp + g_ent H)/dx_i by central differences of the forward oracle (h = 1e-5,
    truncation O(h^2) ~ 1e-10)."""
    rng = np.random.default_rng(21)
    T, V = 3, 7
    x = rng.normal(0, 1.5, (T, V))
    t = np.array([2, 0, 6])
    gl = np.array([1.0, -0.5, 0.25])
    ge = np.array([0.3, 1.2, -0.7])
    tau = 0.7
    g = OB.logits_grad(x, t, tau, gl, ge)

    def f(xx):
        lp, ent = oracle.logprob_entropy(xx, t, tau)
        return float(np.sum(gl * lp + ge * ent))

    h = 1e-5
    for r in range(T):
        for i in range(V):
            xp, xm = x.copy(), x.copy()
            xp[r, i] += h
            xm[r, i] -= h
            fd = (f(xp) - f(xm)) / (2 * h)
            assert abs(fd - g[r, i]) <= 1e-8, (r, i, fd, g[r, i])


def pin_torch_autograd():
    import torch
    rng = np.random.default_rng(22)
    T, V = 5, 33
    x = rng.normal(0, 3, (T, V))
    t = rng.integers(0, V, T)
    gl = rng.normal(size=T)
    ge = rng.normal(size=T)
    tau = float(np.float32(1.3))
    g = OB.logits_grad(x, t, 1.3, gl, ge)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ls = torch.log_softmax(xt / tau, dim=1)
    lp = ls.gather(1, torch.tensor(t).view(-1, 1)).view(-1)
    ent = -(ls.exp() * ls).sum(dim=1)
    (torch.tensor(gl) @ lp + torch.tensor(ge) @ ent).backward()
    assert np.abs(xt.grad.numpy() - g).max() <= 1e-13


def pin_closed_forms():
    """Uniform logits: logprob gradient (delta - 1/V)/tau, entropy gradient 0 (maximum)."""
    V = 16
    x = np.full((2, V), 0.75)
    g = OB.logits_grad(x, np.array([3, 9]), 2.0, np.array([1.0, 0.0]), np.array([0.0, 1.0]))
    want = np.full(V, -1.0 / V) / 2.0
    want[3] += 0.5
    assert np.abs(g[0] - want).max() <= 1e-15
    assert np.abs(g[1]).max() <= 1e-15
    # two tokens: H = binary entropy of p = sigmoid(a - b); dH/da = -p(1-p)(a - b)
    a, b = 0.9, -0.4
    p = 1.0 / (1.0 + math.exp(-(a - b)))
    g2 = OB.logits_grad(np.array([[a, b]]), np.array([0]), 1.0, np.array([0.0]), np.array([1.0]))
    assert abs(g2[0, 0] - (-p * (1 - p) * (a - b))) <= 1e-15
    assert abs(g2[0, 1] - (p * (1 - p) * (a - b))) <= 1e-15


def pin_row_sums_zero():
    """Shift invariance of logprob and entropy: every gradient row sums to 0."""
    rng = np.random.default_rng(23)
    x = rng.normal(0, 4, (6, 500))
    g = OB.logits_grad(x, rng.integers(0, 500, 6), 0.8, rng.normal(size=6), rng.normal(size=6))
    assert np.abs(g.sum(axis=1)).max() <= 1e-13


def pin_masking_and_nonfinite():
    rng = np.random.default_rng(24)
    x = rng.normal(0, 2, (7, 50))
    x[1, 7] = np.nan
    x[2, :] = -np.inf
    x[3, 10:] = -np.inf
    x[6, 10:] = -np.inf
    t = np.array([1, 1, 1, 5, -1, 60, 12])
    gl = np.array([0.0, 1.0, 1.0, 1.0, 0.0, 1.0, 2.0])
    ge = np.array([0.0, 0.0, 0.0, 1.0, 1.0, 0.0, 1.0])
    g = OB.logits_grad(x, t, 0.5, gl, ge)
    assert np.all(g[0] == 0.0)                        # masked row
    assert np.all(np.isnan(g[1])) and np.all(np.isnan(g[2]))
    small = OB.logits_grad(x[3:4, :10], np.array([5]), 0.5, np.array([1.0]), np.array([1.0]))
    assert np.abs(g[3, :10] - small[0]).max() <= 1e-15   # -inf masking = smaller vocabulary
    assert np.all(g[3, 10:] == 0.0)
    assert np.all(np.isfinite(g[4]))                  # out-of-range target, g_lp = 0
    assert np.all(np.isnan(g[5]))                     # out-of-range target, g_lp != 0
    # target at a -inf logit: only its delta term g_lp / tau there, zeros elsewhere beyond
    assert g[6, 12] == 2.0 / 0.5 and np.all(np.delete(g[6, 10:], 2) == 0.0)


def pin_fused_chain_rule_exact():
    """dh = grad W and dW = grad^T h, against exact rational sums of the same products."""
    rng = np.random.default_rng(25)
    T, d, V = 3, 4, 5
    hb = S.to_bf16_bits(rng.normal(size=(T, d)).astype(np.float32))
    wb = S.to_bf16_bits(rng.normal(0, 0.5, size=(V, d)).astype(np.float32))
    h, w = S.bf16_bits_to_f32(hb).astype(np.float64), S.bf16_bits_to_f32(wb).astype(np.float64)
    t = np.array([0, 4, 2])
    gl, ge = np.array([1.0, 0.5, -1.0]), np.array([0.2, 0.0, 1.0])
    dh, dw = OB.linear_grads(h, w, t, 1.0, gl, ge)
    gx = OB.logits_grad(h @ w.T, t, 1.0, gl, ge)
    for r in range(T):
        for k in range(d):
            ex = sum(Fraction(gx[r, v]) * Fraction(w[v, k]) for v in range(V))
            assert abs(dh[r, k] - float(ex)) <= 1e-15
    for v in range(V):
        for k in range(d):
            ex = sum(Fraction(gx[r, v]) * Fraction(h[r, k]) for r in range(T))
            assert abs(dw[v, k] - float(ex)) <= 1e-15


def pin_sampled_fused_gradients_equal_the_full_ones():
    """linear_grads_sampled (row blocks, selected dh and dW rows) equals the selected rows of
    linear_grads (pinned above by exact rational sums) -- with several blocks, a masked row, an
    out-of-range target and the last block short -- and its magnitudes are sum |grad| |W| and
    sum |grad| |h| of exact brute-force sums."""
    rng = np.random.default_rng(26)
    T, d, V = 37, 8, 50
    h = S.bf16_bits_to_f32(S.to_bf16_bits(rng.normal(size=(T, d)).astype(np.float32)))
    w = S.bf16_bits_to_f32(S.to_bf16_bits(rng.normal(0, 0.5, size=(V, d)).astype(np.float32)))
    h, w = h.astype(np.float64), w.astype(np.float64)
    t = rng.integers(0, V, T)
    t[4] = V + 3
    gl, ge = rng.normal(size=T), rng.normal(size=T)
    gl[4] = 0.0                     # out-of-range target without a logprob gradient
    gl[9] = ge[9] = 0.0             # masked row
    hr, wr = np.array([0, 4, 9, 16, 36]), np.array([0, 7, 49, int(t[3])])
    dh_f, dw_f = OB.linear_grads(h, w, t, 0.7, gl, ge)
    dh, dw, dh_mag, dw_mag = OB.linear_grads_sampled(h, w, t, 0.7, gl, ge, hr, wr, block=8)
    assert np.abs(dh - dh_f[hr]).max() <= 1e-14 and np.abs(dw - dw_f[wr]).max() <= 1e-14
    assert np.all(dh[2] == 0.0)
    gx = OB.logits_grad(h @ w.T, t, 0.7, gl, ge)
    for i, r in enumerate(hr):
        for k in range(d):
            ex = float(sum(abs(Fraction(gx[r, v])) * abs(Fraction(w[v, k])) for v in range(V)))
            assert abs(dh_mag[i, k] - ex) <= 1e-14 * max(1.0, ex)
    for i, v in enumerate(wr):
        for k in range(d):
            ex = float(sum(abs(Fraction(gx[r, v])) * abs(Fraction(h[r, k])) for r in range(T)))
            assert abs(dw_mag[i, k] - ex) <= 1e-14 * max(1.0, ex)


PINS = [pin_finite_differences, pin_torch_autograd, pin_closed_forms, pin_row_sums_zero,
        pin_masking_and_nonfinite, pin_fused_chain_rule_exact,
        pin_sampled_fused_gradients_equal_the_full_ones]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


_real = OB.logits_grad


def _entropy_sign(x, t, tau, gl, ge):
    return _real(x, t, tau, gl, None if ge is None else -np.asarray(ge, float))


def _no_tau(x, t, tau, gl, ge):
    return _real(x, t, tau, gl, ge) * float(np.float32(tau))


def _no_h_term(x, t, tau, gl, ge):
    """entropy term p (z - L) instead of p (z - L + H)"""
    g = _real(x, t, tau, gl, None)
    if ge is None:
        return g
    z = np.asarray(x, float) / float(np.float32(tau))
    L = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1, keepdims=True)) + z.max(1, keepdims=True)
    p = np.exp(z - L)
    return g - np.asarray(ge, float)[:, None] * p * (z - L) / float(np.float32(tau))


MUTANTS = {
    "entropy_sign": dict(logits_grad=_entropy_sign),
    "missing_1_over_tau": dict(logits_grad=_no_tau),
    "missing_H_term": dict(logits_grad=_no_h_term),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    for attr, val in MUTANTS[name].items():
        monkeypatch.setattr(OB, attr, val)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"


def test_planted_fused_operand_mistake(monkeypatch):
    """dW rows permuted (a transposed/misindexed operand) is caught by the exact pin."""
    real = OB.linear_grads

    def bad(h, w, t, tau, gl, ge):
        dh, dw = real(h, w, t, tau, gl, ge)
        return dh, dw[::-1].copy()
    monkeypatch.setattr(OB, "linear_grads", bad)
    with pytest.raises(AssertionError):
        pin_fused_chain_rule_exact()
