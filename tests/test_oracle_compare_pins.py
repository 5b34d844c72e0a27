"""Pins of the comparison-metric oracle (oracle/compare.py) to facts outside itself:
exact closed forms, the statistical meaning of the two KL estimators (sign convention),
IEEE value-vs-bit semantics, masking against the unmasked subset, a library evaluation,
and the small-ratio series.  Planted mistakes check that each pin bites."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.compare as OC


def f32(v):
    return np.asarray(v, dtype=np.float32)


def pin_identical():
    x = f32(np.random.default_rng(1).normal(-3, 2, 1000))
    m = OC.logprob_compare(x, x.copy())
    assert m == dict(active_tokens=1000, mismatch_count=0, bitwise_mismatch_count=0,
                     max_abs_diff=0.0, mean_abs_diff=0.0, mismatch_kl=0.0, mismatch_k3_kl=0.0)


def pin_symmetric_pair():
    """r = +a and -a: k1 = 0 exactly, k3 = (e^a + e^-a - 2)/2 = cosh(a) - 1."""
    a = float(np.float32(math.log(2.0)))
    m = OC.logprob_compare(f32([a, 0.0]), f32([0.0, a]))
    assert m["mismatch_kl"] == 0.0
    assert abs(m["mismatch_k3_kl"] - (math.cosh(a) - 1.0)) <= 4.5e-16   # 2 ulp at 1.25
    assert m["max_abs_diff"] == a and m["mean_abs_diff"] == a
    assert m["mismatch_count"] == 2 and m["bitwise_mismatch_count"] == 2


def pin_kl_estimators():
    """Tokens sampled from the rollout distribution q: k1 and k3 are unbiased estimators
    of KL(q || p) for the train distribution p.  (A swapped convention would estimate
    -KL or chi2 - KL; both are far outside the 6-sigma band here.)"""
    q = np.array([0.5, 0.2, 0.15, 0.1, 0.05])
    p = np.array([0.1, 0.3, 0.2, 0.25, 0.15])
    kl = float(np.sum(q * np.log(q / p)))
    rng = np.random.default_rng(11)
    n = 400_000
    tok = rng.choice(5, size=n, p=q)
    train, rollout = f32(np.log(p)[tok]), f32(np.log(q)[tok])
    m = OC.logprob_compare(train, rollout)
    r = np.log(p / q)[tok]
    se1 = float(np.std(-r)) / math.sqrt(n)
    se3 = float(np.std(np.expm1(r) - r)) / math.sqrt(n)
    assert abs(m["mismatch_kl"] - kl) <= 6 * se1, (m["mismatch_kl"], kl)
    assert abs(m["mismatch_k3_kl"] - kl) <= 6 * se3, (m["mismatch_k3_kl"], kl)
    assert m["mismatch_k3_kl"] >= 0.0


def pin_ieee_semantics():
    nan = np.float32("nan")
    t = f32([0.0, -0.0, nan, -1.5, -np.inf, -2.0])
    r = f32([-0.0, 0.0, nan, -1.5, -np.inf, -2.0])
    m = OC.logprob_compare(t, r, np.array([1, 1, 0, 1, 0, 1], np.uint8))
    assert m["active_tokens"] == 4 and m["mismatch_count"] == 0
    assert m["bitwise_mismatch_count"] == 2 and m["max_abs_diff"] == 0.0
    m = OC.logprob_compare(t, r)                      # NaN and -inf - -inf now active
    assert m["mismatch_count"] == 1 and m["bitwise_mismatch_count"] == 2
    assert math.isnan(m["max_abs_diff"]) and math.isnan(m["mismatch_k3_kl"])
    m = OC.logprob_compare(f32([]), f32([]))
    assert m["active_tokens"] == 0 and m["max_abs_diff"] == 0.0 and m["mismatch_kl"] == 0.0


def pin_mask_is_subset():
    rng = np.random.default_rng(5)
    t = f32(rng.normal(-4, 3, 3000))
    r = t + f32(rng.normal(0, 1e-3, 3000))
    r[rng.integers(0, 3000, 900)] = t[rng.integers(0, 3000, 900)]
    mask = rng.random(3000) < 0.37
    mask[np.argmax(np.abs(t.astype(np.float64) - r))] = False   # the global max is masked
    a = OC.logprob_compare(t, r, mask.astype(np.uint8))
    b = OC.logprob_compare(t[mask], r[mask])
    assert a == b and a["active_tokens"] == int(mask.sum())


def pin_library():
    """torch (float64, CPU) evaluation of the same definitions."""
    import torch
    rng = np.random.default_rng(6)
    t = f32(rng.normal(-5, 2, 5000))
    r = f32(t + rng.normal(0, 0.05, 5000).astype(np.float32))
    r[::7] = t[::7]
    m = OC.logprob_compare(t, r)
    tt, rr = torch.from_numpy(t), torch.from_numpy(r)
    d = tt.double() - rr.double()
    assert m["mismatch_count"] == int(torch.ne(tt, rr).sum())
    assert m["max_abs_diff"] == float(d.abs().max())
    assert abs(m["mean_abs_diff"] - float(d.abs().mean())) <= 1e-15
    assert abs(m["mismatch_kl"] - float((-d).mean())) <= 1e-15
    k3 = torch.special.expm1(d) - d
    assert abs(m["mismatch_k3_kl"] - float(k3.mean())) <= 1e-18


def pin_small_ratio_series():
    """r = 2^-20: expm1(r) - r = r^2/2 + r^3/6 + r^4/24 + ...  In float64 expm1(r) carries
    about ulp(r)/2 = 2^-73 of error, i.e. 2e-10 of r^2/2; the cancelling form exp(r) - 1 - r
    carries ulp(1)/2, i.e. 2.5e-4 of it."""
    r = 2.0 ** -20
    m = OC.logprob_compare(f32([r]), f32([0.0]))
    series = r * r / 2 + r ** 3 / 6 + r ** 4 / 24
    assert abs(m["mismatch_k3_kl"] - series) <= 1e-9 * series


PINS = [pin_identical, pin_symmetric_pair, pin_kl_estimators, pin_ieee_semantics,
        pin_mask_is_subset, pin_library, pin_small_ratio_series]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


class _NumpyWith:
    """numpy with some attributes replaced (a planted mistake inside the oracle)."""

    def __init__(self, **over):
        self.over = over

    def __getattr__(self, k):
        return self.over[k] if k in self.over else getattr(np, k)


_real = OC.logprob_compare


def _swapped(t, r, mask=None):
    return _real(r, t, mask)


def _mask_ignored(t, r, mask=None):
    return _real(t, r, None)


def _divide_by_all(t, r, mask=None):
    out = _real(t, r, mask)
    n_all = len(np.asarray(t))
    for k in ("mean_abs_diff", "mismatch_kl", "mismatch_k3_kl"):
        out[k] = out[k] * out["active_tokens"] / max(n_all, 1)
    return out


MUTANTS = {
    "naive_k3": dict(np=_NumpyWith(expm1=lambda x: np.exp(x) - 1.0)),
    "bitwise_by_value": dict(np=_NumpyWith(uint32=np.float32)),
    "swapped_sides": dict(logprob_compare=_swapped),
    "mask_ignored": dict(logprob_compare=_mask_ignored),
    "mean_over_all_tokens": dict(logprob_compare=_divide_by_all),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    for attr, val in MUTANTS[name].items():
        monkeypatch.setattr(OC, attr, val)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
