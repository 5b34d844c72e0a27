"""GPU parity of rlk_logprob_compare (train-vs-rollout comparison metrics) against the
fp64 oracle: counts and the maximum exactly, the means within a bound derived from fp64
summation; the same bits on repeats; and the strict path compared with itself across
vocab splits gives the zero-mismatch result the runbook requires of an R/R control."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import announce, dev

pytestmark = pytest.mark.gpu


def run(lib, train, rollout, mask=None):
    import torch
    t, r = dev(np.asarray(train, np.float32)), dev(np.asarray(rollout, np.float32))
    m = None if mask is None else dev(np.asarray(mask, np.uint8))
    out = lib.logprob_compare(t, r, m)
    torch.cuda.synchronize()
    return out


def assert_close(got: dict, ref: dict):
    """Integers and the max exactly; means within fp64 summation error.  The terms are
    exact (d) or within an ulp or two of |d| (expm1(d) - d); the fixed-tree sums of at most
    a few million fp64 terms stay far inside 1e-13 of the sum of magnitudes."""
    for k in ("active_tokens", "mismatch_count", "bitwise_mismatch_count"):
        assert got[k] == ref[k], (k, got[k], ref[k])
    for k in ("max_abs_diff", "mean_abs_diff", "mismatch_kl", "mismatch_k3_kl"):
        g, o = got[k], ref[k]
        if math.isnan(o) or math.isinf(o):
            assert (math.isnan(g) and math.isnan(o)) or g == o, (k, g, o)
            continue
        if k == "max_abs_diff":
            assert g == o, (k, g, o)
            continue
        scale = ref["mean_abs_diff"] if k != "mismatch_k3_kl" else abs(o)
        tol = 1e-13 * scale + (1e-15 * ref["mean_abs_diff"] if k == "mismatch_k3_kl" else 0.0)
        assert abs(g - o) <= tol, (k, g, o, tol)


def noisy_pair(T, seed, sigma=1e-3, equal_frac=0.3, mask_frac=0.8):
    rng = np.random.default_rng(seed)
    train = rng.normal(-4.0, 3.0, T).astype(np.float32)
    rollout = (train + rng.normal(0, sigma, T)).astype(np.float32)
    eq = rng.random(T) < equal_frac
    rollout[eq] = train[eq]
    mask = (rng.random(T) < mask_frac).astype(np.uint8)
    return train, rollout, mask


@pytest.mark.parametrize("T", [1, 100, 255, 4095, 4096, 4097, 65537, 1 << 20])
def test_vs_oracle(lib, T):
    announce(f"compare T={T}")
    train, rollout, mask = noisy_pair(T, seed=600 + T)
    assert_close(run(lib, train, rollout, mask), oracle.logprob_compare(train, rollout, mask))
    assert_close(run(lib, train, rollout), oracle.logprob_compare(train, rollout))


def test_large_ratios_and_repeats(lib):
    """Log-ratios up to +-20 (k3 dominated by exp), same bits on every call."""
    announce("compare large ratios, repeats")
    rng = np.random.default_rng(61)
    T = 300_001
    train = rng.normal(-6, 4, T).astype(np.float32)
    rollout = (train + rng.uniform(-20, 20, T)).astype(np.float32)
    ref = oracle.logprob_compare(train, rollout)
    got = run(lib, train, rollout)
    assert_close(got, ref)
    for _ in range(3):
        assert run(lib, train, rollout) == got


def test_ieee_cases_and_empty(lib):
    announce("compare IEEE cases")
    nan = np.float32("nan")
    t = np.array([0.0, -0.0, nan, -1.5, -np.inf, -2.0, -3.0, -np.inf], np.float32)
    r = np.array([-0.0, 0.0, nan, -1.5, -np.inf, -2.0, -np.inf, -1.0], np.float32)
    for mask in (None, np.array([1, 1, 0, 1, 0, 1, 0, 0], np.uint8),
                 np.array([1, 1, 0, 1, 0, 1, 1, 0], np.uint8),
                 np.array([1, 1, 0, 1, 0, 1, 0, 1], np.uint8)):
        assert_close(run(lib, t, r, mask), oracle.logprob_compare(t, r, mask))
    z = run(lib, np.zeros(0, np.float32), np.zeros(0, np.float32))
    assert z == dict(active_tokens=0, mismatch_count=0, bitwise_mismatch_count=0,
                     max_abs_diff=0.0, mean_abs_diff=0.0, mismatch_kl=0.0, mismatch_k3_kl=0.0)
    allmasked = run(lib, t[:4], r[:4], np.zeros(4, np.uint8))
    assert allmasked["active_tokens"] == 0 and allmasked["mean_abs_diff"] == 0.0


def test_strict_path_against_itself_is_zero(lib):
    """Selected logprobs of the Qwen3-vocabulary workload computed unsplit ("train") and
    with 4 vocab shards in a permuted batch ("rollout"): zero mismatches, max diff 0."""
    import torch
    announce("compare strict path split 1 vs split 4 permuted")
    case = S.logits_workload(2)
    x, t = dev(case.x), dev(case.targets)
    lp1, _ = lib.logprob_from_logits(x, t, 1.0, 1)
    perm = torch.from_numpy(S.permutations(2, x.shape[0], 1)[0]).cuda()
    lp4p, _ = lib.logprob_from_logits(x[perm], t[perm], 1.0, 4)
    lp4 = torch.empty_like(lp4p)
    lp4[perm] = lp4p
    res = lib.logprob_compare(lp1, lp4)
    torch.cuda.synchronize()
    assert res["active_tokens"] == x.shape[0]
    assert res["mismatch_count"] == 0 and res["bitwise_mismatch_count"] == 0
    assert res["max_abs_diff"] == 0.0 and res["mismatch_kl"] == 0.0
    assert res["mismatch_k3_kl"] == 0.0
