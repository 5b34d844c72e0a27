"""The stored fp64 oracle values of the fused workloads (tests/golden/make_fused_goldens.py):
they are complete, consistent with a fresh oracle evaluation, and the T=16384 workload's
targets really are draws from the tempered softmax.  CPU only."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import load_fused_golden, sha256


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_goldens_cover_every_row(cfg):
    wl = S.WORKLOADS[cfg]
    g = load_fused_golden(wl.name)
    T = wl.n_tokens
    for k in ("targets", "logprob", "entropy", "grad_norm_logprob", "grad_norm_entropy"):
        assert g[k].shape == (T,), k
    assert g["targets"].dtype == np.int64
    assert np.all((g["targets"] >= 0) & (g["targets"] < wl.vocab))
    assert np.all(np.isfinite(g["logprob"])) and np.all(g["logprob"] < 0)
    assert np.all(g["entropy"] > 0) and np.all(g["entropy"] < math.log(wl.vocab))
    # the gradient of logprob w.r.t. the logits is (onehot - p) / tau: its norm lies in
    # [(1 - p_t) / tau, sqrt(2) / tau]; the entropy's gradient norm is non-negative
    beta = 1.0 / float(np.float32(wl.temperature))
    assert np.all(g["grad_norm_logprob"] <= math.sqrt(2) * beta + 1e-12)
    assert np.all(g["grad_norm_logprob"] >= beta * (1 - np.exp(g["logprob"])) - 1e-12)
    assert np.all(g["grad_norm_entropy"] >= 0)
    assert g["meta"]["n_tokens"] == T and g["meta"]["hidden"] == wl.hidden


def test_sampled_targets_follow_the_tempered_softmax():
    """For t drawn from p, E[log p_t] = -H (the entropy is the expected surprisal), so the
    mean of logprob + entropy over the 16384 rows is zero within its standard error; with
    uniform targets it would sit near -(ln V - H) < -1."""
    g = load_fused_golden(S.WORKLOADS[5].name)
    r = g["logprob"] + g["entropy"]
    z = r.mean() / (r.std(ddof=1) / math.sqrt(len(r)))
    assert abs(z) < 5.0, z
    assert np.median(g["logprob"]) > -math.log(S.V_QWEN3) + 1.0


def test_goldens_match_a_fresh_oracle_evaluation():
    """Regenerate the T=1024, d=2048 inputs (their sha256 must match the manifest), evaluate
    a few rows with the oracle directly, and compare with the stored values."""
    wl = S.WORKLOADS[3]
    g = load_fused_golden(wl.name)
    case = S.fused_workload(3)
    assert sha256(case.h_bits) == g["meta"]["sha256_hidden_bits"]
    assert sha256(case.w_bits) == g["meta"]["sha256_weight_bits"]
    assert np.array_equal(case.targets, g["targets"])
    rows = np.array([0, 1, 511, 1023])
    h = S.bf16_bits_to_f32(case.h_bits[rows])
    w = S.bf16_bits_to_f32(case.w_bits)
    lp, ent = oracle.linear_logprob_entropy(h, w, case.targets[rows], wl.temperature)
    assert np.max(np.abs(lp - g["logprob"][rows])) <= 1e-12
    assert np.max(np.abs(ent - g["entropy"][rows])) <= 1e-12
