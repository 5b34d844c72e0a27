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


def _backward_golden(cfg):
    import json
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "fused_goldens.json")) as f:
        meta = json.load(f)["backward"][S.WORKLOADS[cfg].name]
    with np.load(os.path.join(here, meta["file"]), allow_pickle=False) as z:
        return meta, {k: z[k] for k in z.files}


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_backward_goldens_are_complete(cfg):
    """Every fused workload has its sampled backward rows: 48 dH rows and 48 dW rows of d
    values, finite, with rounding magnitudes that dominate them, under the upstream
    gradients the generator names (their sha256 must match)."""
    wl = S.WORKLOADS[cfg]
    meta, g = _backward_golden(cfg)
    T, d, V = wl.n_tokens, wl.hidden, wl.vocab
    assert meta["n_tokens"] == T
    gl, ge = S.upstream_grads(cfg, T)
    assert sha256(gl) == meta["sha256_g_logprob"] and sha256(ge) == meta["sha256_g_entropy"]
    assert g["h_rows"].shape == (48,) and g["w_rows"].shape == (48,)
    assert np.all((g["h_rows"] >= 0) & (g["h_rows"] < T))
    assert np.all((g["w_rows"] >= 0) & (g["w_rows"] < V))
    for k in ("dh", "dh_mag", "dw", "dw_mag"):
        assert g[k].shape == (48, d) and np.all(np.isfinite(g[k])), k
    assert np.all(np.abs(g["dh"]) <= g["dh_mag"] * (1 + 1e-12))
    assert np.all(np.abs(g["dw"]) <= g["dw_mag"] * (1 + 1e-12))


def test_backward_golden_dh_rows_match_a_fresh_oracle_evaluation():
    """Two stored dH rows of the T=1024, d=2048 workload against the oracle's chain rule on
    those rows alone: grad = oracle.logits_grad of the row's logits, dh = grad . W."""
    wl = S.WORKLOADS[3]
    _, g = _backward_golden(3)
    fwd = load_fused_golden(wl.name)
    case = S.fused_workload(3)
    gl, ge = S.upstream_grads(3, wl.n_tokens)
    sel = np.flatnonzero(gl[g["h_rows"]] != 0)[:2]  # two rows that are not masked
    rows = g["h_rows"][sel]
    assert len(rows) == 2
    h = S.bf16_bits_to_f32(case.h_bits[rows]).astype(np.float64)
    w = S.bf16_bits_to_f32(case.w_bits).astype(np.float64)
    grad = oracle.logits_grad(h @ w.T, fwd["targets"][rows], wl.temperature, gl[rows], ge[rows])
    dh = grad @ w
    assert np.max(np.abs(dh - g["dh"][sel])) <= 1e-12 * max(1.0, np.abs(g["dh"][sel]).max())
