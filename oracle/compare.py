"""CPU float64 oracle for the train-vs-rollout selected-logprob comparison metrics.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP path.

Inputs: two fp32 per-token selected-logprob arrays over the same T tokens -- one from the
trainer ("train", the logprob the training side recomputes) and one from the rollout engine
("rollout", the logprob reported when the token was sampled) -- and an optional per-token
active mask (response tokens that enter the loss).  Every metric is over active tokens.

Sources (web pages; none prints a formula):
  * RL-Kernel h100-pcp.json evidence page, ``train_rollout_logprob`` block:
    ``element_count``, ``mismatch_count``, ``bitwise_mismatch_count``, ``max_abs_diff``,
    ``train_rollout_logprob_abs_diff``, ``mismatch_kl``, ``mismatch_k3_kl``; and its
    ``runtime_scalar_logprob`` rows (``active_token_count``, ``bitwise_mismatch_count``,
    ``max_abs_dlogp``, ``mean_abs_dlogp``, mismatch counts obtained with torch.ne / max);
  * RL-Kernel issue #342 "Strict R/R trace and operator ablation runbook", section 2
    (required result: mismatch count 0, max abs diff 0.0 over the 128 reporting rows) and
    the analyzer list (mismatch count and max absolute difference as diagnostics).

Readings (the pages name the metrics but do not define them):
  * d_i = train_i - rollout_i, evaluated in float64 (exact for fp32 operands);
  * mismatch_count: active tokens with train_i != rollout_i as IEEE values (torch.ne:
    a NaN on either side counts, -0 equals +0);
  * bitwise_mismatch_count: active tokens whose 32-bit patterns differ;
  * max_abs_diff = max |d_i|; mean_abs_diff = sum |d_i| / n (the "abs_diff" scalar);
    a NaN d_i makes both NaN (torch's max and sum propagate NaN);
  * the rollout engine sampled the tokens, so with the log-ratio r_i = d_i the two KL
    figures are Schulman's k1 and k3 estimators of KL(rollout || train):
        mismatch_kl    = sum(-r_i) / n
        mismatch_k3_kl = sum(exp(r_i) - 1 - r_i) / n     (written expm1(r) - r)
  * n = number of active tokens; with n = 0 every mean is 0 and the maximum is 0.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["logprob_compare", "METRIC_NAMES"]

METRIC_NAMES = ("active_tokens", "mismatch_count", "bitwise_mismatch_count", "max_abs_diff",
                "mean_abs_diff", "mismatch_kl", "mismatch_k3_kl")


def logprob_compare(train: np.ndarray, rollout: np.ndarray, mask: np.ndarray | None = None):
    """Metrics of the module docstring as a dict of Python ints / floats."""
    train = np.asarray(train, dtype=np.float32)
    rollout = np.asarray(rollout, dtype=np.float32)
    if train.shape != rollout.shape or train.ndim != 1:
        raise ValueError("train and rollout must be 1-D arrays of the same length")
    active = np.ones(train.shape, bool) if mask is None else np.asarray(mask).astype(bool)
    a = train[active]
    b = rollout[active]
    n = int(a.size)
    mismatch = int(np.count_nonzero(a != b))
    bitwise = int(np.count_nonzero(a.view(np.uint32) != b.view(np.uint32)))
    if n == 0:
        return dict(active_tokens=0, mismatch_count=0, bitwise_mismatch_count=0,
                    max_abs_diff=0.0, mean_abs_diff=0.0, mismatch_kl=0.0, mismatch_k3_kl=0.0)
    with np.errstate(invalid="ignore", over="ignore"):
        r = a.astype(np.float64) - b.astype(np.float64)   # exact for fp32 operands
        k3 = np.expm1(r) - r
    absd = np.abs(r)
    has_nan = bool(np.isnan(r).any())
    return dict(
        active_tokens=n,
        mismatch_count=mismatch,
        bitwise_mismatch_count=bitwise,
        max_abs_diff=math.nan if has_nan else float(absd.max()),
        mean_abs_diff=_fsum(absd) / n,
        mismatch_kl=_fsum(-r) / n,
        mismatch_k3_kl=_fsum(k3) / n,
    )


def _fsum(v: np.ndarray) -> float:
    """Correctly rounded sum (NaN if any term is NaN, inf/-inf sums as IEEE)."""
    if np.isnan(v).any():
        return math.nan
    if np.isinf(v).any():
        return float(np.sum(v))
    return math.fsum(v.tolist())
