"""CPU float64 oracle for selected-token log-probability and per-token entropy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP path (no kernels, helpers, constants or pre/post-processing);
both only consume the seeded arrays of ``entropy_rlk_logprob_amd.synthetic``.

What is computed (plain definition, in float64, no blocking beyond independent row
blocks, no reordering beyond what NumPy's reductions do):

  For each row r with logits x (fp32 values, or fp64 dot products of bf16 values on the
  fused path) and fp32 temperature tau:
      z_i      = x_i / tau
      L        = M + ln sum_i exp(z_i - M),   M = max_i z_i
      logprob  = z_t - L                       (t = target id of the row)
      entropy  = sum_{i : p_i > 0} p_i (L - z_i),   p_i = exp(z_i - L)   (nats)

Sources (web pages; the pages print no formula, so the plain reading is used):
  * RL-Kernel "qwen3_next_logprob_prior_art" logprob report (pr549, report.json):
    each candidate is scored against ``"reference": "shared_logits_fp64"``, i.e. the
    same shared logits evaluated in float64 -> steps 1-5 evaluated in float64.
  * RL-Kernel issue #342 "Strict R/R trace and operator ablation runbook", section 2:
    the quantity is the selected-token logprob of each response row -> one output per
    (row, target) pair, full-vocabulary softmax.
  * RL-Kernel h100-pcp.json evidence page, ``train/entropy_loss`` and the scope note
    (rollout temperature .7): per-token entropy of the same tempered distribution.

Readings where the pages are silent (each also listed in the design notes):
  natural log; temperature divides the logits for both outputs; 0*ln 0 = 0; a target
  outside [0, V) gives a NaN logprob (entropy still defined); -inf logits are tokens of
  probability zero; a NaN or +inf anywhere in a row, or a row that is all -inf, makes
  both outputs of that row NaN.

Pinned by tests/test_oracle_pins.py (closed forms, brute force with exact sums,
independent library routines, invariants).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "tempered_logits", "logprob_entropy", "entropy", "linear_logits",
    "linear_logprob_entropy", "sample_targets",
]


def tempered_logits(x: np.ndarray, temperature: float) -> np.ndarray:
    """z = x / tau in float64; tau is the fp32 value a caller passes (0.7 -> 0.69999998...)."""
    tau = float(np.float32(temperature))
    if not (tau > 0.0 and np.isfinite(tau)):
        raise ValueError("temperature must be finite and > 0")
    return np.asarray(x, dtype=np.float64) / tau


def _rows_lse_entropy(z: np.ndarray):
    """Row-wise L = logsumexp(z) and entropy for a float64 block z[R, V].

    Returns (L, H, bad) where bad marks rows whose outputs are NaN by reading c7
    (a NaN or +inf anywhere, or no finite entry at all)."""
    has_nan = np.isnan(z).any(axis=1)
    has_pinf = np.isposinf(z).any(axis=1)
    M = np.max(np.where(np.isnan(z), -np.inf, z), axis=1)
    bad = has_nan | has_pinf | ~np.isfinite(M)
    Ms = np.where(bad, 0.0, M)[:, None]
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        e = np.exp(z - Ms)                       # -inf -> 0
        ssum = e.sum(axis=1)
        L = Ms[:, 0] + np.log(ssum)
        p = np.exp(z - L[:, None])
        gap = L[:, None] - z                     # +inf where z = -inf
        term = np.where(p > 0.0, p * gap, 0.0)
        H = term.sum(axis=1)
    L = np.where(bad, np.nan, L)
    H = np.where(bad, np.nan, H)
    return L, H, bad


def _row_block(n_cols: int) -> int:
    """Rows per block so that one float64 temporary stays near 2M elements (small enough
    for the allocator to reuse; the result does not depend on it: rows are independent)."""
    return max(1, min(256, (1 << 21) // max(1, n_cols)))


def logprob_entropy(x: np.ndarray, targets: np.ndarray | None, temperature: float = 1.0,
                    block: int | None = None):
    """Selected-token logprob and entropy of softmax(x / tau), row by row, in float64.

    x: [T, V] (any real dtype); targets: [T] integer ids or None.
    Returns (logprob[T] or None, entropy[T]) as float64 arrays."""
    x = np.asarray(x)
    T, V = x.shape
    block = block or _row_block(V)
    lp = None if targets is None else np.empty(T, dtype=np.float64)
    H = np.empty(T, dtype=np.float64)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        z = tempered_logits(x[r0:r1], temperature)
        L, h, _ = _rows_lse_entropy(z)
        H[r0:r1] = h
        if targets is not None:
            t = np.asarray(targets[r0:r1], dtype=np.int64)
            ok = (t >= 0) & (t < V)
            zt = np.where(ok, z[np.arange(r1 - r0), np.where(ok, t, 0)], np.nan)
            lp[r0:r1] = zt - L
    return lp, H


def entropy(x: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """Per-row entropy only (the logprob call with no targets)."""
    return logprob_entropy(x, None, temperature)[1]


def linear_logits(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Fused-path logits x = H W^T from the bf16 VALUES, in float64.

    h: [R, d], w: [V, d] float32 arrays holding bf16 values exactly.  Every product of two
    bf16 values is exact in float64 (8-bit x 8-bit significands); the sums are a float64
    matrix product (relative error ~1e-16, far below every tolerance used)."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def linear_logprob_entropy(h: np.ndarray, w: np.ndarray, targets: np.ndarray | None,
                           temperature: float = 1.0, block: int | None = None):
    """Logprob and entropy of softmax((H W^T)/tau) per row; the LM-head projection of the
    strict linear-logp operator followed by the same definition as logprob_entropy."""
    h = np.asarray(h)
    T = h.shape[0]
    lp = None if targets is None else np.empty(T, dtype=np.float64)
    H = np.empty(T, dtype=np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    block = block or _row_block(w64.shape[0])
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        x = linear_logits(h[r0:r1], w64)
        a, b = logprob_entropy(x, None if targets is None else targets[r0:r1], temperature)
        H[r0:r1] = b
        if lp is not None:
            lp[r0:r1] = a
    return lp, H


def sample_targets(z: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Inverse-CDF draw of one id per row from softmax(z) (z already tempered, float64),
    with given uniforms u[R] in [0, 1)."""
    z = np.asarray(z, dtype=np.float64)
    M = z.max(axis=1, keepdims=True)
    p = np.exp(z - M)
    cdf = np.cumsum(p, axis=1)
    thr = np.asarray(u, dtype=np.float64) * cdf[:, -1]
    idx = np.array([np.searchsorted(cdf[r], thr[r], side="right") for r in range(z.shape[0])])
    return np.minimum(idx, z.shape[1] - 1).astype(np.int64)
