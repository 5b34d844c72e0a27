"""CPU float64 oracle for the gradient of c1 * logprob + c2 * entropy with respect to the
logits (and, through the LM-head projection, with respect to the hidden states and weight).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
shares no code with the HIP path.

What is computed (plain calculus on the forward definition of oracle/logprob.py, float64):

  For a row with logits x, temperature tau (the fp32 value passed), target t and upstream
  gradients g_lp (of the row's logprob) and g_ent (of the row's entropy):
      z = x / tau,   L = logsumexp(z),   p = exp(z - L),   H = -sum p log p = L - sum p z
      d logprob / d x_i = (delta_it - p_i) / tau
      d H / d x_i       = -p_i (z_i - L + H) / tau          (0 where p_i = 0)
      grad_i = g_lp (delta_it - p_i) / tau  -  g_ent p_i (z_i - L + H) / tau
  Fused path, logits x = h W^T:   dh = grad W,   dW = sum over rows of grad^T h.

Sources (web pages; none prints a formula):
  * RL-Kernel h100-pcp.json evidence page: training consumes the logprob and entropy
    (train/loss, pg_loss, kl_loss, entropy_loss, grad_norm), and its comparison block finds
    the trained weights of every version and the per-step norms equal between two parallel
    configurations -- the gradient path must be deterministic and configuration-invariant.
  * RL-Kernel issue #342 runbook: linear_logp is one of the operator families the strict
    training side runs.

Readings where the pages are silent (also listed in the design notes):
  * the upstream gradients are per row (g_lp[T], g_ent[T]); a missing one is 0;
  * a row whose two upstream gradients are both 0 gets an all-zero gradient (masked rows,
    e.g. padding), whatever its logits and target;
  * otherwise a target outside [0, V) with g_lp != 0 makes the row's gradient NaN (its
    forward logprob is NaN); with g_lp == 0 the logprob term contributes nothing;
  * a row whose forward outputs are NaN (a NaN or +inf logit, or all logits -inf) gets a
    NaN gradient;
  * a -inf logit has p = 0, so both terms give it exactly 0 (the entropy term's
    p (z - L + H) is taken as its limit 0), except that a target at a -inf logit keeps its
    delta term g_lp / tau.

Pinned by tests/test_oracle_backward_pins.py (finite differences of the forward oracle,
torch.autograd in float64, closed forms, row-sum invariants, masking).
"""
from __future__ import annotations

import numpy as np

__all__ = ["logits_grad", "linear_grads", "linear_grads_sampled"]


def logits_grad(x: np.ndarray, targets: np.ndarray, temperature: float,
                g_lp: np.ndarray | None, g_ent: np.ndarray | None) -> np.ndarray:
    """grad of sum_r g_lp[r] logprob[r] + g_ent[r] entropy[r] w.r.t. x[T, V] (float64)."""
    tau = float(np.float32(temperature))
    if not (tau > 0.0 and np.isfinite(tau)):
        raise ValueError("temperature must be finite and > 0")
    x = np.asarray(x, dtype=np.float64)
    T, V = x.shape
    targets = np.asarray(targets, dtype=np.int64)
    gl = np.zeros(T) if g_lp is None else np.asarray(g_lp, dtype=np.float64)
    ge = np.zeros(T) if g_ent is None else np.asarray(g_ent, dtype=np.float64)
    out = np.zeros((T, V), dtype=np.float64)
    for r in range(T):
        if gl[r] == 0.0 and ge[r] == 0.0:
            continue                                  # masked row: all-zero gradient
        z = x[r] / tau
        if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
            out[r] = np.nan                           # forward outputs are NaN
            continue
        M = z[np.isfinite(z)].max()
        e = np.exp(z - M)                             # exp(-inf) = 0
        L = M + np.log(e.sum())
        p = np.exp(z - L)
        with np.errstate(invalid="ignore"):
            zl = np.where(p > 0.0, z - L, 0.0)        # log p where p > 0
        H = -float(np.sum(p * zl))
        g = -gl[r] * p - ge[r] * p * (zl + H)
        t = int(targets[r])
        if 0 <= t < V:
            g[t] += gl[r]
        elif gl[r] != 0.0:
            g[:] = np.nan
        out[r] = g / tau
    return out


def linear_grads(h: np.ndarray, w: np.ndarray, targets: np.ndarray, temperature: float,
                 g_lp: np.ndarray | None, g_ent: np.ndarray | None):
    """(dh [T, d], dW [V, d]) for logits x = h W^T (h, w given as float values)."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    gx = logits_grad(h @ w.T, targets, temperature, g_lp, g_ent)
    return gx @ w, gx.T @ h


def linear_grads_sampled(h: np.ndarray, w: np.ndarray, targets: np.ndarray, temperature: float,
                         g_lp: np.ndarray | None, g_ent: np.ndarray | None,
                         h_rows: np.ndarray, w_rows: np.ndarray, block: int = 512):
    """Selected rows of the fused gradients of linear_grads, for batches whose full dW or
    logits would not fit: dh[h_rows] [len(h_rows), d] and dW[w_rows] [len(w_rows), d],
    together with the magnitudes sum |grad| |W| (for the dh rows) and sum |grad| |h| (for
    the dW rows) that bound the rounding of these products.

    The same chain rule over row blocks: a block's logits x = h_b W^T (float64), its
    gradient g = logits_grad(x, ...); dh of a selected row is its g row times W, and dW of a
    selected vocabulary row v is the sum over the blocks of g[:, v]^T h_b."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = h.shape[0]
    h_rows = np.asarray(h_rows, dtype=np.int64)
    w_rows = np.asarray(w_rows, dtype=np.int64)
    gl = None if g_lp is None else np.asarray(g_lp)
    ge = None if g_ent is None else np.asarray(g_ent)
    dh = np.zeros((len(h_rows), h.shape[1]))
    dh_mag = np.zeros_like(dh)
    dw = np.zeros((len(w_rows), h.shape[1]))
    dw_mag = np.zeros_like(dw)
    w_abs = np.abs(w)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        g = logits_grad(h[r0:r1] @ w.T, np.asarray(targets)[r0:r1], temperature,
                        None if gl is None else gl[r0:r1], None if ge is None else ge[r0:r1])
        sel = np.flatnonzero((h_rows >= r0) & (h_rows < r1))
        if sel.size:
            gs = g[h_rows[sel] - r0]
            dh[sel] = gs @ w
            dh_mag[sel] = np.abs(gs) @ w_abs
        gv = g[:, w_rows]
        dw += gv.T @ h[r0:r1]
        dw_mag += np.abs(gv).T @ np.abs(h[r0:r1])
    return dh, dw, dh_mag, dw_mag
