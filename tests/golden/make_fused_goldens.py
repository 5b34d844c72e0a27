"""Write the float64 oracle's logprob and entropy for EVERY row of the three fused
workloads (T=1024 d=2048; T=2048 d=4096; T=16384 d=4096 tau=0.7, all at V=151936) into
tests/golden/fused_<name>.npz, plus a manifest (fused_goldens.json) with the sha256 of the
generated inputs, so that a test can check that the generator still yields the same bytes.

Each row also gets the Euclidean norms of the gradients of its logprob and of its entropy
with respect to its logits (the backward oracle, oracle.logits_grad): the first-order
sensitivity of each output to errors in the fp32 logits, which the parity tests use to
scale their error model of the fp32 accumulation.

Calls only the oracle (oracle/) and the seeded input generator (synthetic.py).  For the
T=16384 workload the targets are drawn here, for all rows, from the oracle's tempered
softmax by inverse CDF with the workload's seeded uniforms -- the targets the GPU tests and
the benchmark then use.  The other two workloads keep their uniform targets.

The reference that scores every candidate of the RL-Kernel Qwen3-Next logprob prior-art
report (pr549, report.json) is "shared_logits_fp64" over all 1024 tokens of the call; this
is that reference for the fused workloads: every row, logits as exact float64 dot products
of the bf16 values.

For every fused workload it also stores selected rows of the fused backward's gradients
(dH for 48 tokens, dW for 48 vocabulary rows, oracle.linear_grads_sampled) under seeded
upstream gradients, with the magnitudes that bound their rounding.

Usage:  python tests/golden/make_fused_goldens.py [--rows-per-block 512] [--only CFG]
                                                  [--backward-only]
About 10 minutes on 8 cores (the largest workload's float64 logits, 20 TFLOP, are formed
twice: for the forward values and for the backward rows).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from entropy_rlk_logprob_amd import synthetic as S  # noqa: E402

MANIFEST = os.path.join(HERE, "fused_goldens.json")
CFGS = (3, 4, 5)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def golden_path(cfg: int) -> str:
    return os.path.join(HERE, f"fused_{S.WORKLOADS[cfg].name}.npz")


def make(cfg: int, rows_per_block: int) -> dict:
    wl = S.WORKLOADS[cfg]
    t0 = time.time()
    case = S.fused_workload(cfg)
    T = case.h_bits.shape[0]
    tau = wl.temperature
    h = S.bf16_bits_to_f32(case.h_bits)
    w64 = S.bf16_bits_to_f32(case.w_bits).astype(np.float64)
    draw = case.targets is None
    targets = np.empty(T, np.int64) if draw else case.targets
    u = S.target_uniforms(cfg, T) if draw else None
    lp = np.empty(T, np.float64)
    ent = np.empty(T, np.float64)
    g_norm_lp = np.empty(T, np.float64)
    g_norm_ent = np.empty(T, np.float64)
    for r0 in range(0, T, rows_per_block):
        r1 = min(T, r0 + rows_per_block)
        x = oracle.linear_logits(h[r0:r1], w64)
        if draw:
            targets[r0:r1] = oracle.sample_targets(oracle.tempered_logits(x, tau), u[r0:r1])
        lp[r0:r1], ent[r0:r1] = oracle.logprob_entropy(x, targets[r0:r1], tau)
        ones = np.ones(r1 - r0)
        g_norm_lp[r0:r1] = np.linalg.norm(
            oracle.logits_grad(x, targets[r0:r1], tau, ones, None), axis=1)
        g_norm_ent[r0:r1] = np.linalg.norm(
            oracle.logits_grad(x, targets[r0:r1], tau, None, ones), axis=1)
        print(f"  {wl.name}: rows [{r0}, {r1}) of {T}  {time.time() - t0:.0f} s", flush=True)
    np.savez_compressed(golden_path(cfg), targets=targets, logprob=lp, entropy=ent,
                        grad_norm_logprob=g_norm_lp, grad_norm_entropy=g_norm_ent)
    return {
        "file": os.path.basename(golden_path(cfg)),
        "n_tokens": int(T), "hidden": int(wl.hidden), "vocab": int(wl.vocab),
        "temperature": float(tau),
        "targets": "inverse CDF on the oracle's tempered softmax, uniforms "
                   "synthetic.target_uniforms(cfg, T)" if draw else
                   "uniform (synthetic.fused_workload)",
        "sha256_hidden_bits": sha256(case.h_bits),
        "sha256_weight_bits": sha256(case.w_bits),
        "sha256_targets": sha256(targets),
        "seq_lens": [int(n) for n in case.seq_lens],
        "numpy": np.__version__,
        "seconds": round(time.time() - t0, 1),
    }


def sampled_rows(T: int, V: int, targets: np.ndarray, seed: int = 77):
    """The token rows (of dH) and vocabulary rows (of dW) the backward goldens store: the
    ends, rows around the backward's token-chunk boundaries (multiples of 2048) and the
    canonical vocabulary chunks' boundaries, a few targets, and seeded random rows."""
    rng = np.random.default_rng(seed)
    h = {0, 1, T - 1} | {c + o for c in range(2048, T, 2048) for o in (-1, 0)}
    h |= set(rng.choice(T, 48 - len(h), replace=False).tolist())
    vc = 4 * (((V + 7) // 8 + 3) // 4)
    w = {0, V - 1} | {c * vc + o for c in range(1, 8) for o in (-1, 0)}
    w |= set(int(t) for t in targets[:6])
    w |= set(rng.choice(V, 48 - len(w), replace=False).tolist())
    return np.array(sorted(h)[:48], np.int64), np.array(sorted(w)[:48], np.int64)


def make_backward(cfg: int) -> dict:
    """dH and dW rows of the fused backward on workload cfg with seeded upstream gradients
    (synthetic.upstream_grads), and the magnitudes that bound their rounding."""
    wl = S.WORKLOADS[cfg]
    t0 = time.time()
    case = S.fused_workload(cfg)
    gold = np.load(golden_path(cfg), allow_pickle=False)
    targets = gold["targets"]
    T = case.h_bits.shape[0]
    gl, ge = S.upstream_grads(cfg, T)
    h_rows, w_rows = sampled_rows(T, wl.vocab, targets)
    dh, dw, dh_mag, dw_mag = oracle.linear_grads_sampled(
        S.bf16_bits_to_f32(case.h_bits), S.bf16_bits_to_f32(case.w_bits), targets,
        wl.temperature, gl, ge, h_rows, w_rows)
    path = os.path.join(HERE, f"fused_backward_{wl.name}.npz")
    np.savez_compressed(path, h_rows=h_rows, w_rows=w_rows, dh=dh, dw=dw, dh_mag=dh_mag,
                        dw_mag=dw_mag)
    return {"file": os.path.basename(path), "n_tokens": int(T),
            "upstream": "synthetic.upstream_grads(cfg, T)",
            "sha256_g_logprob": sha256(gl), "sha256_g_entropy": sha256(ge),
            "seconds": round(time.time() - t0, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--rows-per-block", type=int, default=512)
    ap.add_argument("--only", type=int, choices=CFGS, default=None)
    ap.add_argument("--backward-only", action="store_true",
                    help="only the backward rows (needs the forward goldens)")
    args = ap.parse_args()
    manifest = {}
    if os.path.exists(MANIFEST):
        with open(MANIFEST) as f:
            manifest = json.load(f)
    manifest["generator"] = ("tests/golden/make_fused_goldens.py: oracle.linear_logits, "
                             "oracle.tempered_logits, oracle.sample_targets, "
                             "oracle.logprob_entropy, oracle.logits_grad on "
                             "synthetic.fused_workload(cfg)")
    manifest.setdefault("workloads", {})
    manifest.setdefault("backward", {})
    for cfg in CFGS:
        if args.backward_only or (args.only is not None and cfg != args.only):
            continue
        manifest["workloads"][S.WORKLOADS[cfg].name] = make(cfg, args.rows_per_block)
        with open(MANIFEST, "w") as f:
            json.dump(manifest, f, indent=2)
            f.write("\n")
    for cfg in CFGS:
        if args.only is not None and cfg != args.only:
            continue
        manifest["backward"][S.WORKLOADS[cfg].name] = make_backward(cfg)
        with open(MANIFEST, "w") as f:
            json.dump(manifest, f, indent=2)
            f.write("\n")


if __name__ == "__main__":
    main()
