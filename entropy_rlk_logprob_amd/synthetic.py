"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle's tests.

This module draws random numbers and lays them out; it holds none of the method's
arithmetic (no log-softmax, no log-sum-exp, no entropy, no projection).  Every array
is a pure function of the seed, so the oracle and the HIP path see identical bytes.

Workloads (shapes and distributions follow the RL log-probability benchmarks: the
Qwen3-Next prior-art logprob comparison at 1024 tokens, and Qwen3-8B BF16 post-training
with 128-row responses packed 2048 tokens per GPU and rollout temperature 0.7):

  cfg 1  logits, T=64,    V=1024,   X ~ N(0, 2^2) fp32, targets uniform
  cfg 2  logits, T=1024,  V=151936, X ~ N(0, 3^2) fp32, 10 rows (1%) get +25 added at
         one uniformly chosen column, targets sampled from softmax(X)
  cfg 3  fused,  T=1024,  d=2048, V=151936, H ~ N(0,1), W ~ N(0, 0.02^2), bf16, tau=1,
         targets uniform
  cfg 4  fused,  T=2048 = 16 sequences x 128 rows, d=4096, V=151936, tau=1, targets uniform
  cfg 5  fused,  T=16384 in sequences of length uniform in {128..4096}, d=4096,
         V=151936, tau=0.7 (targets drawn from the tempered softmax by the oracle, stored
         with the parity goldens by tests/golden/make_fused_goldens.py)

Seeding: ``numpy.random.SeedSequence(1000 + cfg).spawn(5)`` gives independent streams
for [logits or H, W, spikes, targets, permutations].
"""
from __future__ import annotations

import dataclasses

import numpy as np

V_QWEN3 = 151936

STREAM_X, STREAM_W, STREAM_SPIKE, STREAM_TARGET, STREAM_PERM = range(5)


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    path: str            # "logits" or "fused"
    n_tokens: int
    vocab: int
    hidden: int = 0
    sigma: float = 1.0   # std of logits (logits path) or of H (fused path)
    w_sigma: float = 0.0
    temperature: float = 1.0
    name: str = ""


WORKLOADS = {
    1: Workload(1, "logits", 64, 1024, sigma=2.0, name="logits-T64-V1024"),
    2: Workload(2, "logits", 1024, V_QWEN3, sigma=3.0, name="logits-T1024-V151936-qwen3"),
    3: Workload(3, "fused", 1024, V_QWEN3, hidden=2048, sigma=1.0, w_sigma=0.02,
                name="linear-T1024-d2048-V151936-qwen3next"),
    4: Workload(4, "fused", 2048, V_QWEN3, hidden=4096, sigma=1.0, w_sigma=0.02,
                name="linear-T2048-d4096-V151936-qwen3-8b-16x128"),
    5: Workload(5, "fused", 16384, V_QWEN3, hidden=4096, sigma=1.0, w_sigma=0.02,
                temperature=0.7, name="linear-T16384-d4096-V151936-ragged-tau0.7"),
}


def streams(seed: int) -> list[np.random.Generator]:
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(5)]


def cfg_seed(cfg: int) -> int:
    return 1000 + cfg


def normal_f32(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) samples, drawn and scaled in float32."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); return the raw uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns (a bf16 value is a truncated fp32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def uniform_targets(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    return rng.integers(0, vocab, size=n, dtype=np.int64)


def gumbel_max_targets(rng: np.random.Generator, x: np.ndarray, temperature: float = 1.0,
                       block: int = 8) -> np.ndarray:
    """Draw one id per row with probability proportional to exp(x/tau).

    Gumbel-max: argmax_i(x_i/tau + G_i) with G_i = -log(-log U_i) is an exact sample
    from the tempered softmax, without forming the softmax itself.
    """
    n, v = x.shape
    out = np.empty(n, dtype=np.int64)
    inv_tau = 1.0 / float(np.float32(temperature))
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        u = rng.random(size=(r1 - r0, v))
        g = -np.log(-np.log(u))
        out[r0:r1] = np.argmax(x[r0:r1].astype(np.float64) * inv_tau + g, axis=1)
    return out


def spike_rows(rng: np.random.Generator, x: np.ndarray, frac: float = 0.01,
               amount: float = 25.0) -> np.ndarray:
    """Add `amount` to one uniformly chosen column in round(frac*T) distinct rows (in place).

    Returns the spiked row indices."""
    n, v = x.shape
    k = int(round(frac * n))
    rows = np.sort(rng.choice(n, size=k, replace=False))
    cols = rng.integers(0, v, size=k)
    x[rows, cols] += np.float32(amount)
    return rows


def ragged_lengths(rng: np.random.Generator, total: int, lo: int = 128,
                   hi: int = 4096) -> np.ndarray:
    """Lengths uniform in {lo..hi} drawn until their sum reaches `total`; last one cut."""
    lens = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return np.asarray(lens, dtype=np.int64)


# ---------------------------------------------------------------- workload builders

@dataclasses.dataclass
class LogitsCase:
    x: np.ndarray            # [T, V] float32
    targets: np.ndarray      # [T] int64
    temperature: float
    spiked_rows: np.ndarray | None = None


@dataclasses.dataclass
class FusedCase:
    h_bits: np.ndarray       # [T, d] uint16 (bf16)
    w_bits: np.ndarray       # [V, d] uint16 (bf16)
    targets: np.ndarray | None   # [T] int64 (None: the caller draws them)
    temperature: float
    seq_lens: np.ndarray     # packed sequence lengths, sum = T


def random_logits_case(n_tokens: int, vocab: int, sigma: float, seed: int,
                       temperature: float = 1.0) -> LogitsCase:
    """Generic seeded logits case: X ~ N(0, sigma^2) fp32, uniform targets."""
    st = streams(seed)
    x = normal_f32(st[STREAM_X], (n_tokens, vocab), sigma)
    t = uniform_targets(st[STREAM_TARGET], n_tokens, vocab)
    return LogitsCase(x, t, temperature)


def random_fused_case(n_tokens: int, hidden: int, vocab: int, seed: int,
                      h_sigma: float = 1.0, w_sigma: float = 0.02,
                      temperature: float = 1.0) -> FusedCase:
    """Generic seeded fused case: bf16 H ~ N(0, h_sigma^2), W ~ N(0, w_sigma^2)."""
    st = streams(seed)
    h = to_bf16_bits(normal_f32(st[STREAM_X], (n_tokens, hidden), h_sigma))
    w = to_bf16_bits(normal_f32(st[STREAM_W], (vocab, hidden), w_sigma))
    t = uniform_targets(st[STREAM_TARGET], n_tokens, vocab)
    return FusedCase(h, w, t, temperature, np.asarray([n_tokens], dtype=np.int64))


def logits_workload(cfg: int) -> LogitsCase:
    wl = WORKLOADS[cfg]
    assert wl.path == "logits"
    st = streams(cfg_seed(cfg))
    x = normal_f32(st[STREAM_X], (wl.n_tokens, wl.vocab), wl.sigma)
    if cfg == 2:
        rows = spike_rows(st[STREAM_SPIKE], x)
        t = gumbel_max_targets(st[STREAM_TARGET], x, wl.temperature)
        return LogitsCase(x, t, wl.temperature, rows)
    t = uniform_targets(st[STREAM_TARGET], wl.n_tokens, wl.vocab)
    return LogitsCase(x, t, wl.temperature)


def fused_workload(cfg: int) -> FusedCase:
    wl = WORKLOADS[cfg]
    assert wl.path == "fused"
    st = streams(cfg_seed(cfg))
    h = to_bf16_bits(normal_f32(st[STREAM_X], (wl.n_tokens, wl.hidden), wl.sigma))
    w = to_bf16_bits(normal_f32(st[STREAM_W], (wl.vocab, wl.hidden), wl.w_sigma))
    if cfg == 4:
        lens = np.full(16, 128, dtype=np.int64)
    elif cfg == 5:
        lens = ragged_lengths(st[STREAM_SPIKE], wl.n_tokens)
    else:
        lens = np.asarray([wl.n_tokens], dtype=np.int64)
    t = None if cfg == 5 else uniform_targets(st[STREAM_TARGET], wl.n_tokens, wl.vocab)
    return FusedCase(h, w, t, wl.temperature, lens)


def target_uniforms(cfg: int, n: int) -> np.ndarray:
    """Seeded uniforms in [0,1) for drawing targets by inverse CDF (cfg 5)."""
    return streams(cfg_seed(cfg))[STREAM_TARGET].random(n)


def upstream_grads(cfg: int, n: int, masked_every: int = 7):
    """Seeded per-row upstream gradients (g_logprob, g_entropy) ~ N(0, 1) fp32 for a
    backward call on workload `cfg`; every `masked_every`-th row has both at 0 (a padding
    row of a training batch)."""
    rng = np.random.default_rng(np.random.SeedSequence(cfg_seed(cfg)).spawn(6)[5])
    gl = rng.standard_normal(n, dtype=np.float32)
    ge = rng.standard_normal(n, dtype=np.float32)
    gl[::masked_every] = 0.0
    ge[::masked_every] = 0.0
    return gl, ge


def permutations(cfg: int, n: int, k: int = 3) -> list[np.ndarray]:
    rng = streams(cfg_seed(cfg))[STREAM_PERM]
    return [rng.permutation(n) for _ in range(k)]


def grid_logits(n_tokens: int, vocab: int, seed: int, lo: float = -32.0,
                hi: float = 32.0, step: float = 2.0 ** -8) -> np.ndarray:
    """Logits on the grid step*Z within [lo, hi]: sums and differences with such values
    (and with a shift of 64) are exact in fp32, so shifted inputs give identical bits."""
    rng = streams(seed)[STREAM_X]
    k = rng.integers(int(lo / step), int(hi / step) + 1, size=(n_tokens, vocab))
    return (k.astype(np.float64) * step).astype(np.float32)
