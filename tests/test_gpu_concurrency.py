"""Determinism under contention: the logits path, the fused path and the fused backward
repeated while another stream keeps the GPU busy with unrelated matrix products, so that
workgroups land on other CUs, in another order and next to foreign work.  Every repeat must
give the bits of the call made on an idle GPU (one distinct result per output)."""
from __future__ import annotations

import math

import numpy as np
import pytest

from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import announce, bits_dev, dev

pytestmark = pytest.mark.gpu

REPEATS = 10


def _noise(stream, a, b, n=6):
    """n fp32 products of 4096 x 4096 matrices queued on `stream` (default priority)."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(n):
            a = torch.mm(a, b)
            a = a / (a.abs().amax() + 1.0)
    return a


def _distinct(outputs):
    return len({o.cpu().numpy().tobytes() for o in outputs})


def test_repeats_under_concurrent_load(lib):
    import torch
    rng = np.random.default_rng(777)
    T, V = 512, 32771
    x = dev((rng.standard_normal((T, V)) * 3.0).astype(np.float32))
    t = dev(rng.integers(0, V, T).astype(np.int64))
    case = S.random_fused_case(300, 256, 20000, seed=778, h_sigma=1.0, w_sigma=3.0 / math.sqrt(256))
    h, w, tf = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gl = dev(rng.standard_normal(300).astype(np.float32))
    ge = dev(rng.standard_normal(300).astype(np.float32))

    def run():
        lp, ent = lib.logprob_from_logits(x, t, 0.7, 4)
        flp, fent = lib.linear_logprob(h, w, tf, 0.7, 2)
        dh, dw = lib.linear_logprob_backward(h, w, tf, 0.7, 1, gl, ge)
        return [lp, ent, flp, fent, dh, dw]

    announce("concurrency: idle reference")
    ref = run()
    torch.cuda.synchronize()
    noise_stream = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn(4096, 4096, device="cuda", generator=g)
    b = torch.randn(4096, 4096, device="cuda", generator=g) / 64.0
    results = []
    for i in range(REPEATS):
        announce(f"concurrency: repeat {i} with a busy second stream")
        torch.cuda.synchronize()
        a = _noise(noise_stream, a, b)
        results.append(run())
        torch.cuda.synchronize()
    for k in range(len(ref)):
        assert _distinct([ref[k]] + [r[k] for r in results]) == 1, k


def test_calls_on_a_side_stream_give_the_default_stream_bits(lib):
    """Every binding call given stream= allocates its outputs and workspace on that stream and
    launches there; the bits equal those of the same call on the current stream.  The side
    stream's work is queued behind a long matrix product, so a wrong stream order (workspace
    reused on the current stream while the kernels still run) would show as changed bits."""
    import torch
    rng = np.random.default_rng(779)
    T, V = 300, 20011
    x = dev((rng.standard_normal((T, V)) * 3.0).astype(np.float32))
    t = dev(rng.integers(0, V, T).astype(np.int64))
    case = S.random_fused_case(T, 128, 5000, seed=780, h_sigma=1.0, w_sigma=3.0 / math.sqrt(128))
    h, w, tf = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gl = dev(rng.standard_normal(T).astype(np.float32))

    def run(stream):
        lp, ent = lib.logprob_from_logits(x, t, 0.7, 4, stream=stream)
        ent2 = lib.entropy(x, 0.7, 2, stream=stream)
        flp, fent = lib.linear_logprob(h, w, tf, 1.0, 4, stream=stream)
        g = lib.logprob_backward_from_logits(x, t, 0.7, 2, gl, None, stream=stream)
        dh, dw = lib.linear_logprob_backward(h, w, tf, 1.0, 2, gl, None, stream=stream)
        cmp = lib.logprob_compare(lp, flp[:T], stream=stream)
        return [lp, ent, ent2, flp, fent, g, dh, dw], cmp

    announce("side stream: reference on the current stream")
    ref, ref_cmp = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.Generator(device="cuda").manual_seed(6)
    a = torch.randn(4096, 4096, device="cuda", generator=g)
    b = torch.randn(4096, 4096, device="cuda", generator=g) / 64.0
    for i in range(3):
        announce(f"side stream: repeat {i}")
        _noise(side, a, b, n=4)
        out, cmp = run(side)
        side.synchronize()
        assert cmp == ref_cmp
        for k in range(len(ref)):
            assert _distinct([ref[k], out[k]]) == 1, (i, k)
