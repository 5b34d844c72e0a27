"""GPU parity of the bf16-logits calls (rlk_logprob_from_logits_bf16, rlk_entropy_bf16).

Widening bf16 to fp32 is exact, and the bf16 calls reduce in the fp32 calls' canonical
order, so their outputs must be bitwise equal to the fp32 calls on the widened logits
(every shape, split, stride, alignment and non-finite case below), and within the logits
tolerance of the fp64 oracle evaluated on the widened values."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import TOL_LOGITS, announce, bitwise_equal, dev, max_abs, run_logits

pytestmark = pytest.mark.gpu


def bf16_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def both(lib, bits, t, tau=1.0, split=1):
    """(bf16 call on bits, fp32 call on the widened values)."""
    got = run_logits(lib, bf16_dev(bits), t, tau, split)
    ref = run_logits(lib, S.bf16_bits_to_f32(bits), t, tau, split)
    return got, ref


@pytest.mark.parametrize("T,V,tau", [
    (1, 1, 1.0), (3, 2, 1.0), (5, 3, 0.7), (7, 7, 1.0), (9, 1000, 1.0), (6, 1023, 1.0),
    (3, 4097, 2.0), (33, 20000, 0.7), (5, 257 * 8 + 3, 1.0), (17, 151936, 0.7),
])
def test_shapes_bitwise_vs_f32_and_oracle(lib, T, V, tau):
    announce(f"bf16 logits T={T} V={V} tau={tau}")
    case = S.random_logits_case(T, V, 3.0, seed=7100 + V)
    bits = S.to_bf16_bits(case.x)
    olp, oent = oracle.logprob_entropy(S.bf16_bits_to_f32(bits), case.targets, tau)
    first = None
    for split in (1, 2, 4, 8):
        (lp, ent), (flp, fent) = both(lib, bits, case.targets, tau, split)
        assert bitwise_equal(lp, flp) and bitwise_equal(ent, fent), split
        assert max_abs(lp, olp) <= TOL_LOGITS and max_abs(ent, oent) <= TOL_LOGITS, split
        if first is None:
            first = (lp, ent)
        else:
            assert bitwise_equal(lp, first[0]) and bitwise_equal(ent, first[1]), split


def test_strided_and_unaligned_rows_bitwise(lib):
    """Row strides not a multiple of 4 and bases not 8-byte aligned take element loads;
    a padded stride with an aligned base takes 8-byte loads: all give the dense bits."""
    T, V = 12, 5003
    case = S.random_logits_case(T, V, 2.0, seed=72)
    bits = S.to_bf16_bits(case.x)
    ref = run_logits(lib, bf16_dev(bits), case.targets)
    for off, pad in [(1, 13), (4, 9), (0, 5), (2, 3)]:
        announce(f"bf16 logits view offset={off} ld={V + pad}")
        big = np.full((T, V + pad), 0x7FC0, dtype=np.uint16)   # NaN outside the view
        big[:, off:off + V] = bits
        view = bf16_dev(big)[:, off:off + V]
        got = run_logits(lib, view, case.targets)
        assert bitwise_equal(got[0], ref[0]) and bitwise_equal(got[1], ref[1]), (off, pad)


@pytest.fixture(scope="module")
def cfg2_bf16():
    announce("generating logits workload T=1024 V=151936 (seed 1002) as bf16")
    case = S.logits_workload(2)
    bits = S.to_bf16_bits(case.x)
    return case, bits, bf16_dev(bits), dev(case.targets)


def test_qwen3_vocab_vs_oracle_and_f32(lib, cfg2_bf16):
    case, bits, xd, td = cfg2_bf16
    announce("bf16 logits T=1024 V=151936 vs oracle")
    lp, ent = run_logits(lib, xd, td)
    olp, oent = oracle.logprob_entropy(S.bf16_bits_to_f32(bits), case.targets)
    e1, e2 = max_abs(lp, olp), max_abs(ent, oent)
    print(f"max_abs_vs_fp64 logprob={e1:.3e} entropy={e2:.3e}")
    assert e1 <= TOL_LOGITS and e2 <= TOL_LOGITS
    flp, fent = run_logits(lib, S.bf16_bits_to_f32(bits), case.targets)
    assert bitwise_equal(lp, flp) and bitwise_equal(ent, fent)
    for split in (2, 4, 8):
        announce(f"bf16 logits T=1024 split={split} vs 1")
        got = run_logits(lib, xd, td, 1.0, split)
        assert bitwise_equal(got[0], lp) and bitwise_equal(got[1], ent), split


def test_qwen3_vocab_batch_order_and_entropy_call(lib, cfg2_bf16):
    import torch
    _, _, xd, td = cfg2_bf16
    ref_lp, ref_ent = run_logits(lib, xd, td)
    for perm in S.permutations(2, 1024, 1):
        announce("bf16 logits T=1024 row permutation")
        lp, ent = run_logits(lib, xd[perm], td[perm])
        assert bitwise_equal(lp, ref_lp[perm]) and bitwise_equal(ent, ref_ent[perm])
    for lo, hi in [(0, 1), (1000, 1024), (3, 515)]:
        announce(f"bf16 logits rows [{lo},{hi}) alone, split 4")
        lp, ent = run_logits(lib, xd[lo:hi], td[lo:hi], 1.0, 4)
        assert bitwise_equal(lp, ref_lp[lo:hi]) and bitwise_equal(ent, ref_ent[lo:hi])
    for split in (1, 8):
        announce(f"rlk_entropy_bf16 T=1024 split={split}")
        e = lib.entropy(xd, 1.0, split)
        torch.cuda.synchronize()
        assert bitwise_equal(e.cpu().numpy(), ref_ent)


def test_closed_forms_and_nonfinite(lib):
    announce("bf16 logits closed forms")
    for V in (1, 2, 1024, 151936):
        bits = S.to_bf16_bits(np.full((3, V), 1.5, dtype=np.float32))
        lp, ent = run_logits(lib, bf16_dev(bits), np.array([0, V - 1, V // 2]))
        assert np.all(np.abs(lp + math.log(V)) <= TOL_LOGITS), V
        assert np.all(np.abs(ent - math.log(V)) <= TOL_LOGITS), V
    rng = np.random.default_rng(4)
    T, V = 8, 3000
    x = rng.normal(0, 2, size=(T, V)).astype(np.float32)
    x[0, 5] = np.nan
    x[1, 2999] = np.inf
    x[2, :] = -np.inf
    x[3, 1000:] = -np.inf
    x[4, :2999] = -np.inf
    bits = S.to_bf16_bits(x)
    t = np.array([1, 1, 1, 1500, 2999, -1, V, 7])
    announce("bf16 logits non-finite rows")
    olp, oent = oracle.logprob_entropy(S.bf16_bits_to_f32(bits), t)
    for split in (1, 2, 8):
        (lp, ent), (flp, fent) = both(lib, bits, t, 1.0, split)
        assert bitwise_equal(lp, flp) and bitwise_equal(ent, fent), split
        assert np.isnan(lp[0]) and np.isnan(lp[1]) and np.isnan(lp[2])
        assert np.isneginf(lp[3]) and lp[4] == 0.0 and ent[4] == 0.0
        assert max_abs(ent[3:], oent[3:]) <= TOL_LOGITS
        assert abs(lp[7] - olp[7]) <= TOL_LOGITS


def test_empty_batch(lib):
    import torch
    announce("bf16 logits T=0")
    x = torch.empty((0, 100), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((0,), dtype=torch.int64, device="cuda")
    lp, ent = lib.logprob_from_logits(x, t)
    torch.cuda.synchronize()
    assert lp.numel() == 0 and ent.numel() == 0
