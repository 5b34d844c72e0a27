"""GPU parity of rlk_logprob_backward_from_logits against the fp64 gradient oracle, element
by element, and its strictness: bitwise invariance to vocab split, batch composition, row
order, in-place use and repeats; masking and non-finite rows; zero row sums at full size."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import announce, bitwise_equal, dev

pytestmark = pytest.mark.gpu


def run_grad(lib, x, t, tau=1.0, split=1, gl=None, ge=None, out=None):
    import torch
    xd = x if isinstance(x, torch.Tensor) else dev(np.asarray(x, np.float32))
    td = None if t is None else (t if isinstance(t, torch.Tensor) else dev(np.asarray(t, np.int64)))
    gld = None if gl is None else dev(np.asarray(gl, np.float32))
    ged = None if ge is None else dev(np.asarray(ge, np.float32))
    g = lib.logprob_backward_from_logits(xd, td, tau, split, gld, ged, out=out)
    torch.cuda.synchronize()
    return g.cpu().numpy()


def tolerance(x, t, tau, gl, ge):
    """Per-element bound from the fp32 arithmetic of the kernel: p = 2^q with
    q = c (x - m) - log2 s carries a relative error of about 2^-24 (3|a| + 2 log2 s + |q|)
    plus the exp's ulp, taken as 2e-6 (8 + 2|q| + log2 s); the delta term adds one rounding
    at 1.  Scaled by the row's weights |g_lp| and |g_ent| (1 + |ln p| + |H|) and by 1/tau."""
    tau = float(np.float32(tau))
    z = np.asarray(x, np.float64) / tau
    T, V = z.shape
    M = np.where(np.isfinite(z), z, -np.inf).max(axis=1, keepdims=True)
    L = M + np.log(np.exp(z - M).sum(axis=1, keepdims=True))
    p = np.exp(z - L)
    with np.errstate(invalid="ignore", divide="ignore"):
        lnp = np.where(p > 0, z - L, 0.0)
    H = -(p * lnp).sum(axis=1, keepdims=True)
    q = lnp / np.log(2.0)
    with np.errstate(invalid="ignore"):
        lg2s = np.nan_to_num((L - M) / np.log(2.0))     # log2 s, s = sum 2^(c (x - m))
    erel = 2e-6 * (8.0 + 2.0 * np.abs(q) + np.abs(lg2s))
    delta = np.zeros((T, V))
    tt = np.asarray(t)
    ok = (tt >= 0) & (tt < V)
    delta[np.arange(T)[ok], tt[ok]] = 1.0
    glv = np.abs(np.zeros(T) if gl is None else np.asarray(gl, np.float64))[:, None]
    gev = np.abs(np.zeros(T) if ge is None else np.asarray(ge, np.float64))[:, None]
    w = glv + gev * (1.0 + np.abs(lnp) + np.abs(H))
    return (w * (p * erel + 1.2e-7 * delta)) / tau + 1e-37


def check(gpu, ref, tol):
    assert np.array_equal(np.isnan(gpu), np.isnan(ref)), "NaN pattern differs"
    fin = ~np.isnan(ref)
    err = np.abs(gpu[fin].astype(np.float64) - ref[fin])
    assert np.all(err <= tol[fin]), (float(err.max()), float((err / tol[fin]).max()))


def weights(T, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(size=T).astype(np.float32), rng.normal(size=T).astype(np.float32)


@pytest.mark.parametrize("T,V,tau", [
    (1, 1, 1.0), (3, 2, 1.0), (5, 3, 0.7), (7, 1000, 1.0), (6, 1023, 0.7), (3, 4097, 2.0),
    (33, 20000, 0.7), (5, 257 * 8 + 3, 1.0), (9, 151936, 0.7),
])
def test_shapes_vs_oracle_and_split_bitwise(lib, T, V, tau):
    announce(f"grad T={T} V={V} tau={tau}")
    case = S.random_logits_case(T, V, 3.0, seed=8100 + V)
    gl, ge = weights(T, V)
    ref = oracle.logits_grad(case.x, case.targets, tau, gl, ge)
    tol = tolerance(case.x, case.targets, tau, gl, ge)
    first = None
    for split in (1, 2, 4, 8):
        g = run_grad(lib, case.x, case.targets, tau, split, gl, ge)
        check(g, ref, tol)
        if first is None:
            first = g
        else:
            assert bitwise_equal(g, first), split


def test_logprob_only_entropy_only_and_in_place(lib):
    import torch
    T, V = 12, 5003
    case = S.random_logits_case(T, V, 2.0, seed=81)
    gl, ge = weights(T, 82)
    announce("grad logprob-only / entropy-only / in place")
    g_lp = run_grad(lib, case.x, case.targets, 1.0, 1, gl, None)
    check(g_lp, oracle.logits_grad(case.x, case.targets, 1.0, gl, None),
          tolerance(case.x, case.targets, 1.0, gl, None))
    g_ent = run_grad(lib, case.x, None, 1.0, 1, None, ge)
    check(g_ent, oracle.logits_grad(case.x, np.zeros(T, np.int64), 1.0, None, ge),
          tolerance(case.x, np.full(T, -1), 1.0, None, ge))
    both = run_grad(lib, case.x, case.targets, 1.0, 1, gl, ge)
    xd = dev(case.x)
    inplace = run_grad(lib, xd, case.targets, 1.0, 1, gl, ge, out=xd)
    assert bitwise_equal(inplace, both)
    del torch


def test_strided_and_unaligned_bitwise(lib):
    import torch
    T, V = 10, 3001
    case = S.random_logits_case(T, V, 2.0, seed=83)
    gl, ge = weights(T, 84)
    ref = run_grad(lib, case.x, case.targets, 1.0, 1, gl, ge)
    big = np.full((T, V + 7), np.nan, np.float32)
    big[:, 1:V + 1] = case.x
    view = dev(big)[:, 1:V + 1]
    out_big = torch.full((T, V + 5), 7.0, device="cuda")
    out_view = out_big[:, 2:V + 2]
    announce("grad strided unaligned input and output")
    g = run_grad(lib, view, case.targets, 1.0, 1, gl, ge, out=out_view)
    assert bitwise_equal(g, ref)
    ob = out_big.cpu().numpy()
    assert np.all(ob[:, :2] == 7.0) and np.all(ob[:, V + 2:] == 7.0)   # nothing outside the view


def test_masking_and_nonfinite_rows(lib):
    rng = np.random.default_rng(85)
    T, V = 7, 2000
    x = rng.normal(0, 2, (T, V)).astype(np.float32)
    x[1, 7] = np.nan
    x[2, :] = -np.inf
    x[3, 1000:] = -np.inf
    x[6, 1000:] = -np.inf
    t = np.array([1, 1, 1, 5, -1, V, 1200])
    gl = np.array([0.0, 1.0, 1.0, 1.0, 0.0, 1.0, 2.0], np.float32)
    ge = np.array([0.0, 0.0, 0.0, 1.0, 1.0, 0.0, 1.0], np.float32)
    announce("grad masked and non-finite rows")
    ref = oracle.logits_grad(x, t, 0.5, gl, ge)
    for split in (1, 4):
        g = run_grad(lib, x, t, 0.5, split, gl, ge)
        check(g, ref, tolerance(x, t, 0.5, gl, ge))
        assert np.all(g[0] == 0.0)
        assert np.all(g[3, 1000:] == 0.0) and g[6, 1200] == np.float32(4.0)


@pytest.fixture(scope="module")
def cfg2():
    announce("generating logits workload T=1024 V=151936 (seed 1002)")
    case = S.logits_workload(2)
    gl, ge = weights(1024, 1002)
    return case, gl, ge, dev(case.x), dev(case.targets), dev(gl), dev(ge)


def test_qwen3_vocab_vs_oracle_sampled_rows(lib, cfg2):
    import torch
    case, gl, ge, xd, td, gld, ged = cfg2
    announce("grad T=1024 V=151936 vs oracle (sampled rows)")
    g = lib.logprob_backward_from_logits(xd, td, 1.0, 1, gld, ged)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 1024, 61), case.spiked_rows, [1023]]))
    gs = g[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = oracle.logits_grad(case.x[rows], case.targets[rows], 1.0, gl[rows], ge[rows])
    check(gs, ref, tolerance(case.x[rows], case.targets[rows], 1.0, gl[rows], ge[rows]))
    # every row sums to 0 (shift invariance), up to fp32 rounding of 151936 terms
    sums = g.double().sum(dim=1).abs().max().item()
    scale = (gld.abs() + ged.abs() * 20).max().item()
    print(f"max |row sum| {sums:.3e}")
    assert sums <= 1e-4 * scale


def test_qwen3_vocab_split_batch_order_repeats_bitwise(lib, cfg2):
    import torch
    case, gl, ge, xd, td, gld, ged = cfg2
    ref = lib.logprob_backward_from_logits(xd, td, 1.0, 1, gld, ged).cpu()
    for split in (2, 8):
        announce(f"grad T=1024 split={split} vs 1")
        g = lib.logprob_backward_from_logits(xd, td, 1.0, split, gld, ged).cpu()
        assert torch.equal(g.view(torch.int32), ref.view(torch.int32)), split
    perm = torch.from_numpy(S.permutations(2, 1024, 1)[0]).cuda()
    announce("grad T=1024 permuted rows")
    gp = lib.logprob_backward_from_logits(xd[perm].contiguous(), td[perm].contiguous(), 1.0, 1,
                                          gld[perm].contiguous(), ged[perm].contiguous()).cpu()
    assert torch.equal(gp.view(torch.int32), ref[perm.cpu()].view(torch.int32))
    for lo, hi in [(0, 1), (100, 357), (1000, 1024)]:
        announce(f"grad rows [{lo},{hi}) alone, split 4")
        gs = lib.logprob_backward_from_logits(xd[lo:hi], td[lo:hi], 1.0, 4, gld[lo:hi],
                                              ged[lo:hi]).cpu()
        assert torch.equal(gs.view(torch.int32), ref[lo:hi].view(torch.int32))
    again = lib.logprob_backward_from_logits(xd, td, 1.0, 1, gld, ged).cpu()
    assert torch.equal(again.view(torch.int32), ref.view(torch.int32))


def test_saved_row_states_give_the_same_bits(lib):
    """Row states saved by the forward call (at any vocab split) skip the recompute and give
    the recomputing backward's bits; the forward outputs do not change when they are saved."""
    import torch
    T, V = 40, 30011
    case = S.random_logits_case(T, V, 3.0, seed=86)
    gl, ge = weights(T, 87)
    xd, td, gld, ged = dev(case.x), dev(case.targets), dev(gl), dev(ge)
    announce("grad with saved row states")
    ref = lib.logprob_backward_from_logits(xd, td, 0.7, 1, gld, ged).cpu()
    lp0, ent0 = lib.logprob_from_logits(xd, td, 0.7, 1)
    for split in (1, 4):
        states = lib.row_states_buffer(T)
        lp, ent = lib.logprob_from_logits(xd, td, 0.7, split, row_states=states)
        assert torch.equal(lp.view(torch.int32), lp0.view(torch.int32))
        assert torch.equal(ent.view(torch.int32), ent0.view(torch.int32))
        g = lib.logprob_backward_from_logits(xd, td, 0.7, 1, gld, ged, row_states=states).cpu()
        assert torch.equal(g.view(torch.int32), ref.view(torch.int32)), split
