"""GPU parity of rlk_linear_logprob_backward (dH = dX W, dW = dX^T H) against the fp64
oracle, and its strictness: each row of dH bitwise independent of the rest of the batch,
both gradients bitwise independent of the vocab split and of repeats."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from entropy_rlk_logprob_amd import binding as B
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import announce, bits_dev, bitwise_equal, dev

pytestmark = pytest.mark.gpu


def f32(bits):
    return S.bf16_bits_to_f32(bits).astype(np.float64)


def run_bwd(lib, h, w, t, tau, split, gl, ge, need_hidden=True, need_weight=True):
    import torch
    hd = h if isinstance(h, torch.Tensor) else bits_dev(h)
    wd = w if isinstance(w, torch.Tensor) else bits_dev(w)
    td = None if t is None else (t if isinstance(t, torch.Tensor) else dev(np.asarray(t, np.int64)))
    gld = None if gl is None else (gl if isinstance(gl, torch.Tensor) else dev(gl))
    ged = None if ge is None else (ge if isinstance(ge, torch.Tensor) else dev(ge))
    dh, dw = lib.linear_logprob_backward(hd, wd, td, tau, split, gld, ged, need_hidden,
                                         need_weight)
    torch.cuda.synchronize()
    return (None if dh is None else dh.cpu().numpy(), None if dw is None else dw.cpu().numpy())


def bound(gx, other, K):
    """|error| bound of a product dX . other computed from bf16(dX) with fp32 accumulation
    over K terms: bf16 rounding of dX (2^-9, taken as 2^-8) plus the worst-case fp32
    accumulation K * 2^-24, both of sum |dX| |other|."""
    mag = np.abs(gx) @ np.abs(other)
    return (2.0 ** -8 + K * 2.0 ** -24) * mag + 1e-30


def check(gpu, ref, tol):
    assert np.array_equal(np.isnan(gpu), np.isnan(ref)), "NaN pattern differs"
    fin = ~np.isnan(ref)
    err = np.abs(gpu[fin].astype(np.float64) - ref[fin])
    assert np.all(err <= tol[fin]), (float(err.max()), float((err / tol[fin]).max()))


def weights(T, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(size=T).astype(np.float32), rng.normal(size=T).astype(np.float32)


@pytest.mark.parametrize("T,d,V,tau", [
    (3, 64, 100, 1.0), (37, 128, 1000, 0.7), (300, 192, 5003, 1.0), (513, 64, 2049, 1.0),
    (64, 512, 20000, 0.7), (777, 320, 12345, 0.7), (1100, 256, 3001, 1.0),
])
def test_shapes_vs_oracle_and_split_bitwise(lib, T, d, V, tau):
    announce(f"linear backward T={T} d={d} V={V} tau={tau}")
    case = S.random_fused_case(T, d, V, seed=9500 + T + V, h_sigma=1.0,
                               w_sigma=3.0 / math.sqrt(d), temperature=tau)
    gl, ge = weights(T, T + V)
    h, w = f32(case.h_bits), f32(case.w_bits)
    gx = oracle.logits_grad(h @ w.T, case.targets, tau, gl, ge)
    ref_dh, ref_dw = gx @ w, gx.T @ h
    Vp, Tp = -(-V // 64) * 64, -(-T // 64) * 64
    tol_dh, tol_dw = bound(gx, w, Vp), bound(gx.T, h, Tp)
    first = None
    for split in (1, 4):
        dh, dw = run_bwd(lib, case.h_bits, case.w_bits, case.targets, tau, split, gl, ge)
        check(dh, ref_dh, tol_dh)
        check(dw, ref_dw, tol_dw)
        if first is None:
            first = (dh, dw)
        else:
            assert bitwise_equal(dh, first[0]) and bitwise_equal(dw, first[1]), split
    # one gradient at a time gives the same bits
    dh_only, none_w = run_bwd(lib, case.h_bits, case.w_bits, case.targets, tau, 1, gl, ge, True,
                              False)
    none_h, dw_only = run_bwd(lib, case.h_bits, case.w_bits, case.targets, tau, 1, gl, ge, False,
                              True)
    assert none_w is None and none_h is None
    assert bitwise_equal(dh_only, first[0]) and bitwise_equal(dw_only, first[1])


def test_tile_groups_with_partial_last_group(lib):
    """T = 2600 (11 token tiles) and d = 2304 (9 hidden tiles): the tile grids of the
    logit-gradient kernel and of both GEMMs run a full group of 8 column tiles and a
    partial one.  dH and dW against the oracle; dH rows of the partial token group alone
    give the same bits."""
    T, d, V = 2600, 2304, 1000
    announce(f"linear backward T={T} d={d} V={V} (tile groups 8 + 3 and 8 + 1)")
    case = S.random_fused_case(T, d, V, seed=9600, h_sigma=1.0, w_sigma=3.0 / math.sqrt(d))
    gl, ge = weights(T, 9601)
    h, w = f32(case.h_bits), f32(case.w_bits)
    gx = oracle.logits_grad(h @ w.T, case.targets, 1.0, gl, ge)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gld, ged = dev(gl), dev(ge)
    dh, dw = run_bwd(lib, hd, wd, td, 1.0, 1, gld, ged)
    check(dh, gx @ w, bound(gx, w, -(-V // 64) * 64))
    check(dw, gx.T @ h, bound(gx.T, h, -(-T // 64) * 64))
    lo = 8 * 256
    part, _ = run_bwd(lib, hd[lo:], wd, td[lo:], 1.0, 1, gld[lo:], ged[lo:], True, False)
    assert bitwise_equal(part, dh[lo:])


def test_entropy_only_and_masked_rows(lib):
    T, d, V = 70, 128, 3001
    case = S.random_fused_case(T, d, V, seed=96, w_sigma=0.25)
    rng = np.random.default_rng(97)
    ge = rng.normal(size=T).astype(np.float32)
    ge[::5] = 0.0                                   # masked rows (no logprob gradient either)
    announce("linear backward entropy only, masked rows")
    h, w = f32(case.h_bits), f32(case.w_bits)
    gx = oracle.logits_grad(h @ w.T, np.zeros(T, np.int64), 1.0, None, ge)
    dh, dw = run_bwd(lib, case.h_bits, case.w_bits, None, 1.0, 1, None, ge)
    check(dh, gx @ w, bound(gx, w, -(-V // 64) * 64))
    check(dw, gx.T @ h, bound(gx.T, h, -(-T // 64) * 64))
    assert np.all(dh[::5] == 0.0)


def test_rows_of_dh_independent_of_batch(lib):
    """Sequences of a packed batch alone give the packed rows of dH bitwise."""
    import torch
    T, d, V = 640, 256, 20011
    case = S.random_fused_case(T, d, V, seed=98, w_sigma=3.0 / math.sqrt(d))
    gl, ge = weights(T, 99)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gld, ged = dev(gl), dev(ge)
    announce("linear backward packed batch")
    dh, _ = run_bwd(lib, hd, wd, td, 1.0, 1, gld, ged, True, False)
    for lo, hi in [(0, 1), (1, 129), (129, 600), (600, 640)]:
        announce(f"linear backward rows [{lo},{hi}) alone")
        part, _ = run_bwd(lib, hd[lo:hi], wd, td[lo:hi], 1.0, 1, gld[lo:hi], ged[lo:hi], True,
                          False)
        assert bitwise_equal(part, dh[lo:hi]), (lo, hi)
    perm = torch.from_numpy(np.random.default_rng(100).permutation(T)).cuda()
    dhp, _ = run_bwd(lib, hd[perm].contiguous(), wd, td[perm].contiguous(), 1.0, 1,
                     gld[perm].contiguous(), ged[perm].contiguous(), True, False)
    assert bitwise_equal(dhp, dh[perm.cpu().numpy()])


def test_qwen3_vocab_full_hidden_vs_oracle(lib):
    """V = 151936, d = 4096, T = 256 (several token tiles of work per vocabulary tile):
    sampled rows of dH and sampled vocabulary rows of dW against the oracle; repeats bitwise."""
    T, d, V = 256, 4096, 151936
    announce("generating linear backward case T=256 d=4096 V=151936")
    case = S.random_fused_case(T, d, V, seed=101, h_sigma=1.0, w_sigma=0.02)
    gl, ge = weights(T, 102)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gld, ged = dev(gl), dev(ge)
    announce("linear backward T=256 d=4096 V=151936")
    dh, dw = run_bwd(lib, hd, wd, td, 1.0, 1, gld, ged)
    h = f32(case.h_bits)
    w = f32(case.w_bits)
    gx = np.empty((T, V))
    for lo in range(0, T, 32):                       # row blocks keep the fp64 logits small
        gx[lo:lo + 32] = oracle.logits_grad(h[lo:lo + 32] @ w.T, case.targets[lo:lo + 32], 1.0,
                                            gl[lo:lo + 32], ge[lo:lo + 32])
    rows = np.array([0, 1, 77, 128, 255])
    check(dh[rows], gx[rows] @ w, bound(gx[rows], w, V))
    vrows = np.unique(np.concatenate([[0, 1, 255, 256, 18991, 18992, 151935],
                                      np.random.default_rng(103).integers(0, V, 20)]))
    check(dw[vrows], gx[:, vrows].T @ h, bound(gx[:, vrows].T, h, T))
    announce("linear backward T=256 repeat and split 8")
    dh2, dw2 = run_bwd(lib, hd, wd, td, 1.0, 8, gld, ged)
    assert bitwise_equal(dh2, dh) and bitwise_equal(dw2, dw)


def test_vocab_past_the_buffer_load_limit_vs_oracle(lib):
    """V = 2^22 + 100: the logit gradient's padded row stride Vp exceeds 2^22, so dH stages
    its operands with global-address loads instead of buffer loads to LDS (whose 32-bit
    per-lane offsets it would overflow).  dH and sampled vocabulary rows of dW against the
    oracle (the last rows included); vocab split 4 bitwise."""
    T, d, V = 3, 64, (1 << 22) + 100
    announce(f"generating linear backward case T={T} d={d} V={V}")
    case = S.random_fused_case(T, d, V, seed=105, h_sigma=1.0, w_sigma=3.0 / math.sqrt(d))
    gl, ge = weights(T, 106)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gld, ged = dev(gl), dev(ge)
    announce(f"linear backward T={T} d={d} V={V} (global-address loads for dH)")
    dh, dw = run_bwd(lib, hd, wd, td, 1.0, 1, gld, ged)
    h = f32(case.h_bits)
    w = f32(case.w_bits)
    gx = oracle.logits_grad(h @ w.T, case.targets, 1.0, gl, ge)
    check(dh, gx @ w, bound(gx, w, V))
    vrows = np.unique(np.concatenate([[0, 1, 255, 256, V - 101, V - 2, V - 1],
                                      np.random.default_rng(107).integers(0, V, 20)]))
    check(dw[vrows], gx[:, vrows].T @ h, bound(gx[:, vrows].T, h, T))
    announce(f"linear backward T={T} d={d} V={V} split 4")
    dh4, dw4 = run_bwd(lib, hd, wd, td, 1.0, 4, gld, ged)
    assert bitwise_equal(dh4, dh) and bitwise_equal(dw4, dw)


def test_saved_row_states_give_the_same_bits(lib):
    import torch
    T, d, V = 200, 128, 9001
    case = S.random_fused_case(T, d, V, seed=104, w_sigma=3.0 / math.sqrt(d), temperature=0.7)
    gl, ge = weights(T, 105)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gld, ged = dev(gl), dev(ge)
    announce("linear backward with saved row states")
    dh0, dw0 = lib.linear_logprob_backward(hd, wd, td, 0.7, 1, gld, ged)
    lp0, ent0 = lib.linear_logprob(hd, wd, td, 0.7, 1)
    for split in (1, 2):
        states = lib.row_states_buffer(T)
        lp, ent = lib.linear_logprob(hd, wd, td, 0.7, split, row_states=states)
        assert torch.equal(lp.view(torch.int32), lp0.view(torch.int32))
        assert torch.equal(ent.view(torch.int32), ent0.view(torch.int32))
        dh, dw = lib.linear_logprob_backward(hd, wd, td, 0.7, 1, gld, ged, row_states=states)
        assert torch.equal(dh.view(torch.int32), dh0.view(torch.int32)), split
        assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32)), split


def test_strided_operands_give_the_same_bits(lib):
    """Hidden states and LM head given as column slices of wider tensors (row strides above
    d; W is read in place by the dH contraction) give the contiguous inputs' bits."""
    import torch
    T, d, V = 100, 192, 3001
    case = S.random_fused_case(T, d, V, seed=106, w_sigma=3.0 / math.sqrt(d))
    gl, ge = weights(T, 107)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    gld, ged = dev(gl), dev(ge)
    announce("linear backward strided hidden and weight")
    dh0, dw0 = lib.linear_logprob_backward(hd, wd, td, 1.0, 1, gld, ged)
    h_big = torch.zeros((T, d + 64), dtype=torch.int16, device="cuda")
    w_big = torch.zeros((V, d + 72), dtype=torch.int16, device="cuda")
    h_big[:, 8:8 + d] = hd
    w_big[:, 16:16 + d] = wd
    dh, dw = lib.linear_logprob_backward(h_big[:, 8:8 + d], w_big[:, 16:16 + d], td, 1.0, 1, gld,
                                         ged)
    assert torch.equal(dh.view(torch.int32), dh0.view(torch.int32))
    assert torch.equal(dw.view(torch.int32), dw0.view(torch.int32))


def test_chunked_weight_gradient_continues_the_earlier_chunks(lib):
    """The backward runs over the tokens in chunks of 4096; each chunk's share of dW is
    accumulated onto the stored sum of the chunks before it (the MFMA accumulators start from
    it), so dW is one fp32 sum in increasing token order whatever the chunking.  A row whose
    two upstream gradients are 0 has an all-zero logit gradient and adds exact zeros, so
    masking the rows of some chunks must give the dW of the other rows run alone (equal
    values; only the sign of a zero may differ), and the unmasked rows' dH bits."""
    T, d, V = 8300, 128, 1500       # chunks of 4096, 4096 and 108 tokens
    announce(f"linear backward T={T} d={d} V={V} (token chunks)")
    case = S.random_fused_case(T, d, V, seed=9700, h_sigma=1.0, w_sigma=3.0 / math.sqrt(d))
    gl, ge = weights(T, 9701)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    h, w = f32(case.h_bits), f32(case.w_bits)
    gx = oracle.logits_grad(h @ w.T, case.targets, 1.0, gl, ge)
    dh, dw = run_bwd(lib, hd, wd, td, 1.0, 1, dev(gl), dev(ge))
    check(dh, gx @ w, bound(gx, w, -(-V // 64) * 64))
    check(dw, gx.T @ h, bound(gx.T, h, -(-T // 64) * 64))
    for lo, hi in ((0, 4096), (4096, T), (3000, 5000), (8192, T)):
        announce(f"linear backward: rows [{lo},{hi}) unmasked, alone vs in the batch")
        glm, gem = np.zeros_like(gl), np.zeros_like(ge)
        glm[lo:hi], gem[lo:hi] = gl[lo:hi], ge[lo:hi]
        dh_m, dw_m = run_bwd(lib, hd, wd, td, 1.0, 1, dev(glm), dev(gem))
        dh_a, dw_a = run_bwd(lib, hd[lo:hi], wd, td[lo:hi], 1.0, 1, dev(gl[lo:hi]),
                             dev(ge[lo:hi]))
        assert np.array_equal(dw_m, dw_a), (lo, hi)
        assert bitwise_equal(dh_m[lo:hi], dh_a) and np.all(dh_m[:lo] == 0) and \
            np.all(dh_m[hi:] == 0)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_fused_workload_backward_sampled_rows_vs_oracle(lib, cfg):
    """Each fused workload (T = 1024 / d = 2048; T = 2048 / d = 4096; T = 16384 / d = 4096,
    tau = 0.7, the golden targets) with seeded upstream gradients (every 7th row masked):
    48 rows of dH and 48 rows of dW against the fp64 oracle (tests/golden,
    oracle.linear_grads_sampled) within the bf16-rounding + fp32-accumulation bound, and
    vocab split 4 bitwise equal to split 1.  At T = 16384 the workspace is that of one
    4096-token chunk (the call runs four)."""
    import torch
    from tests.helpers import load_fused_golden
    wl = S.WORKLOADS[cfg]
    fwd = load_fused_golden(wl.name)
    import json
    import os
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "fused_goldens.json")) as f:
        meta = json.load(f)["backward"][wl.name]
    with np.load(os.path.join(here, meta["file"]), allow_pickle=False) as z:
        g = {k: z[k] for k in z.files}
    announce(f"generating fused workload {wl.name} (backward)")
    case = S.fused_workload(cfg)
    T, d = case.h_bits.shape
    V = case.w_bits.shape[0]
    tau = wl.temperature
    gl, ge = S.upstream_grads(cfg, T)
    if T > 4096:
        assert lib.workspace_bytes(B.OP_LINEAR_BACKWARD, T, V, d, 1) == \
            lib.workspace_bytes(B.OP_LINEAR_BACKWARD, 4096, V, d, 1)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(fwd["targets"])
    gld, ged = dev(gl), dev(ge)
    announce(f"linear backward T={T} d={d} split=1")
    dh, dw = lib.linear_logprob_backward(hd, wd, td, tau, 1, gld, ged)
    torch.cuda.synchronize()
    hr, wr = torch.from_numpy(g["h_rows"]).cuda(), torch.from_numpy(g["w_rows"]).cuda()
    dh_s, dw_s = dh[hr].cpu().numpy(), dw[wr].cpu().numpy()
    Vp, Tp = -(-V // 64) * 64, -(-T // 64) * 64
    check(dh_s, g["dh"], (2.0 ** -8 + Vp * 2.0 ** -24) * g["dh_mag"] + 1e-30)
    check(dw_s, g["dw"], (2.0 ** -8 + Tp * 2.0 ** -24) * g["dw_mag"] + 1e-30)
    rel_dh = np.abs(dh_s - g["dh"]).max() / np.abs(g["dh"]).max()
    rel_dw = np.abs(dw_s - g["dw"]).max() / np.abs(g["dw"]).max()
    print(f"[T={T} d={d} backward] max |err| / max |ref|: dH {rel_dh:.2e}, dW {rel_dw:.2e}",
          flush=True)
    masked = np.flatnonzero((gl[g["h_rows"]] == 0) & (ge[g["h_rows"]] == 0))
    assert masked.size > 0 and np.all(dh_s[masked] == 0)
    announce(f"linear backward T={T} d={d} split=4")
    dh4, dw4 = lib.linear_logprob_backward(hd, wd, td, tau, 4, gld, ged)
    torch.cuda.synchronize()
    assert torch.equal(dh4.view(torch.int32), dh.view(torch.int32))
    assert torch.equal(dw4.view(torch.int32), dw.view(torch.int32))
