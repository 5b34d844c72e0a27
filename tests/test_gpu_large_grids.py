"""Launch grids with more blocks than one dispatch dimension holds (2^22 here): the kernels
then take the split (x, z) grid.  Rows and tiles beyond the split must match the oracle or a
closed form, and give the same bits as in a small batch (whose grid is not split)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from tests.helpers import TOL_LOGITS, announce, bitwise_equal, dev, max_abs
from tests.test_gpu_backward import check, tolerance

pytestmark = pytest.mark.gpu

SPLIT = 1 << 22  # blocks along x before the grid is split over z


def test_logits_path_and_backward_past_the_grid_split(lib):
    """T = 2^22 + 1000 rows of V = 3: one workgroup per row, so the last 1000 rows sit in the
    second z slice of the grid."""
    import torch
    T, V = SPLIT + 1000, 3
    announce(f"logits T={T} V={V} (split grid)")
    rng = np.random.default_rng(4242)
    x = rng.normal(0.0, 2.0, (T, V)).astype(np.float32)
    t = rng.integers(0, V, T).astype(np.int64)
    xd, td = dev(x), dev(t)
    lp, ent = lib.logprob_from_logits(xd, td)
    torch.cuda.synchronize()
    lp, ent = lp.cpu().numpy(), ent.cpu().numpy()
    olp, oent = oracle.logprob_entropy(x, t)
    assert max_abs(lp, olp) <= TOL_LOGITS and max_abs(ent, oent) <= TOL_LOGITS
    lo = T - 2000  # straddles the split
    lps, ents = lib.logprob_from_logits(xd[lo:], td[lo:])
    torch.cuda.synchronize()
    assert bitwise_equal(lps.cpu().numpy(), lp[lo:]) and bitwise_equal(ents.cpu().numpy(), ent[lo:])
    lp4, ent4 = lib.logprob_from_logits(xd, td, 1.0, 4)
    torch.cuda.synchronize()
    assert bitwise_equal(lp4.cpu().numpy(), lp) and bitwise_equal(ent4.cpu().numpy(), ent)

    announce(f"logits backward T={T} V={V} (split grid)")
    gl = rng.normal(size=T).astype(np.float32)
    ge = rng.normal(size=T).astype(np.float32)
    gld, ged = dev(gl), dev(ge)
    g = lib.logprob_backward_from_logits(xd, td, 1.0, 1, gld, ged)
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 64), SPLIT - 8 + np.arange(16),
                                     T - 64 + np.arange(64),
                                     rng.integers(0, T, 256)]))
    ref = oracle.logits_grad(x[rows], t[rows], 1.0, gl[rows], ge[rows])
    check(g[rows], ref, tolerance(x[rows], t[rows], 1.0, gl[rows], ge[rows]))
    gs = lib.logprob_backward_from_logits(xd[lo:], td[lo:], 1.0, 1, gld[lo:], ged[lo:])
    torch.cuda.synchronize()
    assert bitwise_equal(gs.cpu().numpy(), g[lo:])


def two_level(delta, k, V):
    """Closed forms for logits taking the value delta on k of V entries and 0 elsewhere:
    (logprob at a delta entry, logprob at a 0 entry, entropy), in nats."""
    Z = k * math.exp(delta) + (V - k)
    lnZ = math.log(Z)
    ent = lnZ - k * delta * math.exp(delta) / Z
    return delta - lnZ, -lnZ, ent


def test_fused_tiles_past_the_grid_split(lib):
    """V = 2^26, d = 64, T = 4352: 262144 vocabulary tiles x 17 token tiles = 4456448 tiles,
    so the tile grid is split.  The weight holds delta in column 0 of one row per vocabulary
    tile (row 256 j + j % 256) and zeros elsewhere, the hidden rows hold s_t in column 0, so a
    token's logits are two-level (s_t delta on 262144 entries, 0 on the rest): a tile that is
    skipped or taken twice changes the sum.  All rows against the closed form; the first and
    last 256 rows alone (unsplit grids) give the same bits."""
    import torch
    V, d, T = 1 << 26, 64, 17 * 256
    n_vt = V // 256
    announce(f"linear T={T} d={d} V={V} (split tile grid)")
    delta = 2.0
    w = torch.zeros((V, d), dtype=torch.bfloat16, device="cuda")
    j = torch.arange(n_vt, device="cuda", dtype=torch.int64)
    w[256 * j + (j % 256), 0] = delta
    scales = np.array([1.0, 0.5, 2.0, 0.25], np.float32)
    s_t = scales[np.arange(T) % 4]
    h = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    h[:, 0] = torch.from_numpy(s_t).cuda().to(torch.bfloat16)
    hi_rows = 256 * np.arange(n_vt, dtype=np.int64) + (np.arange(n_vt) % 256)
    rng = np.random.default_rng(4343)
    q = rng.integers(0, n_vt, T)  # odd rows: another row of tile q than its delta row
    lo_rows = 256 * q + (q % 256 + 1 + rng.integers(0, 255, T)) % 256
    t = np.where(np.arange(T) % 2 == 0, hi_rows[rng.integers(0, n_vt, T)], lo_rows)
    assert not np.isin(t[1::2], hi_rows).any()
    td = dev(t.astype(np.int64))
    hv, wv = h.view(torch.int16), w.view(torch.int16)
    lp, ent = lib.linear_logprob(hv, wv, td)
    torch.cuda.synchronize()
    lp, ent = lp.cpu().numpy(), ent.cpu().numpy()
    exp_lp = np.empty(T)
    exp_ent = np.empty(T)
    for i, s in enumerate(scales):
        hi, lo_, e = two_level(float(s) * delta, n_vt, V)
        sel = np.arange(T) % 4 == i
        exp_lp[sel] = np.where(np.arange(T)[sel] % 2 == 0, hi, lo_)
        exp_ent[sel] = e
    # The logits are exact, so only the fp32 softmax arithmetic is left (well inside the
    # fused path's tolerance).
    assert max_abs(lp, exp_lp) <= 2e-5 and max_abs(ent, exp_ent) <= 2e-5
    for a, b in ((0, 256), (T - 256, T)):
        announce(f"linear rows [{a},{b}) alone")
        lps, ents = lib.linear_logprob(hv[a:b], wv, td[a:b])
        torch.cuda.synchronize()
        assert bitwise_equal(lps.cpu().numpy(), lp[a:b]) and bitwise_equal(ents.cpu().numpy(),
                                                                           ent[a:b])
