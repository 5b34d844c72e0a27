"""Large-size cases: row offsets past 2^31 bytes on the logits path, thousands of tiles per
chunk (a deep tile tree) on the fused path, against the fp64 oracle; T = 0 backward calls."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import TOL_LINEAR, TOL_LOGITS, announce, bits_dev, dev, max_abs, run_logits

pytestmark = pytest.mark.gpu


def test_logits_rows_beyond_2gib(lib):
    """3 rows of V = 2^28 + 3 fp32 logits: the last row starts past 2^31 bytes, every chunk
    is ~134 MB, and V is not a multiple of 4 (element loads on every row after the first)."""
    import torch
    T, V = 3, (1 << 28) + 3
    announce(f"generating logits T={T} V={V}")
    rng = np.random.default_rng(1234)
    x = rng.standard_normal((T, V), dtype=np.float32) * np.float32(2.0)
    t = np.array([5, V - 1, V // 2], dtype=np.int64)
    announce(f"logits T={T} V={V}")
    lp, ent = run_logits(lib, x, t, 1.0, 1)
    lp4, ent4 = run_logits(lib, x, t, 1.0, 4)
    assert lp.tobytes() == lp4.tobytes() and ent.tobytes() == ent4.tobytes()
    olp, oent = oracle.logprob_entropy(x, t)
    assert max_abs(lp, olp) <= TOL_LOGITS and max_abs(ent, oent) <= TOL_LOGITS
    del torch


def test_fused_deep_tile_tree(lib):
    """V = 2^23 + 5, d = 64: 4097 tiles per chunk (an 8192-leaf tile tree), vocab splits 1
    and 8 bitwise, against fp64 dot products of the bf16 values."""
    T, d, V = 5, 64, (1 << 23) + 5
    announce(f"generating fused T={T} d={d} V={V}")
    case = S.random_fused_case(T, d, V, seed=4321, w_sigma=0.35)
    h = S.bf16_bits_to_f32(case.h_bits).astype(np.float64)
    x = np.empty((T, V))
    for lo in range(0, V, 1 << 20):                  # fp64 logits in vocabulary blocks
        hi = min(V, lo + (1 << 20))
        x[:, lo:hi] = h @ S.bf16_bits_to_f32(case.w_bits[lo:hi]).astype(np.float64).T
    olp, oent = oracle.logprob_entropy(x, case.targets)
    hd, wd, td = bits_dev(case.h_bits), bits_dev(case.w_bits), dev(case.targets)
    import torch
    announce(f"fused T={T} d={d} V={V}")
    out = []
    for split in (1, 8):
        lp, ent = lib.linear_logprob(hd, wd, td, 1.0, split)
        torch.cuda.synchronize()
        out.append((lp.cpu().numpy(), ent.cpu().numpy()))
    assert out[0][0].tobytes() == out[1][0].tobytes() and out[0][1].tobytes() == out[1][1].tobytes()
    assert max_abs(out[0][0], olp) <= TOL_LINEAR and max_abs(out[0][1], oent) <= TOL_LINEAR


def test_backward_calls_with_no_tokens(lib):
    import torch
    x = torch.empty((0, 100), dtype=torch.float32, device="cuda")
    t = torch.empty((0,), dtype=torch.int64, device="cuda")
    g = lib.logprob_backward_from_logits(x, t, 1.0, 1, torch.empty(0, device="cuda"), None)
    h = torch.empty((0, 64), dtype=torch.int16, device="cuda")
    w = torch.zeros((10, 64), dtype=torch.int16, device="cuda")
    dh, dw = lib.linear_logprob_backward(h, w, t, 1.0, 1, torch.empty(0, device="cuda"), None)
    torch.cuda.synchronize()
    assert g.numel() == 0 and dh.numel() == 0 and dw.shape == (10, 64)
    # the weight gradient of an empty batch is zero, also into a strided caller buffer whose
    # padding columns must stay untouched
    assert torch.equal(dw, torch.zeros_like(dw))
    buf = torch.full((10, 72), 7.0, device="cuda")
    lib.linear_logprob_backward(h, w, t, 1.0, 1, None, None, need_hidden=False,
                                out=(None, buf[:, :64]))
    torch.cuda.synchronize()
    assert torch.equal(buf[:, :64], torch.zeros(10, 64, device="cuda"))
    assert torch.equal(buf[:, 64:], torch.full((10, 8), 7.0, device="cuda"))
