"""The library's calls inside a captured HIP graph: every entry point launches kernels only
(no allocation, no memset, no synchronization), so a captured sequence replays with the
eager bits -- checked on several replays with eager work and synchronizations between."""
from __future__ import annotations

import math

import numpy as np
import pytest

from entropy_rlk_logprob_amd import binding as B
from entropy_rlk_logprob_amd import synthetic as S
from tests.helpers import announce, bits_dev, dev

pytestmark = pytest.mark.gpu


def test_captured_sequence_replays_with_eager_bits(lib):
    import torch
    T, V, d = 96, 20011, 128
    lc = S.random_logits_case(T, V, 3.0, seed=120)
    fc = S.random_fused_case(T, d, V, seed=121, w_sigma=3.0 / math.sqrt(d))
    rng = np.random.default_rng(122)
    gl = dev(rng.normal(size=T).astype(np.float32))
    ge = dev(rng.normal(size=T).astype(np.float32))
    x, t = dev(lc.x), dev(lc.targets)
    h, w, tf = bits_dev(fc.h_bits), bits_dev(fc.w_bits), dev(fc.targets)
    # A second fused batch above 128 tokens runs the persistent tile kernel (the batch of 96
    # runs the paired-tile kernel).
    T2 = 300
    fc2 = S.random_fused_case(T2, d, V, seed=123, w_sigma=3.0 / math.sqrt(d))
    h2, tf2 = bits_dev(fc2.h_bits), dev(fc2.targets)
    mask = torch.ones(T, dtype=torch.uint8, device="cuda")

    # every output and workspace exists before capture
    def buffers():
        return dict(
            lp=torch.empty(T, device="cuda"), ent=torch.empty(T, device="cuda"),
            st=lib.row_states_buffer(T), grad=torch.empty((T, V), device="cuda"),
            flp=torch.empty(T, device="cuda"), fent=torch.empty(T, device="cuda"),
            fst=lib.row_states_buffer(T), dh=torch.empty((T, d), device="cuda"),
            dw=torch.empty((V, d), device="cuda"), cmp=torch.empty(64, dtype=torch.uint8,
                                                                  device="cuda"),
            flp2=torch.empty(T2, device="cuda"), fent2=torch.empty(T2, device="cuda"))
    ws = {op: torch.empty(max(1, lib.workspace_bytes(op, T, V, dd, 4)), dtype=torch.uint8,
                          device="cuda")
          for op, dd in ((B.OP_FROM_LOGITS, 0), (B.OP_BACKWARD_FROM_LOGITS, 0),
                         (B.OP_LINEAR, d), (B.OP_LINEAR_BACKWARD, d))}
    ws_cmp = torch.empty(max(1, lib.workspace_bytes(B.OP_COMPARE, T, 1)), dtype=torch.uint8,
                         device="cuda")
    ws2 = torch.empty(lib.workspace_bytes(B.OP_LINEAR, T2, V, d, 1), dtype=torch.uint8,
                      device="cuda")

    def sequence(o):
        lib.logprob_from_logits(x, t, 0.7, 4, out=(o["lp"], o["ent"]),
                                workspace=ws[B.OP_FROM_LOGITS], row_states=o["st"])
        lib.logprob_backward_from_logits(x, t, 0.7, 4, gl, ge, out=o["grad"],
                                         workspace=ws[B.OP_BACKWARD_FROM_LOGITS],
                                         row_states=o["st"])
        lib.linear_logprob(h, w, tf, 1.0, 4, out=(o["flp"], o["fent"]),
                           workspace=ws[B.OP_LINEAR], row_states=o["fst"])
        lib.linear_logprob_backward(h, w, tf, 1.0, 4, gl, ge, out=(o["dh"], o["dw"]),
                                    workspace=ws[B.OP_LINEAR_BACKWARD], row_states=o["fst"])
        lib.logprob_compare_async(o["lp"], o["flp"], mask, out=o["cmp"], workspace=ws_cmp)
        lib.linear_logprob(h2, w, tf2, 0.7, 1, out=(o["flp2"], o["fent2"]), workspace=ws2)

    announce("graph capture: eager reference")
    eager = buffers()
    sequence(eager)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}

    announce("graph capture: capture")
    cap = buffers()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sequence(cap)                  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for v in cap.values():
        v.zero_()
    with torch.cuda.graph(g):
        sequence(cap)
    for replay in range(3):
        announce(f"graph capture: replay {replay}")
        for v in cap.values():
            v.fill_(7)                 # stale contents must be overwritten
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            a, b = cap[k], ref[k]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (replay, k)
        sequence(eager)                # eager work between replays
        torch.cuda.synchronize()
