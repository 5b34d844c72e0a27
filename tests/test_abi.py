"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, sizes
workspaces on the host, and rejects bad arguments before touching any device.

Pointers passed here are never dereferenced: validation is host-only and returns before
anything is launched.  The one test that reaches the device check (valid arguments on a
machine without a gfx950 GPU) is skipped wherever a GPU is visible, since there it would
launch kernels on those placeholder pointers.
"""
from __future__ import annotations

import ctypes
import math

import struct

import pytest

from entropy_rlk_logprob_amd import binding as B

FAKE = 0x10000  # placeholder device address (never dereferenced on these paths)


@pytest.fixture(scope="module")
def L():
    return B.load()


def no_gpu_visible() -> bool:
    import torch
    return torch.cuda.device_count() == 0


def test_exports_every_header_symbol(L):
    names = B.header_functions()
    assert set(names) == {"rlk_workspace_bytes", "rlk_logprob_from_logits", "rlk_linear_logprob",
                          "rlk_entropy", "rlk_status_string", "rlk_backend_id",
                          "rlk_logprob_from_logits_with_states",
                          "rlk_linear_logprob_with_states", "rlk_linear_logprob_noalloc",
                          "rlk_logprob_from_logits_bf16", "rlk_entropy_bf16",
                          "rlk_logprob_compare", "rlk_logprob_backward_from_logits",
                          "rlk_linear_logprob_backward"}
    for n in names:
        assert hasattr(L.lib, n), n
        assert ctypes.cast(getattr(L.lib, n), ctypes.c_void_p).value


def test_probe_library_exports_its_header():
    """librlk_probes.so (the benchmark's measurement probes) exports what
    include/rlk_probes.h declares and rejects bad arguments without launching."""
    names = B.header_functions(B.PROBES_HEADER)
    assert set(names) == {"rlk_probe_stream_read", "rlk_probe_mfma", "rlk_probe_device_info"}
    P = B.load_probes()
    for n in names:
        assert ctypes.cast(getattr(P.lib, n), ctypes.c_void_p).value
    vp = ctypes.c_void_p
    assert P.lib.rlk_probe_stream_read(None, 1024, vp(FAKE), None) == -1
    assert P.lib.rlk_probe_stream_read(vp(FAKE), 1000, vp(FAKE), None) == -1     # not 16 B
    assert P.lib.rlk_probe_stream_read(vp(FAKE + 8), 1024, vp(FAKE), None) == -1  # misaligned
    assert P.lib.rlk_probe_mfma(0, 4, 1, vp(FAKE), None) == -1
    assert P.lib.rlk_probe_mfma(1, 6, 1, vp(FAKE), None) == -1                    # iters % 4
    assert P.lib.rlk_probe_mfma(1, 4, 1, None, None) == -1
    i32 = ctypes.c_int32()
    assert P.lib.rlk_probe_device_info(None, ctypes.byref(i32), ctypes.byref(i32),
                                       ctypes.byref(i32), ctypes.create_string_buffer(8), 8) == -1
    assert P.lib.rlk_probe_device_info(ctypes.byref(i32), ctypes.byref(i32), ctypes.byref(i32),
                                       ctypes.byref(i32), ctypes.create_string_buffer(8), 0) == -1


def test_backend_and_status_strings(L):
    assert L.backend_id() == "rlk.logprob.strict.gfx950.v1"
    for st in range(5):
        assert L.status_string(st)
    assert L.status_string(99) == "unknown status"


def test_workspace_sizes(L):
    assert L.workspace_bytes(B.OP_FROM_LOGITS, 1024, 151936, 0, 1) == 0
    assert L.workspace_bytes(B.OP_FROM_LOGITS, 1024, 151936, 0, 4) == 4 * 1024 * 24
    assert L.workspace_bytes(B.OP_ENTROPY, 1024, 151936, 0, 8) == 8 * 1024 * 24
    # fused: 8 chunks x ceil(18992 / 256) = 600 tile states per token, + target logits
    lin = L.workspace_bytes(B.OP_LINEAR, 1024, 151936, 2048, 1)
    assert lin == 600 * 1024 * 24 + 4096
    lin4 = L.workspace_bytes(B.OP_LINEAR, 1024, 151936, 2048, 4)
    assert lin4 == lin + 4 * 1024 * 24
    assert L.workspace_bytes(B.OP_LINEAR, 0, 151936, 2048, 1) == 0
    bad = B.WORKSPACE_INVALID
    assert L.lib.rlk_workspace_bytes(7, 1, 1, 0, 1) == bad          # op code
    assert L.lib.rlk_workspace_bytes(0, 1, 1, 0, 3) == bad          # split count
    assert L.lib.rlk_workspace_bytes(0, -1, 1, 0, 1) == bad         # negative n_tokens
    assert L.lib.rlk_workspace_bytes(0, 1, 0, 0, 1) == bad          # empty vocabulary
    assert L.lib.rlk_workspace_bytes(1, 1, (1 << 26) + 1, 64, 1) == bad  # fused vocabulary
    assert L.lib.rlk_workspace_bytes(3, -1, 0, 0, 0) == bad         # compare: negative
    with pytest.raises(B.RlkError):
        L.workspace_bytes(B.OP_FROM_LOGITS, 1, 1, 0, 3)


def call_logits(L, logits=FAKE, ld=1024, T=4, V=1024, targets=FAKE, tau=1.0, S=1, lp=FAKE,
                ent=FAKE, ws=None, wsb=0):
    return L.logprob_from_logits_raw(logits, ld, T, V, targets, tau, S, lp, ent, ws, wsb, None)


def test_with_states_variants_validate_like_the_plain_calls(L):
    """The _with_states calls take the plain call's arguments plus the row-state output;
    a misaligned state pointer is rejected, and every plain-call error is returned alike."""
    f = L.lib.rlk_logprob_from_logits_with_states
    assert f(FAKE, 1024, 4, 1024, FAKE, 1.0, 1, FAKE, FAKE, FAKE + 4, None, 0, None) == \
        B.RLK_ERR_INVALID_ARGUMENT
    assert f(FAKE, 1000, 4, 1024, FAKE, 1.0, 1, FAKE, FAKE, FAKE, None, 0, None) == \
        B.RLK_ERR_INVALID_ARGUMENT
    assert f(FAKE, 1024, 4, 1024, FAKE, 1.0, 4, FAKE, FAKE, FAKE, None, 0, None) == \
        B.RLK_ERR_WORKSPACE_TOO_SMALL
    assert f(None, 1024, 0, 1024, None, 1.0, 1, None, None, None, None, 0, None) == B.RLK_OK
    g = L.lib.rlk_linear_logprob_with_states
    assert g(FAKE, 2048, FAKE, 2048, 4, 2048, 1000, FAKE, 1.0, 1, FAKE, None, FAKE + 4, FAKE,
             1 << 30, None) == B.RLK_ERR_INVALID_ARGUMENT
    assert g(FAKE, 2048, FAKE, 2048, 4, 2048, 1000, FAKE, 1.0, 1, FAKE, None, FAKE, FAKE, 100,
             None) == B.RLK_ERR_WORKSPACE_TOO_SMALL
    assert g(None, 2048, None, 2048, 0, 2048, 1000, None, 1.0, 1, None, None, None, None, 0,
             None) == B.RLK_OK


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(targets=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(lp=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(T=-1), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(V=0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ld=1000), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(tau=0.0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(tau=-1.0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(tau=math.inf), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(tau=math.nan), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=3), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=16), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=4), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(S=4, ws=FAKE, wsb=4 * 4 * 24 - 1), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(S=4, ws=FAKE + 8, wsb=4 * 4 * 24), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(T=0, logits=None, targets=None, lp=None), B.RLK_OK),
])
def test_logits_validation(L, kw, code):
    assert call_logits(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ld=1000), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(tau=0.0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=5), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=2), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(T=0, logits=None, targets=None, lp=None), B.RLK_OK),
])
def test_bf16_logits_validation(L, kw, code):
    a = dict(logits=FAKE, ld=1024, T=4, V=1024, targets=FAKE, tau=1.0, S=1, lp=FAKE, ent=FAKE,
             ws=None, wsb=0)
    a.update(kw)
    assert L.lib.rlk_logprob_from_logits_bf16(a["logits"], a["ld"], a["T"], a["V"], a["targets"],
                                              a["tau"], a["S"], a["lp"], a["ent"], a["ws"],
                                              a["wsb"], None) == code
    if kw.get("T") != 0 and "targets" not in kw:
        assert L.lib.rlk_entropy_bf16(a["logits"], a["ld"], a["T"], a["V"], a["tau"], a["S"],
                                      a["ent"], a["ws"], a["wsb"], None) == code


def test_entropy_validation(L):
    e = L.entropy_raw
    assert e(FAKE, 1024, 4, 1024, 1.0, 1, None, None, 0, None) == B.RLK_ERR_INVALID_ARGUMENT
    assert e(FAKE, 1024, 4, 1024, 1.0, 5, FAKE, None, 0, None) == B.RLK_ERR_INVALID_ARGUMENT
    assert e(FAKE, 1024, 4, 1024, 1.0, 2, FAKE, None, 0, None) == B.RLK_ERR_WORKSPACE_TOO_SMALL
    assert e(None, 1024, 0, 1024, 1.0, 1, None, None, 0, None) == B.RLK_OK


def test_compare_workspace_and_result_layout(L):
    assert L.workspace_bytes(B.OP_COMPARE, 0, 1) == 0
    assert L.workspace_bytes(B.OP_COMPARE, 1, 1) == 64
    assert L.workspace_bytes(B.OP_COMPARE, 4096, 1) == 64
    assert L.workspace_bytes(B.OP_COMPARE, 4097, 1) == 128
    assert L.workspace_bytes(B.OP_COMPARE, 16384, 0, 0, 3) == 4 * 64   # vocab/splits ignored
    raw = struct.pack("<4q4d", 7, 2, 3, 0, 0.5, 0.25, -0.125, 0.0625)
    assert B.unpack_compare(raw) == dict(active_tokens=7, mismatch_count=2,
                                         bitwise_mismatch_count=3, max_abs_diff=0.5,
                                         mean_abs_diff=0.25, mismatch_kl=-0.125,
                                         mismatch_k3_kl=0.0625)


@pytest.mark.parametrize("kw,code", [
    (dict(train=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(rollout=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(res=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(res=FAKE + 4), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(T=-1), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ws=None), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(wsb=127), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=FAKE + 64), B.RLK_ERR_INVALID_ARGUMENT),
])
def test_compare_validation(L, kw, code):
    a = dict(train=FAKE, rollout=FAKE, mask=None, T=5000, res=FAKE, ws=FAKE, wsb=128)
    a.update(kw)
    assert L.lib.rlk_logprob_compare(a["train"], a["rollout"], a["mask"], a["T"], a["res"],
                                     a["ws"], a["wsb"], None) == code


def test_backward_workspace(L):
    assert L.workspace_bytes(B.OP_BACKWARD_FROM_LOGITS, 0, 100, 0, 1) == 0
    assert L.workspace_bytes(B.OP_BACKWARD_FROM_LOGITS, 1024, 151936, 0, 1) == 1024 * 24
    assert L.workspace_bytes(B.OP_BACKWARD_FROM_LOGITS, 1024, 151936, 0, 4) == 4 * 1024 * 24 + 1024 * 24
    assert L.workspace_bytes(B.OP_BACKWARD_FROM_LOGITS, 10, 100, 0, 2) == 512 + 240


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(grad=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ld=1000), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ldg=1000), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(targets=None), B.RLK_ERR_INVALID_ARGUMENT),            # grad_logprob without targets
    (dict(grad=FAKE, ldg=1028), B.RLK_ERR_INVALID_ARGUMENT),       # in place with another ld
    (dict(tau=-1.0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=3), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ws=None), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(wsb=4 * 24 - 1), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=FAKE + 16), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(T=0, logits=None, grad=None, ws=None, wsb=0), B.RLK_OK),
    (dict(states=FAKE + 4), B.RLK_ERR_INVALID_ARGUMENT),             # misaligned row states
])
def test_backward_validation(L, kw, code):
    assert call_backward(L, **kw) == code


def call_backward(L, **kw):
    a = dict(logits=FAKE, ld=1024, T=4, V=1024, targets=FAKE, tau=1.0, S=1, glp=FAKE, gent=None,
             grad=FAKE + 0x100000, ldg=1024, ws=FAKE, wsb=4 * 24)
    a.update(kw)
    return L.lib.rlk_logprob_backward_from_logits(
        a["logits"], a["ld"], a["T"], a["V"], a["targets"], a["tau"], a["S"], a["glp"],
        a["gent"], a.get("states"), a["grad"], a["ldg"], a["ws"], a["wsb"], None)


def test_linear_backward_workspace_and_validation(L):
    T, V, d = 2048, 151936, 4096
    ws = L.workspace_bytes(B.OP_LINEAR_BACKWARD, T, V, d, 1)
    Vp, Tp = 151936, 2048
    fwd = L.workspace_bytes(B.OP_LINEAR, T, V, d, 1)
    # forward workspace, row states and constants, H^T, dX and dX^T in bf16, 4 dH partials
    # (one per fixed K range); W is read in place (no transposed copy)
    need = fwd + d * Tp * 2 + T * Vp * 2 + V * Tp * 2 + 4 * T * d * 4
    assert need <= ws <= need + (1 << 20)
    assert L.workspace_bytes(B.OP_LINEAR_BACKWARD, 0, V, d, 1) == 0
    # the backward runs in token chunks of 4096: its workspace stops growing there
    ws4k = L.workspace_bytes(B.OP_LINEAR_BACKWARD, 4096, V, d, 1)
    assert ws4k > ws
    for big in (4097, 8192, 16384, 1 << 20):
        assert L.workspace_bytes(B.OP_LINEAR_BACKWARD, big, V, d, 1) == ws4k, big
    with pytest.raises(B.RlkError):
        L.workspace_bytes(B.OP_LINEAR_BACKWARD, T, V, 100, 1)         # d not a multiple of 64
    call = lambda **kw: call_linear_backward(L, **kw)  # noqa: E731
    assert call(d=96) == B.RLK_ERR_INVALID_ARGUMENT
    assert call(lddh=1000) == B.RLK_ERR_INVALID_ARGUMENT
    assert call(lddw=1000) == B.RLK_ERR_INVALID_ARGUMENT
    assert call(tg=None) == B.RLK_ERR_INVALID_ARGUMENT
    assert call(h=FAKE + 2) == B.RLK_ERR_INVALID_ARGUMENT
    assert call(wsb=1000) == B.RLK_ERR_WORKSPACE_TOO_SMALL
    assert call(ws=FAKE + 64) == B.RLK_ERR_INVALID_ARGUMENT
    assert call(dh=None, dw=None) == B.RLK_OK                      # nothing requested
    assert call(T=0, h=None, w=None, ws=None, wsb=0, dh=None, dw=None) == B.RLK_OK
    assert call(states=FAKE + 4) == B.RLK_ERR_INVALID_ARGUMENT


def call_linear_backward(L, **kw):
    a = dict(h=FAKE, ldh=2048, w=FAKE, ldw=2048, T=4, d=2048, V=1000, tg=FAKE, tau=1.0, S=1,
             glp=FAKE, gent=None, dh=FAKE, lddh=2048, dw=FAKE, lddw=2048, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return L.lib.rlk_linear_logprob_backward(
        a["h"], a["ldh"], a["w"], a["ldw"], a["T"], a["d"], a["V"], a["tg"], a["tau"], a["S"],
        a["glp"], a["gent"], a.get("states"), a["dh"], a["lddh"], a["dw"], a["lddw"], a["ws"],
        a["wsb"], None)


def call_linear(L, h=FAKE, ldh=2048, w=FAKE, ldw=2048, T=4, d=2048, V=1000, tg=FAKE, tau=1.0,
                S=1, lp=FAKE, ent=None, ws=FAKE, wsb=1 << 30):
    return L.linear_logprob_raw(h, ldh, w, ldw, T, d, V, tg, tau, S, lp, ent, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(w=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(tg=None), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(d=100, ldh=100, ldw=100), B.RLK_ERR_INVALID_ARGUMENT),   # not a multiple of 64
    (dict(d=0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ldh=2040), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ldw=2052), B.RLK_ERR_INVALID_ARGUMENT),                   # not a multiple of 8
    (dict(ldw=(1 << 22) + 8), B.RLK_ERR_INVALID_ARGUMENT),           # stride too large
    (dict(V=(1 << 26) + 1), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(h=FAKE + 2), B.RLK_ERR_INVALID_ARGUMENT),                 # not 16-byte aligned
    (dict(tau=0.0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(S=6), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(V=0), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(ws=None), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(wsb=100), B.RLK_ERR_WORKSPACE_TOO_SMALL),
    (dict(ws=FAKE + 64), B.RLK_ERR_INVALID_ARGUMENT),
    (dict(T=0, h=None, w=None, tg=None, lp=None, ws=None, wsb=0), B.RLK_OK),
])
def test_linear_validation(L, kw, code):
    assert call_linear(L, **kw) == code


def test_noalloc_validates_and_bounds_its_scratch_on_the_host(L):
    """rlk_linear_logprob_noalloc checks its arguments as rlk_linear_logprob does, and rejects
    a call whose workspace would not fit its static scratch before touching any device."""
    f = L.lib.rlk_linear_logprob_noalloc
    V, d = 151936, 2048
    assert L.workspace_bytes(B.OP_LINEAR, 4659, V, d, 1) <= B.NOALLOC_SCRATCH_BYTES
    assert L.workspace_bytes(B.OP_LINEAR, 4660, V, d, 1) > B.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, d, FAKE, d, 4660, d, V, FAKE, 1.0, 1, FAKE, FAKE, None) == \
        B.RLK_ERR_WORKSPACE_TOO_SMALL
    assert f(FAKE, d, FAKE, d, 4600, d, V, FAKE, 1.0, 8, FAKE, FAKE, None) == \
        B.RLK_ERR_WORKSPACE_TOO_SMALL          # fits at split 1; 8 splits add 8 x 24 B per token
    assert f(FAKE, d, FAKE, d, 4, 100, V, FAKE, 1.0, 1, FAKE, FAKE, None) == \
        B.RLK_ERR_INVALID_ARGUMENT             # hidden_dim not a multiple of 64
    assert f(FAKE, d, FAKE, d, 4, d, V, None, 1.0, 1, FAKE, FAKE, None) == \
        B.RLK_ERR_INVALID_ARGUMENT             # no targets
    assert f(FAKE, d, FAKE, d, 4, d, V, FAKE, 0.0, 1, FAKE, FAKE, None) == \
        B.RLK_ERR_INVALID_ARGUMENT             # temperature
    assert f(FAKE + 2, d, FAKE, d, 4, d, V, FAKE, 1.0, 1, FAKE, FAKE, None) == \
        B.RLK_ERR_INVALID_ARGUMENT             # misaligned hidden
    assert f(None, d, None, d, 0, d, V, None, 1.0, 1, None, None, None) == B.RLK_OK


@pytest.mark.skipif(not no_gpu_visible(), reason="would launch on placeholder pointers")
def test_valid_call_without_gfx950_is_unsupported_device(L):
    """Arguments that pass validation reach the device check (run only where no GPU is
    visible: on a GPU these calls would launch on the placeholder pointers)."""
    cmp = L.lib.rlk_logprob_compare
    assert cmp(FAKE, FAKE, None, 5000, FAKE, FAKE, 128, None) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert cmp(None, None, None, 0, FAKE, None, 0, None) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_backward(L, targets=None, glp=None) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_backward(L, states=FAKE) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_backward(L) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_linear_backward(L) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_linear_backward(L, tg=None, glp=None, gent=FAKE) == B.RLK_ERR_UNSUPPORTED_DEVICE
    # an empty batch still writes its zero weight gradient
    assert call_linear_backward(L, T=0, h=None, w=None, ws=None, wsb=0) == \
        B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_logits(L) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert call_linear(L) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert L.lib.rlk_linear_logprob_noalloc(FAKE, 2048, FAKE, 2048, 4, 2048, 1000, FAKE, 1.0, 1,
                                            FAKE, None, None) == B.RLK_ERR_UNSUPPORTED_DEVICE
    assert L.entropy_raw(FAKE, 1024, 4, 1024, 1.0, 1, FAKE, None, 0, None) == \
        B.RLK_ERR_UNSUPPORTED_DEVICE
    assert L.lib.rlk_logprob_from_logits_bf16(FAKE, 1024, 4, 1024, FAKE, 1.0, 1, FAKE, None, None,
                                              0, None) == B.RLK_ERR_UNSUPPORTED_DEVICE
