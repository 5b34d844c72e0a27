"""The Python binding's argument checks (CPU only: every case is rejected before any call
into the library, so nothing is launched)."""
from __future__ import annotations

import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    from entropy_rlk_logprob_amd import binding
    return binding.load()


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def i64(*shape):
    return torch.zeros(*shape, dtype=torch.int64)


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("call", [
    lambda L: L.logprob_from_logits(torch.zeros(2, 3, dtype=torch.float64), i64(2)),
    lambda L: L.logprob_from_logits(f32(6), i64(2)),
    lambda L: L.logprob_from_logits(f32(3, 2).t(), i64(2)),
    lambda L: L.logprob_from_logits(f32(2, 3), torch.zeros(2, dtype=torch.int32)),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2)),                    # not on a GPU
    lambda L: L.entropy(torch.zeros(2, 3, dtype=torch.float16)),
    lambda L: L.linear_logprob(bf16(2, 64), bf16(5, 128), i64(2)),         # d differs
    lambda L: L.linear_logprob(f32(2, 64), bf16(5, 64), i64(2)),           # 4-byte hidden
    lambda L: L.logprob_backward_from_logits(f32(2, 3), i64(2), grad_logprob=f32(3)),
    lambda L: L.logprob_backward_from_logits(f32(2, 3), i64(2), out=f32(2, 4)),
    lambda L: L.linear_logprob_backward(bf16(2, 64), bf16(5, 64), i64(2),
                                        grad_entropy=torch.zeros(2, dtype=torch.float64)),
    lambda L: L.linear_logprob_backward(bf16(2, 64), bf16(5, 64), i64(2),
                                        out=(f32(2, 64), f32(4, 64))),
    lambda L: L.logprob_compare_async(f32(4), f32(5)),
    lambda L: L.logprob_compare_async(f32(4), f32(4), mask=f32(4)),
    # targets must hold exactly T ids
    lambda L: L.logprob_from_logits(f32(2, 3), i64(3)),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(1)),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2, 1)),
    lambda L: L.linear_logprob(bf16(2, 64), bf16(5, 64), i64(3)),
    lambda L: L.logprob_backward_from_logits(f32(2, 3), i64(1), grad_logprob=f32(2)),
    lambda L: L.linear_logprob_backward(bf16(2, 64), bf16(5, 64), i64(5), grad_logprob=f32(2)),
    # caller-given outputs: contiguous fp32 of shape (T,)
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2), out=(f32(3), f32(2))),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2), out=(f32(2), f32(1))),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2),
                                    out=(torch.zeros(2, dtype=torch.float64), None)),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2), out=(f32(4)[::2], None)),
    lambda L: L.logprob_from_logits(f32(2, 3), i64(2), out=(None, f32(2))),
    lambda L: L.linear_logprob(bf16(2, 64), bf16(5, 64), i64(2), out=(f32(2, 1), None)),
    lambda L: L.entropy(f32(2, 3), out=f32(3)),
    lambda L: L.logprob_compare_async(f32(4), f32(4), out=torch.zeros(63, dtype=torch.uint8)),
    # float16 is not bf16: its bits would be misread
    lambda L: L.linear_logprob(torch.zeros(2, 64, dtype=torch.float16), bf16(5, 64), i64(2)),
    lambda L: L.linear_logprob(bf16(2, 64), torch.zeros(5, 64, dtype=torch.float16), i64(2)),
    lambda L: L.linear_logprob_backward(torch.zeros(2, 64, dtype=torch.float16), bf16(5, 64),
                                        None, grad_entropy=f32(2)),
])
def test_bad_arguments_raise_before_any_launch(L, call):
    with pytest.raises(ValueError):
        call(L)
