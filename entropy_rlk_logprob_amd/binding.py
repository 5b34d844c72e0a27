"""Thin ctypes binding of librlk_logprob.so (include/rlk_logprob.h).

Argument marshalling only: torch tensors provide device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  There is no
fallback: if the library is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re
import struct

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "librlk_logprob.so")
HEADER = os.path.join(ROOT, "include", "rlk_logprob.h")
PROBES_PATH = os.path.join(PKG, "librlk_probes.so")
PROBES_HEADER = os.path.join(ROOT, "include", "rlk_probes.h")

RLK_OK = 0
RLK_ERR_INVALID_ARGUMENT = 1
RLK_ERR_UNSUPPORTED_DEVICE = 2
RLK_ERR_WORKSPACE_TOO_SMALL = 3
RLK_ERR_HIP = 4

OP_FROM_LOGITS, OP_LINEAR, OP_ENTROPY, OP_COMPARE, OP_BACKWARD_FROM_LOGITS = 0, 1, 2, 3, 4
OP_LINEAR_BACKWARD = 5
ROW_STATE_BYTES = 24   # sizeof(rlk_row_state)
WORKSPACE_INVALID = 2**64 - 1   # RLK_WORKSPACE_INVALID, (size_t)-1
NOALLOC_SCRATCH_BYTES = 64 << 20  # RLK_NOALLOC_SCRATCH_BYTES

# Field order of rlk_compare_result (8 x 8 bytes: four int64, then four double).
COMPARE_FIELDS = ("active_tokens", "mismatch_count", "bitwise_mismatch_count", "reserved",
                  "max_abs_diff", "mean_abs_diff", "mismatch_kl", "mismatch_k3_kl")


class RlkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _require(cond: bool, msg: str):
    """Argument check that survives `python -O` (unlike assert)."""
    if not cond:
        raise ValueError(msg)


def _same_device(device, *tensors):
    for t in tensors:
        if t is not None:
            _require(t.device == device, f"tensor on {t.device}, expected {device}")


_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p


def header_functions(header: str = HEADER) -> list[str]:
    """Names of the functions a header (default include/rlk_logprob.h) declares."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\*?\s*(rlk_[a-z0-9_]+)\s*\(",
                      text, flags=re.M)


class Library:
    """Loaded library with typed entry points."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run `python -m entropy_rlk_logprob_amd.build` "
                "(there is no fallback implementation)")
        self.path = path
        # torch ships its own HIP runtime under the same soname (libamdhip64.so.7); load it
        # first so this library binds to that one instance instead of pulling in a second
        # HIP runtime (with its own device state) from the system ROCm.
        import torch  # noqa: F401
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.rlk_workspace_bytes.restype = ctypes.c_size_t
        L.rlk_workspace_bytes.argtypes = [ctypes.c_int, _c_i64, _c_i64, _c_i64, ctypes.c_int32]
        L.rlk_logprob_from_logits.restype = ctypes.c_int
        L.rlk_logprob_from_logits.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_float,
                                              ctypes.c_int32, _c_p, _c_p, _c_p,
                                              ctypes.c_size_t, _c_p]
        L.rlk_logprob_from_logits_with_states.restype = ctypes.c_int
        L.rlk_logprob_from_logits_with_states.argtypes = [
            _c_p, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_float, ctypes.c_int32, _c_p, _c_p, _c_p,
            _c_p, ctypes.c_size_t, _c_p]
        L.rlk_linear_logprob.restype = ctypes.c_int
        L.rlk_linear_logprob.argtypes = [_c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p,
                                         ctypes.c_float, ctypes.c_int32, _c_p, _c_p, _c_p,
                                         ctypes.c_size_t, _c_p]
        L.rlk_linear_logprob_with_states.restype = ctypes.c_int
        L.rlk_linear_logprob_with_states.argtypes = [
            _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_float,
            ctypes.c_int32, _c_p, _c_p, _c_p, _c_p, ctypes.c_size_t, _c_p]
        L.rlk_linear_logprob_noalloc.restype = ctypes.c_int
        L.rlk_linear_logprob_noalloc.argtypes = [
            _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_float,
            ctypes.c_int32, _c_p, _c_p, _c_p]
        L.rlk_entropy.restype = ctypes.c_int
        L.rlk_entropy.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, ctypes.c_float, ctypes.c_int32,
                                  _c_p, _c_p, ctypes.c_size_t, _c_p]
        L.rlk_logprob_from_logits_bf16.restype = ctypes.c_int
        L.rlk_logprob_from_logits_bf16.argtypes = [_c_p, _c_i64, _c_i64, _c_i64, _c_p,
                                                   ctypes.c_float, ctypes.c_int32, _c_p, _c_p,
                                                   _c_p, ctypes.c_size_t, _c_p]
        L.rlk_entropy_bf16.restype = ctypes.c_int
        L.rlk_entropy_bf16.argtypes = L.rlk_entropy.argtypes
        L.rlk_logprob_compare.restype = ctypes.c_int
        L.rlk_logprob_compare.argtypes = [_c_p, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                          ctypes.c_size_t, _c_p]
        L.rlk_logprob_backward_from_logits.restype = ctypes.c_int
        L.rlk_logprob_backward_from_logits.argtypes = [
            _c_p, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_float, ctypes.c_int32, _c_p, _c_p, _c_p,
            _c_p, _c_i64, _c_p, ctypes.c_size_t, _c_p]
        L.rlk_linear_logprob_backward.restype = ctypes.c_int
        L.rlk_linear_logprob_backward.argtypes = [
            _c_p, _c_i64, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_float,
            ctypes.c_int32, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_i64, _c_p, ctypes.c_size_t,
            _c_p]
        L.rlk_status_string.restype = ctypes.c_char_p
        L.rlk_status_string.argtypes = [ctypes.c_int]
        L.rlk_backend_id.restype = ctypes.c_char_p
        L.rlk_backend_id.argtypes = []

    # ------------------------------------------------------------------ raw C calls
    def status_string(self, status: int) -> str:
        return self.lib.rlk_status_string(status).decode()

    def backend_id(self) -> str:
        return self.lib.rlk_backend_id().decode()

    def check(self, status: int, what: str):
        if status != RLK_OK:
            raise RlkError(status, f"{what}: {self.status_string(status)}")

    def workspace_bytes(self, op: int, n_tokens: int, vocab: int, hidden: int = 0,
                        vocab_splits: int = 1) -> int:
        n = self.lib.rlk_workspace_bytes(op, n_tokens, vocab, hidden, vocab_splits)
        if n == WORKSPACE_INVALID:
            raise RlkError(RLK_ERR_INVALID_ARGUMENT,
                           f"rlk_workspace_bytes(op={op}, n_tokens={n_tokens}, vocab={vocab}, "
                           f"hidden={hidden}, vocab_splits={vocab_splits}): invalid request")
        return n

    def logprob_from_logits_raw(self, *args) -> int:
        return self.lib.rlk_logprob_from_logits(*args)

    def linear_logprob_raw(self, *args) -> int:
        return self.lib.rlk_linear_logprob(*args)

    def entropy_raw(self, *args) -> int:
        return self.lib.rlk_entropy(*args)

    # ------------------------------------------------------------------ torch wrappers
    # Every wrapper makes the tensors' GPU current and the launch stream torch's current
    # stream while it allocates outputs and workspace (so the caching allocator orders the
    # reuse of that memory after the library's kernels on that stream), then passes the
    # stream's handle to the library.

    @staticmethod
    @contextlib.contextmanager
    def _on(device, stream=None):
        """Yield the stream to launch on, with `device` current and that stream current."""
        import torch
        _require(device.type == "cuda", f"tensors must be on a GPU, got {device}")
        with torch.cuda.device(device):
            s = stream if stream is not None else torch.cuda.current_stream(device)
            with torch.cuda.stream(s):
                yield s

    @staticmethod
    def _workspace(nbytes: int, device, workspace=None):
        import torch
        if nbytes == 0:
            return None, 0
        if workspace is not None:
            _require(workspace.is_contiguous(), "workspace must be contiguous")
            if workspace.numel() * workspace.element_size() < nbytes:
                raise RlkError(RLK_ERR_WORKSPACE_TOO_SMALL, "workspace tensor too small")
            return workspace, workspace.numel() * workspace.element_size()
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return ws, nbytes

    @staticmethod
    def row_states_buffer(n_tokens: int, device="cuda"):
        """Storage for n_tokens rlk_row_state records (24 bytes each)."""
        import torch
        return torch.empty(max(1, n_tokens) * ROW_STATE_BYTES, dtype=torch.uint8, device=device)

    @staticmethod
    def _check_states(states, T: int):
        if states is not None:
            _require(states.is_contiguous() and
                     states.numel() * states.element_size() >= T * ROW_STATE_BYTES,
                     f"row_states must be contiguous with room for {T} x {ROW_STATE_BYTES} bytes")
            _require(states.data_ptr() % 8 == 0, "row_states must be 8-byte aligned")

    @staticmethod
    def _check_targets(targets, T: int):
        import torch
        _require(targets.dtype == torch.int64 and targets.is_contiguous() and
                 targets.dim() == 1 and targets.numel() == T,
                 f"targets must be a contiguous int64 tensor of {T} elements")

    @staticmethod
    def _check_vec_out(t, T: int, what: str):
        import torch
        if t is not None:
            _require(t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (T,),
                     f"{what} must be a contiguous fp32 tensor of shape ({T},)")

    @staticmethod
    def _ptr(t) -> int | None:
        return None if t is None else t.data_ptr()

    def _vec_outputs(self, out, T: int, dev, with_entropy: bool):
        import torch
        if out is None:
            return (torch.empty(T, dtype=torch.float32, device=dev),
                    torch.empty(T, dtype=torch.float32, device=dev) if with_entropy else None)
        _require(isinstance(out, (tuple, list)) and len(out) == 2, "out must be (logprob, entropy)")
        lp, ent = out
        _require(lp is not None, "out[0] (logprob) is required")
        self._check_vec_out(lp, T, "out[0] (logprob)")
        self._check_vec_out(ent, T, "out[1] (entropy)")
        return lp, ent

    def logprob_from_logits(self, logits, targets, temperature: float = 1.0,
                            vocab_splits: int = 1, with_entropy: bool = True, out=None,
                            workspace=None, stream=None, row_states=None):
        """logits: [T, >=V] float32 or bfloat16 CUDA tensor (row stride = ld);
        targets: [T] int64; row_states: optional [T * 24] uint8 tensor (fp32 logits only)
        that receives the rows' states for the backward call."""
        import torch
        _require(logits.dtype in (torch.float32, torch.bfloat16), "logits must be fp32 or bf16")
        _require(logits.dim() == 2 and logits.stride(1) == 1, "logits must be [T, V], unit stride")
        T, V = logits.shape
        dev = logits.device
        self._check_targets(targets, T)
        lp, ent = (None, None) if out is None else self._vec_outputs(out, T, dev, with_entropy)
        _same_device(dev, targets, lp, ent, row_states, workspace)
        self._check_states(row_states, T)
        _require(row_states is None or logits.dtype == torch.float32,
                 "row states are saved by the fp32 logits call only")
        with self._on(dev, stream) as s:
            if out is None:
                lp, ent = self._vec_outputs(None, T, dev, with_entropy)
            ws, wsb = self._workspace(self.workspace_bytes(OP_FROM_LOGITS, T, V, 0, vocab_splits),
                                      dev, workspace)
            args = (self._ptr(logits), logits.stride(0), T, V, self._ptr(targets), temperature,
                    vocab_splits, self._ptr(lp), self._ptr(ent))
            tail = (self._ptr(ws), wsb, s.cuda_stream)
            if logits.dtype == torch.bfloat16:
                st = self.lib.rlk_logprob_from_logits_bf16(*args, *tail)
            elif row_states is None:
                st = self.lib.rlk_logprob_from_logits(*args, *tail)
            else:
                st = self.lib.rlk_logprob_from_logits_with_states(*args, self._ptr(row_states),
                                                                  *tail)
        self.check(st, "rlk_logprob_from_logits")
        return lp, ent

    def entropy(self, logits, temperature: float = 1.0, vocab_splits: int = 1, out=None,
                workspace=None, stream=None):
        import torch
        _require(logits.dtype in (torch.float32, torch.bfloat16), "logits must be fp32 or bf16")
        _require(logits.dim() == 2 and logits.stride(1) == 1, "logits must be [T, V], unit stride")
        T, V = logits.shape
        dev = logits.device
        self._check_vec_out(out, T, "out (entropy)")
        _same_device(dev, out, workspace)
        with self._on(dev, stream) as s:
            ent = out if out is not None else torch.empty(T, dtype=torch.float32, device=dev)
            ws, wsb = self._workspace(self.workspace_bytes(OP_ENTROPY, T, V, 0, vocab_splits),
                                      dev, workspace)
            fn = (self.lib.rlk_entropy if logits.dtype == torch.float32
                  else self.lib.rlk_entropy_bf16)
            st = fn(self._ptr(logits), logits.stride(0), T, V, temperature, vocab_splits,
                    self._ptr(ent), self._ptr(ws), wsb, s.cuda_stream)
        self.check(st, "rlk_entropy")
        return ent

    def linear_logprob(self, hidden, weight, targets, temperature: float = 1.0,
                       vocab_splits: int = 1, with_entropy: bool = True, out=None,
                       workspace=None, stream=None, row_states=None):
        """hidden: [T, d] bf16 (or int16/uint16 bits); weight: [V, d] same; targets [T] int64."""
        self._check_operands(hidden, weight)
        T, d = hidden.shape
        V = weight.shape[0]
        dev = hidden.device
        self._check_targets(targets, T)
        lp, ent = (None, None) if out is None else self._vec_outputs(out, T, dev, with_entropy)
        _same_device(dev, weight, targets, lp, ent, row_states, workspace)
        self._check_states(row_states, T)
        with self._on(dev, stream) as s:
            if out is None:
                lp, ent = self._vec_outputs(None, T, dev, with_entropy)
            ws, wsb = self._workspace(self.workspace_bytes(OP_LINEAR, T, V, d, vocab_splits), dev,
                                      workspace)
            args = (self._ptr(hidden), hidden.stride(0), self._ptr(weight), weight.stride(0), T,
                    d, V, self._ptr(targets), temperature, vocab_splits, self._ptr(lp),
                    self._ptr(ent))
            tail = (self._ptr(ws), wsb, s.cuda_stream)
            if row_states is None:
                st = self.lib.rlk_linear_logprob(*args, *tail)
            else:
                st = self.lib.rlk_linear_logprob_with_states(*args, self._ptr(row_states), *tail)
        self.check(st, "rlk_linear_logprob")
        return lp, ent

    def linear_logprob_noalloc(self, hidden, weight, targets, temperature: float = 1.0,
                               vocab_splits: int = 1, with_entropy: bool = True, out=None,
                               stream=None):
        """rlk_linear_logprob_noalloc: the fused call on the library's static device scratch
        (no workspace; the library allocates nothing).  Outputs are allocated here unless
        `out` is given.  Calls that overlap on one GPU share its scratch and must not run
        concurrently."""
        self._check_operands(hidden, weight)
        T, d = hidden.shape
        V = weight.shape[0]
        dev = hidden.device
        self._check_targets(targets, T)
        lp, ent = (None, None) if out is None else self._vec_outputs(out, T, dev, with_entropy)
        _same_device(dev, weight, targets, lp, ent)
        with self._on(dev, stream) as s:
            if out is None:
                lp, ent = self._vec_outputs(None, T, dev, with_entropy)
            st = self.lib.rlk_linear_logprob_noalloc(
                self._ptr(hidden), hidden.stride(0), self._ptr(weight), weight.stride(0), T, d,
                V, self._ptr(targets), temperature, vocab_splits, self._ptr(lp), self._ptr(ent),
                s.cuda_stream)
        self.check(st, "rlk_linear_logprob_noalloc")
        return lp, ent

    @staticmethod
    def _check_operands(hidden, weight):
        import torch
        bits16 = (torch.bfloat16, torch.int16, torch.uint16)
        _require(hidden.dim() == 2 and weight.dim() == 2, "hidden and weight must be 2-D")
        _require(hidden.dtype in bits16 and weight.dtype in bits16,
                 "hidden and weight must be bfloat16 (or int16 / uint16 holding bf16 bits)")
        _require(hidden.stride(1) == 1 and weight.stride(1) == 1,
                 "hidden and weight must have unit column stride")
        _require(hidden.shape[1] == weight.shape[1], "hidden and weight disagree on hidden_dim")

    @staticmethod
    def _check_row_grads(T: int, *grads):
        import torch
        for g in grads:
            _require(g is None or (g.dtype == torch.float32 and tuple(g.shape) == (T,) and
                                   g.is_contiguous()),
                     "upstream gradients must be contiguous fp32 [T]")

    def logprob_backward_from_logits(self, logits, targets, temperature: float = 1.0,
                                     vocab_splits: int = 1, grad_logprob=None, grad_entropy=None,
                                     out=None, workspace=None, stream=None, row_states=None):
        """Gradient of sum g_lp * logprob + g_ent * entropy w.r.t. fp32 logits [T, >=V];
        returns `out` (new [T, V] fp32 tensor if None; may be `logits` itself)."""
        import torch
        _require(logits.dtype == torch.float32 and logits.dim() == 2 and logits.stride(1) == 1,
                 "logits must be fp32 [T, V] with unit column stride")
        T, V = logits.shape
        dev = logits.device
        self._check_row_grads(T, grad_logprob, grad_entropy)
        if targets is not None:
            self._check_targets(targets, T)
        if out is not None:
            _require(out.dtype == torch.float32 and out.dim() == 2 and out.stride(1) == 1 and
                     tuple(out.shape) == (T, V),
                     "out must be fp32 [T, V] with unit column stride")
        _same_device(dev, targets, grad_logprob, grad_entropy, out, row_states, workspace)
        self._check_states(row_states, T)
        with self._on(dev, stream) as s:
            grad = out if out is not None else torch.empty((T, V), dtype=torch.float32,
                                                           device=dev)
            ws, wsb = self._workspace(self.workspace_bytes(OP_BACKWARD_FROM_LOGITS, T, V, 0,
                                                           vocab_splits), dev, workspace)
            st = self.lib.rlk_logprob_backward_from_logits(
                self._ptr(logits), logits.stride(0), T, V, self._ptr(targets), temperature,
                vocab_splits, self._ptr(grad_logprob), self._ptr(grad_entropy),
                self._ptr(row_states), self._ptr(grad), grad.stride(0), self._ptr(ws), wsb,
                s.cuda_stream)
        self.check(st, "rlk_logprob_backward_from_logits")
        return grad

    def linear_logprob_backward(self, hidden, weight, targets, temperature: float = 1.0,
                                vocab_splits: int = 1, grad_logprob=None, grad_entropy=None,
                                need_hidden: bool = True, need_weight: bool = True, out=None,
                                workspace=None, stream=None, row_states=None):
        """Gradients (dH [T, d], dW [V, d], fp32; None where not requested) of
        sum g_lp * logprob + g_ent * entropy for logits = hidden @ weight^T (bf16 bits)."""
        import torch
        self._check_operands(hidden, weight)
        T, d = hidden.shape
        V = weight.shape[0]
        dev = hidden.device
        self._check_row_grads(T, grad_logprob, grad_entropy)
        if targets is not None:
            self._check_targets(targets, T)
        dh, dw = out if out is not None else (None, None)
        for g, shape in ((dh, (T, d)), (dw, (V, d))):
            _require(g is None or (g.dtype == torch.float32 and g.dim() == 2 and
                                   tuple(g.shape) == shape and g.stride(1) == 1),
                     f"gradient outputs must be fp32 {shape} with unit column stride")
        _same_device(dev, weight, targets, grad_logprob, grad_entropy, row_states, dh, dw,
                     workspace)
        self._check_states(row_states, T)
        with self._on(dev, stream) as s:
            if out is None:
                dh = torch.empty((T, d), dtype=torch.float32, device=dev) if need_hidden else None
                dw = torch.empty((V, d), dtype=torch.float32, device=dev) if need_weight else None
            ws, wsb = self._workspace(self.workspace_bytes(OP_LINEAR_BACKWARD, T, V, d,
                                                           vocab_splits), dev, workspace)
            st = self.lib.rlk_linear_logprob_backward(
                self._ptr(hidden), hidden.stride(0), self._ptr(weight), weight.stride(0), T, d,
                V, self._ptr(targets), temperature, vocab_splits, self._ptr(grad_logprob),
                self._ptr(grad_entropy), self._ptr(row_states), self._ptr(dh),
                dh.stride(0) if dh is not None else 0,
                self._ptr(dw), dw.stride(0) if dw is not None else 0, self._ptr(ws), wsb,
                s.cuda_stream)
        self.check(st, "rlk_linear_logprob_backward")
        return dh, dw

    def logprob_compare_async(self, train, rollout, mask=None, out=None, workspace=None,
                              stream=None):
        """Launch rlk_logprob_compare; returns the 64-byte device result tensor (uint8)."""
        import torch
        _require(train.dtype == torch.float32 and rollout.dtype == torch.float32,
                 "logprobs must be fp32")
        _require(train.dim() == 1 and train.shape == rollout.shape, "logprobs must be [T] alike")
        _require(train.is_contiguous() and rollout.is_contiguous(), "logprobs must be contiguous")
        if mask is not None:
            _require(mask.dtype in (torch.uint8, torch.bool) and mask.shape == train.shape and
                     mask.is_contiguous(), "mask must be a contiguous [T] bool or uint8 tensor")
        if out is not None:
            _require(out.numel() * out.element_size() >= 64 and out.is_contiguous() and
                     out.data_ptr() % 8 == 0, "out must hold 64 contiguous, 8-aligned bytes")
        T = train.shape[0]
        dev = train.device
        _same_device(dev, rollout, mask, out, workspace)
        with self._on(dev, stream) as s:
            res = out if out is not None else torch.empty(64, dtype=torch.uint8, device=dev)
            ws, wsb = self._workspace(self.workspace_bytes(OP_COMPARE, T, 1), dev, workspace)
            st = self.lib.rlk_logprob_compare(self._ptr(train), self._ptr(rollout),
                                              self._ptr(mask), T, self._ptr(res), self._ptr(ws),
                                              wsb, s.cuda_stream)
        self.check(st, "rlk_logprob_compare")
        return res

    def logprob_compare(self, train, rollout, mask=None, workspace=None, stream=None) -> dict:
        """Comparison metrics as a dict (copies the 64-byte result to the host once the
        launch stream has written it)."""
        import torch
        res = self.logprob_compare_async(train, rollout, mask, None, workspace, stream)
        if stream is not None:
            stream.synchronize()
        else:
            torch.cuda.current_stream(train.device).synchronize()
        return unpack_compare(bytes(res.cpu().numpy().tobytes()))


_LIB: Library | None = None


def unpack_compare(raw: bytes) -> dict:
    """rlk_compare_result bytes -> dict (the reserved field dropped)."""
    ints = struct.unpack("<4q", raw[:32])
    dbls = struct.unpack("<4d", raw[32:64])
    out = dict(zip(COMPARE_FIELDS, ints + dbls))
    del out["reserved"]
    return out


def load(path: str = LIB_PATH) -> Library:
    """Load (once) and return the library; raises if it is not built."""
    global _LIB
    if _LIB is None or _LIB.path != path:
        _LIB = Library(path)
    return _LIB


class Probes:
    """The measurement probes of include/rlk_probes.h (librlk_probes.so), for bench.py."""

    READ_BLOCKS, THREADS = 2048, 256

    def __init__(self, path: str = PROBES_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m entropy_rlk_logprob_amd.build`")
        import torch  # noqa: F401  (bind to torch's HIP runtime first, as Library does)
        self.lib = ctypes.CDLL(path)
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        self.lib.rlk_probe_stream_read.argtypes = [vp, sz, vp, vp]
        self.lib.rlk_probe_stream_read.restype = ctypes.c_int
        self.lib.rlk_probe_mfma.argtypes = [i32, i32, u32, vp, vp]
        self.lib.rlk_probe_mfma.restype = ctypes.c_int
        pi32 = ctypes.POINTER(ctypes.c_int32)
        self.lib.rlk_probe_device_info.argtypes = [pi32, pi32, pi32, pi32, ctypes.c_char_p, sz]
        self.lib.rlk_probe_device_info.restype = ctypes.c_int

    @staticmethod
    def _stream(dev):
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def stream_read(self, buf, sink):
        """Reads all bytes of the contiguous CUDA tensor `buf`; sink: >= 2048 * 256 floats."""
        _require(buf.is_contiguous() and buf.is_cuda, "buf must be a contiguous CUDA tensor")
        _require(sink.numel() >= self.READ_BLOCKS * self.THREADS, "sink too small")
        nbytes = buf.numel() * buf.element_size()
        st = self.lib.rlk_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                            ctypes.c_void_p(sink.data_ptr()),
                                            self._stream(buf.device))
        if st != 0:
            raise RuntimeError(f"rlk_probe_stream_read failed ({st})")
        return nbytes

    def device_info(self) -> dict:
        """rlk_probe_device_info of the current device, with the dense bf16 MFMA peak it implies
        (compute units x engine clock x 4096 flop per clock)."""
        cu, clk, mclk, bus = (ctypes.c_int32() for _ in range(4))
        arch = ctypes.create_string_buffer(64)
        st = self.lib.rlk_probe_device_info(ctypes.byref(cu), ctypes.byref(clk), ctypes.byref(mclk),
                                            ctypes.byref(bus), arch, len(arch))
        if st != 0:
            raise RuntimeError(f"rlk_probe_device_info failed ({st})")
        return {"arch": arch.value.decode(), "compute_units": cu.value,
                "engine_clock_mhz": clk.value / 1e3, "memory_clock_mhz": mclk.value / 1e3,
                "memory_bus_bits": bus.value,
                "mfma_bf16_dense_peak_tflops": round(cu.value * clk.value * 1e3 * 4096 / 1e12, 1)}

    def mfma(self, blocks: int, iters: int, sink, seed: int = 1):
        """Returns the flops of one launch; sink: >= blocks * 256 floats."""
        _require(sink.numel() >= blocks * self.THREADS, "sink too small")
        st = self.lib.rlk_probe_mfma(blocks, iters, seed, ctypes.c_void_p(sink.data_ptr()),
                                     self._stream(sink.device))
        if st != 0:
            raise RuntimeError(f"rlk_probe_mfma failed ({st})")
        return blocks * 4 * iters * 8 * 32768.0


def load_probes(path: str = PROBES_PATH) -> Probes:
    return Probes(path)
