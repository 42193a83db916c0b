"""Route torch's own ops to the batch-invariant kernels.

The pages present the batch-invariant kernels as a drop-in replacement for
PyTorch's mm, addmm, log_softmax and mean, switched on around ordinary model
code ("thinking-machines-lab/batch_invariant_ops" catalogue page, section
"What it is"; "Batch-invariant inference kernels (Thinking Machines) --
Evidence & limits", section "Evidence", on SGLang using the mean,
log-softmax and matmul kernels). This module is that switch for this
library:

    with batch_invariant_mode():
        logits = model(tokens)          # unchanged model code

Inside the mode, on CUDA tensors:

* ``aten.mm`` / ``aten.mm.dtype`` (bf16 x bf16) -> ``bi_mm``
* ``aten.addmm`` (bf16 x bf16, bias a [N] vector) -> ``bi_addmm``
* ``aten._log_softmax`` (fp32, last dim) -> ``bi_log_softmax``
* ``aten.mean.dim`` (bf16/fp32, last dim) -> ``bi_mean``
* ``torch.nn.functional.rms_norm`` (bf16, last dim, bf16 weight) ->
  ``bi_rmsnorm``. That function decomposes above the dispatcher, so the
  mode swaps it for the duration of the ``with`` block.

``F.linear`` and ``@`` on 2-D or batched-as-2-D inputs reach the dispatcher
as ``mm``/``addmm`` with the weight as a transposed view of a row-major
[N, K] matrix; that is passed as the library's [N, K] layout (``b_is_nk``),
without a copy.

Every routed call is argument marshalling: outputs are allocated with torch
and the kernels run on the current stream. Where torch's result dtype is
bf16 and the kernel's fp32 (mean), the fp32 result is rounded once with
torch's own cast, which is elementwise and so cannot depend on the batch.

A routed op whose operands fall outside what the kernels take (another
dtype, a reduction over another dim, a misaligned stride) raises
``BiUnsupported`` under ``strict=True`` (the default) -- silently running
torch's kernel would silently lose the invariance the caller asked for.
With ``strict=False`` such calls run torch's own kernel and are counted in
``mode.passthrough``. Ops the library does not cover at all, and CPU
tensors, always run torch's kernels.
"""
from __future__ import annotations

import collections
import contextlib

import torch
import torch.nn.functional as F
from torch.utils._python_dispatch import TorchDispatchMode

from . import bi_addmm, bi_log_softmax, bi_mean, bi_mm, bi_rmsnorm

__all__ = ["BatchInvariantMode", "BiUnsupported", "batch_invariant_mode", "gemm_operands"]

aten = torch.ops.aten


class BiUnsupported(RuntimeError):
    """An op the mode routes was called with operands the kernels do not take."""


def _aligned(t: torch.Tensor, nbytes: int = 16) -> bool:
    return t.data_ptr() % nbytes == 0


def _rows(t: torch.Tensor, quantum: int):
    """Row-major [M, N] view of t with unit inner stride, or None.

    quantum: the row stride must be a multiple of this many elements (a
    single row is exempt: its stride is never used)."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.size(1) > 1):
        return None
    if t.size(0) > 1 and t.stride(0) % quantum != 0:
        return None
    if not _aligned(t):
        return None
    return t


def gemm_operands(a: torch.Tensor, b: torch.Tensor):
    """(a, b, b_is_nk) in the forms bi_mm takes for torch's a @ b, or a reason string.

    b [K, N] row-major -> b_is_nk False; b a transposed view of a row-major
    [N, K] matrix (nn.Linear's weight.t()) -> b.t() with b_is_nk True."""
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        return f"dtypes {a.dtype} x {b.dtype} (bf16 x bf16 only)"
    if a.dim() != 2 or b.dim() != 2:
        return "operands must be 2-D"
    k = a.shape[1]
    if k % 8 != 0:
        return f"K = {k} is not a multiple of 8"
    if _rows(a, 8) is None:
        return "a is not row-major with a 16-byte aligned base and a row stride multiple of 8"
    if _rows(b, 8) is not None and b.shape[1] % 8 == 0:
        return a, b, False
    bt = b.t()
    if _rows(bt, 8) is not None:
        return a, bt, True
    return "b is neither row-major [K, N] (N a multiple of 8) nor the transpose of a row-major [N, K]"


class BatchInvariantMode(TorchDispatchMode):
    """Dispatch mode that sends the covered aten ops to the invariant kernels."""

    def __init__(self, strict: bool = True):
        super().__init__()
        self.strict = strict
        self.routed = collections.Counter()
        self.passthrough = collections.Counter()
        self._rms_norm_saved = None

    # --- entering / leaving: rms_norm is swapped at the functional level
    def __enter__(self):
        self._rms_norm_saved = F.rms_norm
        F.rms_norm = self._rms_norm
        return super().__enter__()

    def __exit__(self, *exc):
        F.rms_norm = self._rms_norm_saved
        return super().__exit__(*exc)

    def _refuse(self, op: str, why: str, fallback):
        if self.strict:
            raise BiUnsupported(f"{op}: {why}")
        self.passthrough[op] += 1
        return fallback()

    def _rms_norm(self, input, normalized_shape, weight=None, eps=None):
        fallback = lambda: self._rms_norm_saved(input, normalized_shape, weight, eps)  # noqa: E731
        if not input.is_cuda:
            return fallback()
        n = input.shape[-1]
        why = None
        if tuple(normalized_shape) != (n,):
            why = "normalisation over more than the last dim"
        elif input.dtype != torch.bfloat16 or weight is None or weight.dtype != torch.bfloat16:
            why = "bf16 input with a bf16 weight only"
        elif n % 8 != 0:
            why = f"width {n} is not a multiple of 8"
        if why is None:
            x = input.reshape(-1, n)
            w = weight.contiguous()
            if _rows(x, 8) is None or not _aligned(w):
                why = "input rows not contiguous and 16-byte aligned"
        if why is not None:
            return self._refuse("rms_norm", why, fallback)
        self.routed["rms_norm"] += 1
        e = torch.finfo(input.dtype).eps if eps is None else float(eps)  # torch's default
        return bi_rmsnorm(x, w, e, out_dtype=torch.bfloat16).view(input.shape)

    def __torch_dispatch__(self, func, types, args=(), kwargs=None):
        kwargs = kwargs or {}
        run = lambda: func(*args, **kwargs)  # noqa: E731
        if func in (aten.mm.default, aten.mm.dtype):
            a, b = args[0], args[1]
            if not a.is_cuda:
                return run()
            out_dtype = kwargs.get("out_dtype", args[2] if len(args) > 2 else None) if func is aten.mm.dtype else None
            if out_dtype is None:
                out_dtype = torch.bfloat16
            ops = gemm_operands(a, b)
            if isinstance(ops, str) or out_dtype not in (torch.bfloat16, torch.float32):
                return self._refuse("mm", ops if isinstance(ops, str) else f"out_dtype {out_dtype}", run)
            self.routed["mm"] += 1
            a2, b2, nk = ops
            return bi_mm(a2, b2, b_is_nk=nk, out_dtype=out_dtype)

        if func is aten.addmm.default:
            bias, a, b = args[0], args[1], args[2]
            if not a.is_cuda:
                return run()
            beta = kwargs.get("beta", args[3] if len(args) > 3 else 1)
            alpha = kwargs.get("alpha", args[4] if len(args) > 4 else 1)
            ops = gemm_operands(a, b)
            why = ops if isinstance(ops, str) else None
            if why is None:
                n = ops[1].shape[0] if ops[2] else ops[1].shape[1]
                if bias.dim() == 2 and bias.shape[0] == 1:
                    bias = bias[0]
                if bias.dim() != 1 or bias.shape[0] != n or bias.dtype not in (torch.bfloat16, torch.float32):
                    why = "bias must be a bf16/fp32 [N] vector (broadcast over rows)"
                else:
                    bias = bias.contiguous()
                    if not _aligned(bias, bias.element_size()):
                        why = "bias misaligned"
            if why is not None:
                return self._refuse("addmm", why, run)
            self.routed["addmm"] += 1
            a2, b2, nk = ops
            return bi_addmm(bias, a2, b2, beta=float(beta), alpha=float(alpha), b_is_nk=nk, out_dtype=torch.bfloat16)

        if func is aten._log_softmax.default:
            x, dim, half_to_float = args[0], args[1], args[2]
            if not x.is_cuda:
                return run()
            why = None
            if x.dtype != torch.float32 or half_to_float:
                why = "fp32 input and output only"
            elif x.dim() == 0 or dim % x.dim() != x.dim() - 1:
                why = "over the last dim only"
            elif x.shape[-1] % 4 != 0:
                why = f"width {x.shape[-1]} is not a multiple of 4"
            else:
                x2 = x.reshape(-1, x.shape[-1])
                if _rows(x2, 4) is None:
                    why = "rows not contiguous and 16-byte aligned"
            if why is not None:
                return self._refuse("log_softmax", why, run)
            self.routed["log_softmax"] += 1
            y, _ = bi_log_softmax(x2, want_argmax=False)
            return y.view(x.shape)

        if func is aten.mean.dim:
            x, dims = args[0], args[1]
            if not x.is_cuda:
                return run()
            keepdim = kwargs.get("keepdim", args[2] if len(args) > 2 else False)
            dtype = kwargs.get("dtype", args[3] if len(args) > 3 else None)
            why = None
            if x.dtype not in (torch.bfloat16, torch.float32) or dtype not in (None, x.dtype):
                why = "bf16/fp32 input with its own result dtype only"
            elif x.dim() == 0 or dims is None or len(dims) != 1 or dims[0] % x.dim() != x.dim() - 1:
                why = "over the last dim only"
            else:
                q = 8 if x.dtype == torch.bfloat16 else 4
                x2 = x.reshape(-1, x.shape[-1])
                if x.shape[-1] % q != 0 or _rows(x2, q) is None:
                    why = "rows not contiguous, 16-byte aligned, with a width multiple of 16 bytes"
            if why is not None:
                return self._refuse("mean", why, run)
            self.routed["mean"] += 1
            y = bi_mean(x2)
            if x.dtype != torch.float32:
                y = y.to(x.dtype)
            shape = list(x.shape[:-1]) + ([1] if keepdim else [])
            return y.view(shape)

        return run()


@contextlib.contextmanager
def batch_invariant_mode(strict: bool = True):
    """Context manager: inside it the covered torch ops run the invariant kernels."""
    mode = BatchInvariantMode(strict=strict)
    with mode:
        yield mode
