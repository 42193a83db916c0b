"""Python binding for libbi.so, the batch-invariant kernel library (gfx950).

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in ``include/bi.h``; PyTorch supplies device memory and the
current stream. The functions carry the C names (``bi_mm``, ``bi_addmm``,
...). There is no fallback: if ``libbi.so`` is missing or cannot be loaded,
importing this package raises ``ImportError``.

The library links ``libamdhip64.so.7``. torch is imported first so that
name resolves to the HIP runtime torch has already loaded (same soname):
the ``hipStream_t`` handles torch hands out are only meaningful inside that
runtime instance.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded before libbi.so, see above)

__all__ = [
    "BiError", "LIB_PATH", "lib",
    "bi_mm", "bi_addmm", "bi_gemm", "bi_gemm_config", "bi_gemm_plan", "BI_GEMM_FIXED_TILE", "bi_rmsnorm", "bi_mean", "bi_log_softmax",
    "bi_decode_plan", "bi_decode_workspace_bytes", "bi_decode_attention", "bi_decode_attention_noalloc",
    "BI_DECODE_NOALLOC_MAX_BYTES",
    "bi_add_rmsnorm", "bi_embed", "bi_silu_mul", "bi_qknorm_rope_append",
    "bi_prefill_plan", "bi_prefill_attention", "v_pages_shape",
    "bi_status_string", "bi_last_error_message",
    "BI_BF16", "BI_F32", "STATUS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbi.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m invariant_bi_mm_amd._build` "
        "(or __graft_entry__.build()). There is no fallback implementation.")
lib = ctypes.CDLL(LIB_PATH)

BI_BF16, BI_F32 = 0, 1
BI_GEMM_FIXED_TILE = 1
BI_DECODE_NOALLOC_MAX_BYTES = 64 << 20
STATUS = {0: "BI_OK", 1: "BI_ERR_NULL", 2: "BI_ERR_SHAPE", 3: "BI_ERR_STRIDE", 4: "BI_ERR_ALIGN",
          5: "BI_ERR_DTYPE", 6: "BI_ERR_WORKSPACE", 7: "BI_ERR_UNSUPPORTED", 8: "BI_ERR_HIP"}

_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_st = ctypes.c_int

lib.bi_mm.argtypes = [_vp, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _i64, _i64, _i64, _vp]
lib.bi_mm.restype = _st
lib.bi_addmm.argtypes = [_vp, _i32, _f32, _f32, _vp, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _i64, _i64, _i64, _vp]
lib.bi_addmm.restype = _st
lib.bi_gemm_config.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(ctypes.c_int32)]
lib.bi_gemm_config.restype = _st
lib.bi_gemm.argtypes = [_vp, _i32, _f32, _f32, _vp, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _i64, _i64, _i64, _i32,
                        _vp]
lib.bi_gemm.restype = _st
lib.bi_gemm_plan.argtypes = [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(ctypes.c_int32),
                             ctypes.POINTER(ctypes.c_int32)]
lib.bi_gemm_plan.restype = _st
lib.bi_rmsnorm.argtypes = [_vp, _i64, _vp, _f32, _vp, _i64, _i32, _i64, _i64, _vp]
lib.bi_rmsnorm.restype = _st
lib.bi_mean.argtypes = [_vp, _i32, _i64, _vp, _i64, _i64, _vp]
lib.bi_mean.restype = _st
lib.bi_log_softmax.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp]
lib.bi_log_softmax.restype = _st
lib.bi_decode_plan.argtypes = [_vp, _i64, _i32, _vp]
lib.bi_decode_plan.restype = _i64
lib.bi_decode_workspace_bytes.argtypes = [_i64, _i32, _i32]
lib.bi_decode_workspace_bytes.restype = _sz
lib.bi_decode_attention.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                    _f32, _vp, _sz, _vp, _i32, _i32, _vp]
lib.bi_decode_attention.restype = _st
lib.bi_decode_attention_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32,
                                            _i32, _f32, _vp, _i32, _i32, _vp]
lib.bi_decode_attention_noalloc.restype = _st
lib.bi_add_rmsnorm.argtypes = [_vp, _i64, _vp, _i64, _vp, _f32, _vp, _i64, _i32, _i64, _i64, _vp]
lib.bi_add_rmsnorm.restype = _st
lib.bi_embed.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp]
lib.bi_embed.restype = _st
lib.bi_silu_mul.argtypes = [_vp, _i64, _vp, _i64, _i64, _i64, _vp]
lib.bi_silu_mul.restype = _st
lib.bi_qknorm_rope_append.argtypes = [_vp, _i64, _vp, _vp, _f32, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                      _i64, _i32, _i32, _i32, _i32, _vp]
lib.bi_qknorm_rope_append.restype = _st
lib.bi_prefill_plan.argtypes = [_vp, _vp, _i64, _i32, _vp, _vp, _vp, _vp]
lib.bi_prefill_plan.restype = _st
lib.bi_prefill_attention.argtypes = [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _i32,
                                     _i32, _i32, _i32, _f32, _vp, _sz, _vp, _i32, _vp]
lib.bi_prefill_attention.restype = _st
lib.bi_status_string.argtypes = [_st]
lib.bi_status_string.restype = ctypes.c_char_p
lib.bi_last_error_message.argtypes = []
lib.bi_last_error_message.restype = ctypes.c_char_p


class BiError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


def bi_status_string(s: int) -> str:
    return lib.bi_status_string(s).decode()


def bi_last_error_message() -> str:
    return lib.bi_last_error_message().decode()


def _check(status: int):
    if status != 0:
        raise BiError(status, bi_last_error_message() or bi_status_string(status))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BI_BF16
    if dt == torch.float32:
        return BI_F32
    raise TypeError(f"unsupported dtype {dt}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_device(stream, **tensors):
    """Every tensor the kernels dereference must be GPU memory on the device
    whose stream runs them: a host pointer reaching a kernel is a GPU memory
    fault, so this is checked (before anything is launched) rather than left
    to the caller. None entries (optional arguments) are skipped."""
    for name, t in tensors.items():
        if t is not None and (not isinstance(t, torch.Tensor) or not t.is_cuda):
            raise ValueError(f"{name} must be a CUDA (GPU) tensor")
    devs = {t.device for t in tensors.values() if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(str(d) for d in devs)}")
    if stream is not None and devs and stream.device not in devs:
        raise ValueError(f"stream is on {stream.device}, tensors on {devs.pop()}")


def _stream(stream=None, device=None) -> ctypes.c_void_p:
    s = (torch.cuda.current_stream(device) if stream is None else stream)
    return ctypes.c_void_p(s.cuda_stream)


def _out_ok(out, shape, dtypes, name="out"):
    """A caller-supplied output must have the shape and dtype the kernel
    writes (it writes every element of that shape)."""
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {out.dtype}, expected one of {dtypes}")


def _mat(t: torch.Tensor, name: str):
    """(tensor, leading dimension) for a row-major 2-D operand."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.size(1) > 1:
        raise ValueError(f"{name} must have unit stride along its rows")
    if t.size(0) > 1:
        return t, t.stride(0)
    # a single row: the stride is never used for addressing
    return t, ((t.size(1) + 7) // 8) * 8


def _need_bf16(t, name):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")


def _gemm_shapes(a, b, b_is_nk):
    _need_bf16(a, "a")
    _need_bf16(b, "b")
    m, k = a.shape
    n = b.shape[0] if b_is_nk else b.shape[1]
    kb = b.shape[1] if b_is_nk else b.shape[0]
    if kb != k:
        raise ValueError(f"inner dimensions differ: a is {tuple(a.shape)}, b is {tuple(b.shape)} (b_is_nk={b_is_nk})")
    return m, n, k


def bi_mm(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, *, b_is_nk: bool = False,
          out_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """C = a @ b (b [K, N]) or a @ b.T (b [N, K], b_is_nk=True); bf16 in, fp32 accumulate."""
    m, n, k = _gemm_shapes(a, b, b_is_nk)
    _on_device(stream, a=a, b=b, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _out_ok(out, (m, n), (torch.float32, torch.bfloat16))
    a, lda = _mat(a, "a")
    b, ldb = _mat(b, "b")
    out, ldc = _mat(out, "out")
    _check(lib.bi_mm(_ptr(a), lda, _ptr(b), ldb, int(b_is_nk), _ptr(out), ldc, _dtype_code(out.dtype),
                     m, n, k, _stream(stream, a.device)))
    return out


def bi_addmm(bias: torch.Tensor, a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, *,
             beta: float = 1.0, alpha: float = 1.0, b_is_nk: bool = False,
             out_dtype: torch.dtype = torch.float32, stream=None) -> torch.Tensor:
    """C = beta * bias[None, :] + alpha * (a @ b), bias applied after the full K reduction."""
    m, n, k = _gemm_shapes(a, b, b_is_nk)
    if bias.dim() != 1 or bias.shape[0] != n or not bias.is_contiguous():
        raise ValueError("bias must be a contiguous [N] vector")
    _on_device(stream, bias=bias, a=a, b=b, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _out_ok(out, (m, n), (torch.float32, torch.bfloat16))
    a, lda = _mat(a, "a")
    b, ldb = _mat(b, "b")
    out, ldc = _mat(out, "out")
    _check(lib.bi_addmm(_ptr(bias), _dtype_code(bias.dtype), float(beta), float(alpha), _ptr(a), lda, _ptr(b), ldb,
                        int(b_is_nk), _ptr(out), ldc, _dtype_code(out.dtype), m, n, k, _stream(stream, a.device)))
    return out


def bi_gemm(a: torch.Tensor, b: torch.Tensor, bias: torch.Tensor | None = None, out: torch.Tensor | None = None, *,
            beta: float = 1.0, alpha: float = 1.0, b_is_nk: bool = False, out_dtype: torch.dtype = torch.float32,
            fixed_tile: bool = False, stream=None) -> torch.Tensor:
    """bi_mm (bias None) or bi_addmm, with the flags argument: fixed_tile selects
    one tile configuration per (N, K, layout) for every M (same bits)."""
    m, n, k = _gemm_shapes(a, b, b_is_nk)
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != n or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [N] vector")
    _on_device(stream, bias=bias, a=a, b=b, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _out_ok(out, (m, n), (torch.float32, torch.bfloat16))
    a, lda = _mat(a, "a")
    b, ldb = _mat(b, "b")
    out, ldc = _mat(out, "out")
    flags = BI_GEMM_FIXED_TILE if fixed_tile else 0
    _check(lib.bi_gemm(_ptr(bias), _dtype_code(bias.dtype) if bias is not None else BI_F32, float(beta),
                       float(alpha), _ptr(a), lda, _ptr(b), ldb, int(b_is_nk), _ptr(out), ldc, _dtype_code(out.dtype),
                       m, n, k, flags, _stream(stream, a.device)))
    return out


def bi_gemm_plan(m: int, n: int, k: int, b_is_nk: bool = False, fixed_tile: bool = False) -> list:
    """The launches a GEMM of these sizes makes: a list of (tile_m, tile_n,
    tile_k, waves, first column) tuples (two when a 256x256 GEMM splits its
    last columns onto 256x128 tiles)."""
    out = (ctypes.c_int32 * 10)()
    cnt = ctypes.c_int32()
    _check(lib.bi_gemm_plan(m, n, k, int(b_is_nk), BI_GEMM_FIXED_TILE if fixed_tile else 0, out,
                            ctypes.byref(cnt)))
    return [tuple(out[5 * i:5 * i + 5]) for i in range(cnt.value)]


def bi_gemm_config(m: int, n: int, k: int, b_is_nk: bool = False) -> tuple:
    """(tile_m, tile_n, tile_k, waves) the GEMM uses for (m, n, k, layout). Every
    configuration gives each output element the same bits."""
    out = (ctypes.c_int32 * 4)()
    _check(lib.bi_gemm_config(m, n, k, int(b_is_nk), out))
    return tuple(out)


def bi_rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, out: torch.Tensor | None = None, *,
               out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """y = (x * r) * w, r = 1/sqrt(mean(x^2) + eps) per row; x bf16 [M, N], w bf16 [N]."""
    _need_bf16(x, "x")
    _need_bf16(w, "w")
    m, n = x.shape
    if w.dim() != 1 or w.shape[0] != n or not w.is_contiguous():
        raise ValueError("w must be a contiguous [N] vector")
    _on_device(stream, x=x, w=w, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _out_ok(out, (m, n), (torch.float32, torch.bfloat16))
    x, ldx = _mat(x, "x")
    out, ldy = _mat(out, "out")
    _check(lib.bi_rmsnorm(_ptr(x), ldx, _ptr(w), float(eps), _ptr(out), ldy, _dtype_code(out.dtype), m, n,
                          _stream(stream, x.device)))
    return out


def bi_mean(x: torch.Tensor, out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    """y[i] = mean_j x[i, j] in fp32; x bf16 or fp32 [M, N]."""
    m, n = x.shape
    _on_device(stream, x=x, out=out)
    if out is None:
        out = torch.empty((m,), dtype=torch.float32, device=x.device)
    _out_ok(out, (m,), (torch.float32,))
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    x, ldx = _mat(x, "x")
    _check(lib.bi_mean(_ptr(x), _dtype_code(x.dtype), ldx, _ptr(out), m, n, _stream(stream, x.device)))
    return out


def bi_log_softmax(x: torch.Tensor, out: torch.Tensor | None = None, argmax: torch.Tensor | None = None, *,
                   want_argmax: bool = True, stream=None):
    """(log_softmax(x) [M, N] fp32, argmax [M] int64 or None) over fp32 logits."""
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    m, n = x.shape
    _on_device(stream, x=x, out=out, argmax=argmax if want_argmax else None)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _out_ok(out, (m, n), (torch.float32,))
    if want_argmax and argmax is None:
        argmax = torch.empty((m,), dtype=torch.int64, device=x.device)
    if want_argmax:
        _out_ok(argmax, (m,), (torch.int64,), "argmax")
        if not argmax.is_contiguous():
            raise ValueError("argmax must be contiguous")
    x, ldx = _mat(x, "x")
    out, ldy = _mat(out, "out")
    _check(lib.bi_log_softmax(_ptr(x), ldx, _ptr(out), ldy, _ptr(argmax if want_argmax else None), m, n,
                              _stream(stream, x.device)))
    return out, (argmax if want_argmax else None)


def bi_decode_plan(context_lens_host: torch.Tensor, split_tokens: int = 256):
    """Host plan: (split_offsets int32 [B+1] on the host, total splits)."""
    lens = context_lens_host.to(torch.int32).contiguous().cpu()
    offs = torch.empty(lens.numel() + 1, dtype=torch.int32)
    total = lib.bi_decode_plan(_ptr(lens), lens.numel(), int(split_tokens), _ptr(offs))
    if total < 0:
        raise BiError(2, bi_last_error_message())
    return offs, int(total)


def bi_decode_workspace_bytes(total_splits: int, num_q_heads: int, head_dim: int) -> int:
    return int(lib.bi_decode_workspace_bytes(total_splits, num_q_heads, head_dim))


def v_pages_shape(k_pages) -> tuple:
    """Shape of the V page pool that goes with k_pages [P, Hkv, page, D]:
    [P, Hkv, D, page] (d-major, so a value tile of 8 tokens of one head-dim
    element is one 16-byte load)."""
    p, hkv, page, d = k_pages.shape
    return (p, hkv, d, page)


def bi_decode_attention(q, k_pages, v_pages, block_table, context_lens, split_offsets, total_splits: int, *,
                        scale: float | None = None, split_tokens: int = 256, workspace=None, out=None,
                        out_dtype: torch.dtype = torch.float32, stream_kv: bool = False, stream=None):
    """Split-KV decode attention over a paged cache.

    stream_kv loads K and V non-temporal (a cache hint; same bits).

    q [B, Hq, D] bf16; k_pages [P, Hkv, page, D] and v_pages [P, Hkv, D, page]
    (d-major) bf16; block_table
    [B, max_pages] int32; context_lens [B] int32 and split_offsets [B+1]
    int32 on the device (split_offsets from bi_decode_plan)."""
    _need_bf16(q, "q")
    _need_bf16(k_pages, "k_pages")
    _need_bf16(v_pages, "v_pages")
    bsz, hq, d = q.shape
    _, hkv, page, d2 = k_pages.shape
    if d2 != d or v_pages.shape != v_pages_shape(k_pages):
        raise ValueError("q/k/v shapes disagree (v_pages is [P, Hkv, D, page])")
    for t, nm in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                  (context_lens, "context_lens"), (split_offsets, "split_offsets")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32 or split_offsets.dtype != torch.int32:
        raise TypeError("block_table, context_lens, split_offsets must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != bsz:
        raise ValueError(f"block_table must be [B={bsz}, max_pages], got {tuple(block_table.shape)}")
    if context_lens.numel() != bsz or split_offsets.numel() != bsz + 1:
        raise ValueError(f"context_lens must hold B={bsz} entries and split_offsets B+1={bsz + 1} "
                         f"(got {context_lens.numel()} and {split_offsets.numel()})")
    _on_device(stream, q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table, context_lens=context_lens,
               split_offsets=split_offsets, workspace=workspace, out=out)
    if scale is None:
        scale = d ** -0.5
    need = bi_decode_workspace_bytes(total_splits, hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((bsz, hq, d), dtype=out_dtype, device=q.device)
    _out_ok(out, (bsz, hq, d), (torch.float32, torch.bfloat16))
    if not out.is_contiguous() or not workspace.is_contiguous():
        raise ValueError("out and workspace must be contiguous")
    _check(lib.bi_decode_attention(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), block_table.shape[1],
                                   _ptr(context_lens), _ptr(split_offsets), int(total_splits), bsz, hq, hkv, d,
                                   page, int(split_tokens), float(scale), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _ptr(out), _dtype_code(out.dtype), 1 if stream_kv else 0,
                                   _stream(stream, q.device)))
    return out


def bi_decode_attention_noalloc(q, k_pages, v_pages, block_table, context_lens, split_offsets, total_splits: int,
                                out, *, scale: float | None = None, split_tokens: int = 256, stream_kv: bool = False,
                                stream=None):
    """bi_decode_attention with the library's own scratch for the split
    partials instead of a workspace: nothing is allocated, `out` (bf16 or
    fp32 [B, Hq, D], contiguous) is the caller's. Splits whose partials
    exceed BI_DECODE_NOALLOC_MAX_BYTES are refused (BI_ERR_WORKSPACE)."""
    _need_bf16(q, "q")
    _need_bf16(k_pages, "k_pages")
    _need_bf16(v_pages, "v_pages")
    bsz, hq, d = q.shape
    _, hkv, page, d2 = k_pages.shape
    if d2 != d or v_pages.shape != v_pages_shape(k_pages):
        raise ValueError("q/k/v shapes disagree (v_pages is [P, Hkv, D, page])")
    for t, nm in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                  (context_lens, "context_lens"), (split_offsets, "split_offsets"), (out, "out")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32 or split_offsets.dtype != torch.int32:
        raise TypeError("block_table, context_lens, split_offsets must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != bsz:
        raise ValueError(f"block_table must be [B={bsz}, max_pages], got {tuple(block_table.shape)}")
    if context_lens.numel() != bsz or split_offsets.numel() != bsz + 1:
        raise ValueError(f"context_lens must hold B={bsz} entries and split_offsets B+1={bsz + 1}")
    _on_device(stream, q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table, context_lens=context_lens,
               split_offsets=split_offsets, out=out)
    _out_ok(out, (bsz, hq, d), (torch.float32, torch.bfloat16))
    if scale is None:
        scale = d ** -0.5
    _check(lib.bi_decode_attention_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                           block_table.shape[1], _ptr(context_lens), _ptr(split_offsets),
                                           int(total_splits), bsz, hq, hkv, d, page, int(split_tokens), float(scale),
                                           _ptr(out), _dtype_code(out.dtype), 1 if stream_kv else 0,
                                           _stream(stream, q.device)))
    return out


def bi_add_rmsnorm(x: torch.Tensor, d: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, out: torch.Tensor | None = None,
                   *, out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """x <- bf16(x + d) in place; returns rmsnorm(x) (x, d bf16 [M, N], w bf16 [N])."""
    _need_bf16(x, "x")
    _need_bf16(d, "d")
    _need_bf16(w, "w")
    m, n = x.shape
    if d.shape != x.shape:
        raise ValueError("d must have x's shape")
    if w.dim() != 1 or w.shape[0] != n or not w.is_contiguous():
        raise ValueError("w must be a contiguous [N] vector")
    _on_device(stream, x=x, d=d, w=w, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _out_ok(out, (m, n), (torch.float32, torch.bfloat16))
    x, ldx = _mat(x, "x")
    d, ldd = _mat(d, "d")
    out, ldy = _mat(out, "out")
    _check(lib.bi_add_rmsnorm(_ptr(x), ldx, _ptr(d), ldd, _ptr(w), float(eps), _ptr(out), ldy,
                              _dtype_code(out.dtype), m, n, _stream(stream, x.device)))
    return out


def bi_embed(table: torch.Tensor, tokens: torch.Tensor, out: torch.Tensor | None = None, *, stream=None):
    """out[i] = table[tokens[i]] (bf16 [V, N] table, int64 [M] device tokens); bad tokens give zero rows."""
    _need_bf16(table, "table")
    if tokens.dtype != torch.int64 or tokens.dim() != 1 or not tokens.is_contiguous():
        raise TypeError("tokens must be a contiguous int64 vector")
    vocab, n = table.shape
    m = tokens.shape[0]
    _on_device(stream, table=table, tokens=tokens, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=table.device)
    _out_ok(out, (m, n), (torch.bfloat16,))
    table, ld = _mat(table, "table")
    out, ldo = _mat(out, "out")
    _check(lib.bi_embed(_ptr(table), ld, vocab, _ptr(tokens), _ptr(out), ldo, m, n, _stream(stream, table.device)))
    return out


def bi_silu_mul(gu: torch.Tensor, out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    """out = silu(gu[:, :n]) * gu[:, n:] (bf16 [M, 2n] -> bf16 [M, n])."""
    _need_bf16(gu, "gu")
    m, n2 = gu.shape
    if n2 % 2:
        raise ValueError("gu must have an even number of columns")
    n = n2 // 2
    _on_device(stream, gu=gu, out=out)
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=gu.device)
    _out_ok(out, (m, n), (torch.bfloat16,))
    gu, ldg = _mat(gu, "gu")
    out, ldo = _mat(out, "out")
    _check(lib.bi_silu_mul(_ptr(gu), ldg, _ptr(out), ldo, m, n, _stream(stream, gu.device)))
    return out


def bi_qknorm_rope_append(qkv, q_norm_w, k_norm_w, cos_tab, sin_tab, positions, block_table, k_pages, v_pages, *,
                          num_q_heads: int, num_kv_heads: int, eps: float = 1e-6, q_out=None, stream=None):
    """Per-head q/k RMSNorm + rotary embedding; q to q_out [B, Hq, D], k and v into the paged cache at positions."""
    for t, nm in ((qkv, "qkv"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w"), (k_pages, "k_pages"),
                  (v_pages, "v_pages")):
        _need_bf16(t, nm)
    if cos_tab.dtype != torch.float32 or sin_tab.dtype != torch.float32 or cos_tab.shape != sin_tab.shape:
        raise TypeError("cos_tab and sin_tab must be fp32 tables of one shape")
    if positions.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise TypeError("positions and block_table must be int32")
    for t, nm in ((cos_tab, "cos_tab"), (sin_tab, "sin_tab"), (positions, "positions"), (block_table, "block_table"),
                  (k_pages, "k_pages"), (v_pages, "v_pages"), (q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    bsz = qkv.shape[0]
    num_pages, hkv, page, d = k_pages.shape
    if hkv != num_kv_heads or v_pages.shape != v_pages_shape(k_pages):
        raise ValueError("cache shape disagrees with num_kv_heads (k [P, Hkv, page, D], v [P, Hkv, D, page])")
    if qkv.dim() != 2 or qkv.shape[1] < (num_q_heads + 2 * num_kv_heads) * d:
        raise ValueError("qkv must be [B, (Hq + 2 Hkv) D]")
    if positions.numel() != bsz or block_table.dim() != 2 or block_table.shape[0] != bsz:
        raise ValueError(f"positions must hold B={bsz} entries and block_table be [B, max_pages]")
    if cos_tab.dim() != 2 or cos_tab.shape[1] != d // 2 or q_norm_w.numel() != d or k_norm_w.numel() != d:
        raise ValueError("cos/sin tables must be [max_pos, D/2] and the norm weights [D]")
    _on_device(stream, qkv=qkv, q_norm_w=q_norm_w, k_norm_w=k_norm_w, cos_tab=cos_tab, sin_tab=sin_tab,
               positions=positions, block_table=block_table, k_pages=k_pages, v_pages=v_pages, q_out=q_out)
    if q_out is None:
        q_out = torch.empty((bsz, num_q_heads, d), dtype=torch.bfloat16, device=qkv.device)
    _out_ok(q_out, (bsz, num_q_heads, d), (torch.bfloat16,), "q_out")
    if not q_out.is_contiguous():
        raise ValueError("q_out must be contiguous")
    qkv, ldq = _mat(qkv, "qkv")
    _check(lib.bi_qknorm_rope_append(_ptr(qkv), ldq, _ptr(q_norm_w), _ptr(k_norm_w), float(eps), _ptr(cos_tab),
                                     _ptr(sin_tab), cos_tab.shape[0], _ptr(positions), _ptr(block_table),
                                     block_table.shape[1], num_pages, _ptr(k_pages), _ptr(v_pages), _ptr(q_out), bsz,
                                     num_q_heads, num_kv_heads, d, page, _stream(stream, qkv.device)))
    return q_out


def bi_prefill_plan(chunk_lens_host: torch.Tensor, ctx_before_host: torch.Tensor, split_tokens: int = 256):
    """Host plan for bi_prefill_attention: (q_pos [rows], q_offsets [rows+1], work [n_work, 4]) int32 CPU
    tensors and (rows, total_splits, n_work)."""
    cl = chunk_lens_host.to(torch.int32).contiguous()
    cb = ctx_before_host.to(torch.int32).contiguous()
    if cl.device.type != "cpu" or cb.device.type != "cpu" or cl.shape != cb.shape or cl.dim() != 1:
        raise ValueError("chunk_lens and ctx_before must be 1-D host tensors of one length")
    sizes = (ctypes.c_int64 * 3)()
    _check(lib.bi_prefill_plan(_ptr(cl), _ptr(cb), cl.shape[0], int(split_tokens), None, None, None, sizes))
    rows, total, n_work = (int(x) for x in sizes)
    q_pos = torch.empty(max(rows, 1), dtype=torch.int32)
    q_offs = torch.empty(rows + 1, dtype=torch.int32)
    work = torch.empty((max(n_work, 1), 4), dtype=torch.int32)
    _check(lib.bi_prefill_plan(_ptr(cl), _ptr(cb), cl.shape[0], int(split_tokens), _ptr(q_pos), _ptr(q_offs),
                               _ptr(work), sizes))
    return q_pos[:rows], q_offs, work[:n_work], (rows, total, n_work)


def bi_prefill_attention(q, k_pages, v_pages, block_table, q_pos, q_offsets, work, sizes, *, scale=None,
                         split_tokens: int = 256, workspace=None, out=None, out_dtype: torch.dtype = torch.float32,
                         stream=None):
    """Causal attention of chunk tokens over their sequences' paged cache, with the decode split structure.
    q [rows, Hq, D] bf16; q_pos, q_offsets, work: the plan's arrays on the device; sizes: the plan's tuple."""
    _need_bf16(q, "q")
    _need_bf16(k_pages, "k_pages")
    _need_bf16(v_pages, "v_pages")
    rows, total, n_work = sizes
    nr, hq, d = q.shape
    if nr != rows:
        raise ValueError("q has a different number of rows than the plan")
    _, hkv, page, d2 = k_pages.shape
    if d2 != d or v_pages.shape != v_pages_shape(k_pages):
        raise ValueError("q/k/v shapes disagree (v_pages is [P, Hkv, D, page])")
    for t, nm in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                  (q_pos, "q_pos"), (q_offsets, "q_offsets"), (work, "work")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    for t, nm in ((block_table, "block_table"), (q_pos, "q_pos"), (q_offsets, "q_offsets"), (work, "work")):
        if t.dtype != torch.int32:
            raise TypeError(f"{nm} must be int32")
    if q_pos.numel() != rows or q_offsets.numel() != rows + 1 or work.numel() != 4 * n_work:
        raise ValueError("q_pos, q_offsets and work must have the plan's sizes (rows, rows + 1, 4 n_work)")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_pages]")
    _on_device(stream, q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table, q_pos=q_pos,
               q_offsets=q_offsets, work=work, workspace=workspace, out=out)
    if scale is None:
        scale = d ** -0.5
    need = bi_decode_workspace_bytes(total, hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((rows, hq, d), dtype=out_dtype, device=q.device)
    _out_ok(out, (rows, hq, d), (torch.float32, torch.bfloat16))
    if not out.is_contiguous() or not workspace.is_contiguous():
        raise ValueError("out and workspace must be contiguous")
    _check(lib.bi_prefill_attention(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), block_table.shape[1],
                                    _ptr(q_pos), _ptr(q_offsets), _ptr(work), n_work, rows, total,
                                    block_table.shape[0], hq, hkv, d, page, int(split_tokens), float(scale),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
                                    _dtype_code(out.dtype), _stream(stream, q.device)))
    return out
