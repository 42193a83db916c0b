"""Seeded synthetic inputs, shared by the tests, the benchmark and smoke().

This module only draws random numbers and converts them to a storage dtype.
It holds none of the arithmetic of the kernels or of the oracle, so both
sides can be fed from it without sharing any of the method.

Conventions
-----------
* ``N(mu, s)`` in the workload descriptions is read with ``s`` as the
  *variance* (textbook N(mu, sigma^2)); ``normal_bf16(..., var=s)`` therefore
  draws with standard deviation ``sqrt(s)``.
* Draws are fp32 from a seeded ``torch.Generator`` and are converted to
  bfloat16 with torch's round-to-nearest-even conversion.
* Seeds are plain integers; callers derive them as
  ``1000 * config + 100 * role + M`` so that a row drawn with a seed that has
  no ``M`` term is the same row whatever the batch size.
"""
from __future__ import annotations

import math

import torch

__all__ = [
    "generator",
    "normal_f32",
    "normal_bf16",
    "uniform_bf16",
    "rows_with_fixed_row",
    "context_lens",
    "paged_kv_layout",
    "bf16_bits_numpy",
    "f32_numpy",
    "rope_tables",
    "qwen3_weights",
]


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_f32(shape, var: float, seed: int, device="cpu") -> torch.Tensor:
    """fp32 draws from N(0, var) (``var`` is the variance)."""
    g = generator(seed, device)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    if var != 1.0:
        x.mul_(math.sqrt(var))
    return x


def normal_bf16(shape, var: float, seed: int, device="cpu") -> torch.Tensor:
    """bf16 tensor, fp32 N(0, var) draws rounded to nearest-even."""
    return normal_f32(shape, var, seed, device).to(torch.bfloat16)


def uniform_bf16(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    g = generator(seed, device)
    x = torch.rand(*shape, generator=g, dtype=torch.float32, device=device)
    x.mul_(hi - lo).add_(lo)
    return x.to(torch.bfloat16)


def rows_with_fixed_row(m: int, k: int, var: float, fixed_seed: int, other_seed: int,
                        fixed_pos: int = 0, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """[m, k] matrix whose row ``fixed_pos`` comes from ``fixed_seed`` alone
    (so it is the same row for every m) and whose other rows come from
    ``other_seed``."""
    x = normal_f32((m, k), var, other_seed, device)
    x[fixed_pos] = normal_f32((1, k), var, fixed_seed, device)[0]
    return x.to(dtype)


def context_lens(batch: int, seed: int, lo: int = 1, hi: int = 32768) -> torch.Tensor:
    """Context lengths log-uniform in [lo, hi]:
    L = clamp(floor(exp(U * ln(hi + 1))), lo, hi) with U ~ U[0, 1)."""
    g = generator(seed)
    u = torch.rand(batch, generator=g, dtype=torch.float64)
    lens = torch.floor(torch.exp(u * math.log(hi + 1))).clamp_(lo, hi)
    return lens.to(torch.int32)


def paged_kv_layout(lens: torch.Tensor, page_size: int, seed: int):
    """Random physical page placement for a batch of sequences.

    Returns ``(block_table [B, max_pages] int32, num_pages)``: logical page
    ``i`` of sequence ``b`` lives in physical page ``block_table[b, i]``.
    Physical pages are a random permutation, so neighbouring logical pages
    are not neighbours in memory. Unused table entries are 0.
    """
    lens = lens.to(torch.int64)
    pages_per_seq = (lens + page_size - 1) // page_size
    total = int(pages_per_seq.sum())
    max_pages = max(int(pages_per_seq.max()) if len(lens) else 1, 1)
    perm = torch.randperm(max(total, 1), generator=generator(seed), dtype=torch.int64)
    table = torch.zeros((len(lens), max_pages), dtype=torch.int32)
    off = 0
    for b, n in enumerate(pages_per_seq.tolist()):
        table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return table, max(total, 1)


def bf16_bits_numpy(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (no value conversion)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def f32_numpy(t: torch.Tensor):
    return t.detach().cpu().contiguous().to(torch.float32).numpy()


def rope_tables(max_pos: int, head_dim: int = 128, theta: float = 1.0e6):
    """The rotary-embedding angle table both sides take as an input:
    angle[p, i] = p * theta^(-2i / head_dim) for i < head_dim / 2, evaluated
    in float64 and stored as fp32 (cos, sin) [max_pos, head_dim / 2].
    theta = 1e6 is the Qwen3 base. It is the input of the rotation, not the
    rotation itself, which each side applies on its own."""
    i = torch.arange(head_dim // 2, dtype=torch.float64)
    inv = theta ** (-2.0 * i / head_dim)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def qwen3_weights(hidden: int, num_q_heads: int, num_kv_heads: int, head_dim: int, intermediate: int, vocab: int,
                  layers: int, seed: int, device="cpu", max_pos: int = 40000, qk_norm=(0.5, 1.5), b_is_nk: bool = True):
    """Random weights of a Qwen3-style decoder: projections N(0, 0.02) (the
    projection-GEMM workloads' draw), embedding N(0, 1), LM-head bias
    N(0, 0.1), RMSNorm weights U(0.5, 1.5) (the q/k ones U(qk_norm)), and
    the rotary tables of ``rope_tables``. Every projection and the LM head
    is stored [N, K] (nn.Linear's [out, in]) when ``b_is_nk``, else [K, N];
    the dict's "b_is_nk" entry says which. Other keys are the ones the
    decode step takes (embed, w_in, w_qkv, q_norm, k_norm, w_o, w_post,
    w_gu, w_down, w_final, w_lm, b_lm, cos, sin); per-layer entries are
    lists."""
    h, d = hidden, head_dim
    qkv_n = (num_q_heads + 2 * num_kv_heads) * d
    r = lambda shape, var, k: normal_bf16(shape, var, seed=seed + k, device=device)  # noqa: E731
    m = (lambda k_, n_, var, k: r((n_, k_), var, k)) if b_is_nk else (lambda k_, n_, var, k: r((k_, n_), var, k))  # noqa: E731
    u = lambda n, k, lo=0.5, hi=1.5: uniform_bf16((n,), lo, hi, seed=seed + k, device=device)  # noqa: E731
    w = {"embed": r((vocab, h), 1.0, 1),
         "w_in": [u(h, 100 + l) for l in range(layers)], "w_post": [u(h, 200 + l) for l in range(layers)],
         "q_norm": [u(d, 300 + l, *qk_norm) for l in range(layers)],
         "k_norm": [u(d, 400 + l, *qk_norm) for l in range(layers)],
         "w_qkv": [m(h, qkv_n, 0.02, 500 + l) for l in range(layers)],
         "w_o": [m(num_q_heads * d, h, 0.02, 600 + l) for l in range(layers)],
         "w_gu": [m(h, 2 * intermediate, 0.02, 700 + l) for l in range(layers)],
         "w_down": [m(intermediate, h, 0.02, 800 + l) for l in range(layers)],
         "w_final": u(h, 2), "w_lm": m(h, vocab, 0.02, 3), "b_lm": r((vocab,), 0.1, 4), "b_is_nk": b_is_nk}
    cos, sin = rope_tables(max_pos, d)
    w["cos"], w["sin"] = cos.to(device), sin.to(device)
    return w
