"""Plain fp64 CPU oracle for the batch-invariant inference kernels.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path. It imports
numpy and the standard library only.

Sources. The pages describe batch-invariant replacements for PyTorch's
kernels; they change the *order* of the floating-point reduction, never the
quantity computed:

* "thinking-machines-lab/batch_invariant_ops" (catalogue page), sections
  "What it is" (a drop-in replacement for standard PyTorch kernels, so
  PyTorch semantics) and "When to avoid" (the supported ops: mm, addmm,
  log_softmax, mean).
* "Batch-invariant inference kernels (Thinking Machines) -- Evidence &
  limits", section "Evidence" (SGLang took the mean, log-softmax and matmul
  kernels and wrote its own batch-invariant attention).
* readhandoff.com, agent-run reproducibility pinning, section "What does
  temperature zero actually guarantee?" (matmul, RMSNorm and attention are the
  inference kernels whose output depends on batch size; greedy sampling picks
  the highest-probability token) and "Frequently asked questions".
* "How to achieve deterministic LLMs with batch invariant inference", "TL;DR"
  (fixing the reduction order is the whole mechanism).

So each function below is the textbook definition of its op in float64; no
blocking or reordering is applied beyond what numpy's fp64 matmul/sum do
internally (both far more accurate than the fp32 tolerance checked).

Readings where the pages are silent (no formula, tile size or precision is
printed on any page):

* RMSNorm: y = w * x / sqrt(mean(x^2) + eps) (textbook RMSNorm).
* argmax: lowest index attaining the maximum of the fp32 logits (PyTorch's
  tie rule).
* Decode attention: softmax(q.K^T * scale) V over all cached tokens of the
  sequence, grouped-query head map h -> h // (Hq / Hkv), paged K/V cache
  [pages, Hkv, page_size, D].
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "f32_to_f64",
    "mm",
    "addmm",
    "rmsnorm",
    "mean",
    "log_softmax",
    "argmax",
    "gather_kv",
    "decode_attention",
    "decode_attention_split",
    "decode_split_counts",
    "prefill_attention",
    "relative_frobenius",
    "elementwise_ratio",
    "round_bf16",
    "bf16_bits_of",
    "embed",
    "add_rmsnorm",
    "silu_mul",
    "qknorm_rope",
]


# --------------------------------------------------------------------------
# exact decoding of stored values
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 value is the upper 16 bits of the fp32 with the same value, so
    shifting the pattern into the top half of a 32-bit word and reading it as
    fp32 is exact; fp32 -> fp64 is exact too.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 inputs must be uint16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f32_to_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("expected float32")
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# mm / addmm  ("When to avoid": mm, addmm are supported ops; PyTorch semantics)
# --------------------------------------------------------------------------
def mm(a_bits, b_bits, b_is_nk: bool = False) -> np.ndarray:
    """C = A @ B in fp64.

    A is [M, K] bf16. B is [K, N] bf16, or [N, K] when ``b_is_nk`` (the
    nn.Linear weight layout, C = A @ B^T). C_ij = sum_k A_ik B_kj.
    """
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    if b_is_nk:
        b = b.T
    if a.shape[1] != b.shape[0]:
        raise ValueError("inner dimensions differ")
    return a @ b


def addmm(bias, a_bits, b_bits, beta: float = 1.0, alpha: float = 1.0,
          b_is_nk: bool = False) -> np.ndarray:
    """out = beta * bias + alpha * (A @ B), bias [N] broadcast over rows
    (torch.addmm with a 1-D input). ``bias`` is bf16 bits (uint16) or fp32."""
    bias = np.asarray(bias)
    bias64 = bf16_bits_to_f64(bias) if bias.dtype == np.uint16 else f32_to_f64(bias)
    return beta * bias64[None, :] + alpha * mm(a_bits, b_bits, b_is_nk)


# --------------------------------------------------------------------------
# row reductions
# --------------------------------------------------------------------------
def rmsnorm(x_bits, w_bits, eps: float) -> np.ndarray:
    """y_ij = w_j * x_ij / sqrt((1/N) sum_k x_ik^2 + eps).

    RMSNorm is named among the non-invariant inference kernels ("What does
    temperature zero actually guarantee?"); the formula is the textbook one.
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    n = x.shape[1]
    ms = np.sum(x * x, axis=1) / n
    return w[None, :] * x / np.sqrt(ms + eps)[:, None]


def mean(x) -> np.ndarray:
    """y_i = (1/N) sum_j x_ij. ``x`` is bf16 bits or fp32 ("When to avoid":
    mean is a supported op)."""
    x = np.asarray(x)
    x64 = bf16_bits_to_f64(x) if x.dtype == np.uint16 else f32_to_f64(x)
    return np.sum(x64, axis=1) / x64.shape[1]


def log_softmax(x_f32) -> np.ndarray:
    """y_ij = x_ij - m_i - log sum_k exp(x_ik - m_i), m_i = max_k x_ik.

    Subtracting the row max is exact algebra (it cancels); it only keeps
    exp() in range. "When to avoid": log_softmax is a supported op.
    """
    x = f32_to_f64(x_f32)
    m = np.max(x, axis=1, keepdims=True)
    s = np.sum(np.exp(x - m), axis=1, keepdims=True)
    return x - m - np.log(s)


def argmax(x_f32) -> np.ndarray:
    """Greedy (temperature-0) choice: the lowest index attaining the row
    maximum of the fp32 logits. Comparison of the stored fp32 values is
    exact, so no precision question arises."""
    x = np.asarray(x_f32)
    if x.dtype != np.float32:
        raise TypeError("expected float32 logits")
    return np.argmax(x, axis=1).astype(np.int64)  # numpy returns the first maximum


# --------------------------------------------------------------------------
# decode attention over a paged KV cache
# --------------------------------------------------------------------------
def gather_kv(pages_bits, block_table, seq_len: int, kv_head: int, b: int, d_major: bool = False) -> np.ndarray:
    """Logical tokens 0..seq_len-1 of sequence ``b``, head ``kv_head``, as a
    [seq_len, D] fp64 array. ``pages_bits`` is [P, Hkv, page_size, D] bf16
    bits (the key pages), or [P, Hkv, D, page_size] when ``d_major`` (the
    value pages); token t lives in physical page block_table[b, t // page_size]
    at slot t % page_size."""
    page_size = pages_bits.shape[3 if d_major else 2]
    d = pages_bits.shape[2 if d_major else 3]
    out = np.empty((seq_len, d), dtype=np.float64)
    for t0 in range(0, seq_len, page_size):
        p = int(block_table[b, t0 // page_size])
        n = min(page_size, seq_len - t0)
        blk = pages_bits[p, kv_head, :, :n].T if d_major else pages_bits[p, kv_head, :n, :]
        out[t0:t0 + n] = bf16_bits_to_f64(blk)
    return out


def decode_attention(q_bits, k_pages_bits, v_pages_bits, block_table, context_lens,
                     scale: float, seqs=None) -> np.ndarray:
    """out[b, h, :] = sum_t p_t V_t with p = softmax_t(scale * q_bh . K_t),
    t over the sequence's cached tokens, K/V taken from kv head
    g = h // (Hq / Hkv).

    ``seqs`` restricts the computation to some sequences (the others are
    left as NaN) so large batches can be sampled.
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, hq, d = q.shape
    hkv = k_pages_bits.shape[1]
    group = hq // hkv
    out = np.full((bsz, hq, d), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        L = int(context_lens[b])
        for g in range(hkv):
            k = gather_kv(k_pages_bits, block_table, L, g, b)
            v = gather_kv(v_pages_bits, block_table, L, g, b, d_major=True)
            for h in range(g * group, (g + 1) * group):
                s = scale * (k @ q[b, h])
                p = np.exp(s - s.max())
                out[b, h] = (p / p.sum()) @ v
    return out


def prefill_attention(q_bits, k_pages_bits, v_pages_bits, block_table, q_seq, q_pos, scale: float) -> np.ndarray:
    """Causal attention of chunk tokens: row r (sequence q_seq[r], position
    p = q_pos[r]) attends tokens 0..p of its sequence, out[r, h] =
    softmax_t(scale * q[r, h] . K_t) V over those p + 1 tokens, kv head
    h // (Hq / Hkv). The cache already holds the chunk's tokens."""
    q = bf16_bits_to_f64(q_bits)
    rows, hq, d = q.shape
    hkv = k_pages_bits.shape[1]
    group = hq // hkv
    out = np.empty((rows, hq, d))
    for r in range(rows):
        b, L = int(q_seq[r]), int(q_pos[r]) + 1
        for g in range(hkv):
            k = gather_kv(k_pages_bits, block_table, L, g, b)
            v = gather_kv(v_pages_bits, block_table, L, g, b, d_major=True)
            for h in range(g * group, (g + 1) * group):
                sc = scale * (k @ q[r, h])
                p = np.exp(sc - sc.max())
                out[r, h] = (p / p.sum()) @ v
    return out


def decode_split_counts(context_lens, split_tokens: int) -> np.ndarray:
    """Number of KV splits per sequence when splits are cut at fixed
    multiples of ``split_tokens`` of the sequence's own token index:
    ceil(L / split_tokens). It depends on L alone, never on the batch."""
    lens = np.asarray(context_lens, dtype=np.int64)
    return (lens + split_tokens - 1) // split_tokens


def decode_attention_split(q_bits, k_pages_bits, v_pages_bits, block_table, context_lens,
                           scale: float, split_tokens: int, seqs=None) -> np.ndarray:
    """The same attention computed in the split form, in fp64.

    Keys are cut into splits s = [s*split_tokens, (s+1)*split_tokens) of the
    token index. Each split gives (m_s, l_s, o_s) = (max score, sum of
    exp(score - m_s), sum of exp(score - m_s) V_t); the splits are merged in
    increasing s: M = max_s m_s, l = sum_s e^(m_s - M) l_s,
    o = sum_s e^(m_s - M) o_s, out = o / l. This is an identity of softmax,
    so in exact arithmetic it equals ``decode_attention``; the tests check
    that it does in fp64 (which pins the merge algebra the kernels use).
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, hq, d = q.shape
    hkv = k_pages_bits.shape[1]
    group = hq // hkv
    out = np.full((bsz, hq, d), np.nan)
    for b in (range(bsz) if seqs is None else seqs):
        L = int(context_lens[b])
        for g in range(hkv):
            k = gather_kv(k_pages_bits, block_table, L, g, b)
            v = gather_kv(v_pages_bits, block_table, L, g, b, d_major=True)
            for h in range(g * group, (g + 1) * group):
                parts = []
                for t0 in range(0, L, split_tokens):
                    s = scale * (k[t0:t0 + split_tokens] @ q[b, h])
                    m_s = s.max()
                    e = np.exp(s - m_s)
                    parts.append((m_s, e.sum(), e @ v[t0:t0 + split_tokens]))
                M = max(p[0] for p in parts)
                lsum = 0.0
                o = np.zeros(d)
                for m_s, l_s, o_s in parts:
                    c = math.exp(m_s - M)
                    lsum += c * l_s
                    o += c * o_s
                out[b, h] = o / lsum
    return out


# --------------------------------------------------------------------------
# comparison helpers (tolerance: relative Frobenius and elementwise bound)
# --------------------------------------------------------------------------
def relative_frobenius(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)


def elementwise_ratio(got, ref) -> float:
    """max_ij |got - ref| / (|ref| + 1); the bound is 4e-3."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + 1.0)))


# --------------------------------------------------------------------------
# per-token steps of a decode step (the token path of the completions
# experiment: readhandoff.com, agent-run reproducibility pinning, "Where the
# divergence showed up"; Qwen3-8B decoding in its "Key takeaways")
# --------------------------------------------------------------------------
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(v) -> np.ndarray:
    """fp64 -> the nearest bfloat16 value (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits: with v = m * 2^e, 0.5 <= |m| < 1,
    the result is rint(m * 2^8) * 2^(e-8), where rint rounds half to even.
    Magnitudes that round past the largest finite bfloat16 become inf.
    (Below 2^-126, where bfloat16 loses precision gradually, this keeps 8
    bits; no quantity here gets that small.)
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)


def bf16_bits_of(v) -> np.ndarray:
    """Bit patterns (uint16) of fp64 values that are already bfloat16 values
    (as returned by round_bf16): the upper half of their exact fp32 form."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def embed(table_bits, tokens) -> np.ndarray:
    """out[i] = table[tokens[i]] (a token outside the table gives a zero row)."""
    tb = bf16_bits_to_f64(table_bits)
    out = np.zeros((len(tokens), tb.shape[1]))
    for i, t in enumerate(np.asarray(tokens)):
        if 0 <= t < tb.shape[0]:
            out[i] = tb[t]
    return out


def add_rmsnorm(x_bits, d_bits, w_bits, eps: float):
    """Residual add then RMSNorm: x' = round_bf16(x + d) (the residual stream
    is stored in bf16), y = rmsnorm(x'). Returns (x' as bf16 bits, y fp64)."""
    xn = round_bf16(bf16_bits_to_f64(x_bits) + bf16_bits_to_f64(d_bits))
    bits = bf16_bits_of(xn)
    return bits, rmsnorm(bits, w_bits, eps)


def silu_mul(gu_bits) -> np.ndarray:
    """out_ij = silu(g_ij) * u_ij, g = gu[:, :n], u = gu[:, n:],
    silu(g) = g / (1 + e^-g): the gated MLP activation of a Qwen3 layer."""
    gu = bf16_bits_to_f64(gu_bits)
    n = gu.shape[1] // 2
    g, u = gu[:, :n], gu[:, n:]
    return g / (1.0 + np.exp(-g)) * u


def qknorm_rope(qkv_bits, q_norm_w_bits, k_norm_w_bits, eps: float, cos_tab, sin_tab, positions,
                num_q_heads: int, num_kv_heads: int):
    """Qwen3 attention prologue for one new token per sequence.

    Each q and k head x (length D) is RMS-normalised with its weight,
    t = w * x / sqrt(mean(x^2) + eps), then rotated at position p on the
    pairs (i, i + D/2): (t_i, t_{i+D/2}) -> (t_i c - t_{i+D/2} s,
    t_{i+D/2} c + t_i s) with c = cos_tab[p, i], s = sin_tab[p, i]. v heads
    pass unchanged. Returns (q [B, Hq, D], k [B, Hkv, D], v [B, Hkv, D]) in
    fp64.
    """
    qkv = bf16_bits_to_f64(qkv_bits)
    bsz = qkv.shape[0]
    d = 128
    heads = qkv[:, :(num_q_heads + 2 * num_kv_heads) * d].reshape(bsz, num_q_heads + 2 * num_kv_heads, d)
    qw = bf16_bits_to_f64(q_norm_w_bits)
    kw = bf16_bits_to_f64(k_norm_w_bits)
    cos = np.asarray(cos_tab, dtype=np.float64)
    sin = np.asarray(sin_tab, dtype=np.float64)

    def norm_rot(x, w, p):
        t = w * x / np.sqrt(np.mean(x * x) + eps)
        c, s = cos[p], sin[p]
        a, b = t[:d // 2], t[d // 2:]
        return np.concatenate([a * c - b * s, b * c + a * s])

    q = np.empty((bsz, num_q_heads, d))
    k = np.empty((bsz, num_kv_heads, d))
    for i in range(bsz):
        p = int(positions[i])
        for h in range(num_q_heads):
            q[i, h] = norm_rot(heads[i, h], qw, p)
        for g in range(num_kv_heads):
            k[i, g] = norm_rot(heads[i, num_q_heads + g], kw, p)
    v = heads[:, num_q_heads + num_kv_heads:].copy()
    return q, k, v
