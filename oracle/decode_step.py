"""fp64 oracle of one greedy decode step of a Qwen3-style model. TEST
INFRASTRUCTURE ONLY (see the package docstring).

The pages' evidence is a token stream: 1,000 temperature-0 completions of
one prompt, identical for 102 tokens and then forking (readhandoff.com,
agent-run reproducibility pinning, "Where the divergence showed up"), and
the cost of batch invariance is measured on Qwen3-8B decoding (same page,
"Key takeaways"). This module is the plain definition of the per-token
computation such a stream is made of, composed from the op definitions in
``bi_oracle``; it is the reference for the end-to-end decode-step test.

The layer (random weights; no checkpoint is involved):

    x   = embed(token)                                  residual stream, bf16
    h   = rmsnorm(x, w_in)                              -> bf16
    qkv = h @ W_qkv                                     -> bf16
    q, k, v = per-head q/k RMSNorm + rotary at the token's position
                                                        -> bf16; k, v appended
    a   = softmax(q . K^T / sqrt(D)) V over every cached token (GQA)
                                                        -> bf16
    x   = x + a @ W_o                                   (each GEMM -> bf16,
    h   = rmsnorm(x, w_post)                             the sum -> bf16)
    x   = x + (silu(g) * u) @ W_down, [g | u] = h @ W_gu
    next layer's h = rmsnorm(x, w_in'), or rmsnorm(x, w_final) after the last
    logits = h @ W_lm + b_lm                            (fp32 on the GPU)

Readings (the pages give no model code): activations are stored as bf16
between the steps above, which is where the rounding points are; every
weight matrix is stored [K, N] (the GEMM layout of the projection shapes);
the rotary table is an input; the gated activation and the q/k prologue are
each rounded once.
"""
from __future__ import annotations

import numpy as np

from .bi_oracle import (add_rmsnorm, addmm, bf16_bits_of, bf16_bits_to_f64, embed, mm, qknorm_rope, rmsnorm,
                        round_bf16, silu_mul)

__all__ = ["OracleDecoder"]


def _bits(v):
    return bf16_bits_of(round_bf16(v))


class OracleDecoder:
    """Greedy decoding of a few sequences, one token per step.

    weights: dict of numpy arrays (bf16 as uint16 bits, tables fp32):
      embed [V, H]; per layer l: w_in[l] [H], w_qkv[l] [H, (Hq + 2 Hkv) D],
      q_norm[l] [D], k_norm[l] [D], w_o[l] [Hq D, H], w_post[l] [H],
      w_gu[l] [H, 2 I], w_down[l] [I, H]; w_final [H]; w_lm [H, V];
      b_lm [V]; cos, sin [max_pos, D / 2]. The matrices are [K, N] as
      listed, or [N, K] (nn.Linear's layout, C = A B^T) when
      weights["b_is_nk"] is true.
    caches: per sequence, per layer, (K, V) bf16 bits [L, Hkv, D] of the
      tokens already cached (the prompt).
    """

    def __init__(self, weights, layers: int, num_q_heads: int, num_kv_heads: int, eps: float, caches):
        self.w = weights
        self.layers = layers
        self.hq, self.hkv = num_q_heads, num_kv_heads
        self.eps = eps
        self.kv = [[(bf16_bits_to_f64(k).copy(), bf16_bits_to_f64(v).copy()) for (k, v) in seq] for seq in caches]

    def step(self, tokens, seqs=None):
        """Feed tokens[i] to sequence seqs[i] (default: all, in order); return fp64 logits [B, V]."""
        w, eps, hq, hkv = self.w, self.eps, self.hq, self.hkv
        nk = bool(w.get("b_is_nk", False))
        seqs = list(range(len(tokens))) if seqs is None else list(seqs)
        bsz, d = len(tokens), 128
        group = hq // hkv
        x = _bits(embed(w["embed"], tokens))
        h = _bits(rmsnorm(x, w["w_in"][0], eps))
        for l in range(self.layers):
            qkv = _bits(mm(h, w["w_qkv"][l], b_is_nk=nk))
            pos = [len(self.kv[s][l][0]) for s in seqs]
            q, k, v = qknorm_rope(qkv, w["q_norm"][l], w["k_norm"][l], eps, w["cos"], w["sin"], pos, hq, hkv)
            q, k = round_bf16(q), round_bf16(k)
            att = np.empty((bsz, hq, d))
            for i, s in enumerate(seqs):
                K, V = self.kv[s][l]
                K = np.concatenate([K, k[i][None]])
                V = np.concatenate([V, v[i][None]])
                self.kv[s][l] = (K, V)
                for hh in range(hq):
                    g = hh // group
                    sc = (K[:, g, :] @ q[i, hh]) / np.sqrt(d)
                    p = np.exp(sc - sc.max())
                    att[i, hh] = (p / p.sum()) @ V[:, g, :]
            o = _bits(mm(_bits(att.reshape(bsz, hq * d)), w["w_o"][l], b_is_nk=nk))
            x, y = add_rmsnorm(x, o, w["w_post"][l], eps)
            h = _bits(y)
            gu = _bits(mm(h, w["w_gu"][l], b_is_nk=nk))
            dn = _bits(mm(_bits(silu_mul(gu)), w["w_down"][l], b_is_nk=nk))
            w_next = w["w_in"][l + 1] if l + 1 < self.layers else w["w_final"]
            x, y = add_rmsnorm(x, dn, w_next, eps)
            h = _bits(y)
        return addmm(w["b_lm"], h, w["w_lm"], b_is_nk=nk)
