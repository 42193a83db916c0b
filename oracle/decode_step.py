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

Rounding decisions at near-ties. Every "-> bf16" above is a rounding: a
floating-point value deciding which of two adjacent bf16 numbers is stored.
Where the exact (fp64) value lies within a small fraction of a bf16 ulp of the
midpoint between two neighbours, a kernel that evaluates it in fp32 may
legitimately land on the other side and store the other neighbour; one such
one-ulp difference then spreads through everything downstream. The decision
belongs to the kernel's precision, so ``step`` and ``layer`` can be given the
kernel's stored bf16 values (``tie``): at a rounding whose fp64 value is
within ``TIE_WINDOW`` ulp of a midpoint, and only there, the oracle stores the
kernel's neighbour instead of its own. Everywhere else its own rounding
stands, so a wrong value on the kernel's side is never adopted (it would have
to be the adjacent bf16 number of a value that sits on a midpoint).
"""
from __future__ import annotations

import numpy as np

from .bi_oracle import (addmm, bf16_bits_of, bf16_bits_to_f64, embed, mm, qknorm_rope, rmsnorm, round_bf16,
                        silu_mul)

__all__ = ["OracleDecoder", "LAYER_ROUNDINGS", "TIE_WINDOW", "round_at", "attend"]

# The stored bf16 activations of one layer, in the order the layer makes them.
LAYER_ROUNDINGS = ("h_in", "qkv", "q", "k", "att", "o", "x_mid", "h_mid", "gu", "act", "dn", "x_out", "h_out")

# Half-width of the near-tie window around a rounding midpoint, in bf16 ulps.
TIE_WINDOW = 2.0 ** -3


def round_at(u, kernel_bits=None, window: float = TIE_WINDOW):
    """round_bf16(u), with the near-tie decisions taken from the kernel.

    u: fp64 values to be stored as bf16. kernel_bits: the bf16 bit patterns
    the kernel stored for the same quantity (same shape), or None. Returns
    (stored values as fp64, number of decisions taken from the kernel).
    An element takes the kernel's value only when that value is the other
    neighbour of u (adjacent bf16 number: bit patterns one apart, same sign)
    and u lies within ``window`` ulp of the midpoint between the two.
    """
    u = np.asarray(u, dtype=np.float64)
    r = round_bf16(u)
    if kernel_bits is None:
        return r, 0
    kb = np.asarray(kernel_bits)
    if kb.shape != u.shape or kb.dtype != np.uint16:
        raise ValueError("kernel_bits must be uint16 bf16 patterns of u's shape")
    g = bf16_bits_to_f64(kb)
    rb = bf16_bits_of(np.where(np.isfinite(r), r, 0.0)).astype(np.int32)
    adjacent = (np.abs(rb - kb.astype(np.int32)) == 1) & np.isfinite(r) & np.isfinite(g) & (np.sign(r) == np.sign(g))
    mid = 0.5 * (r + g)
    spacing = np.abs(g - r)
    near = np.abs(u - mid) <= window * spacing
    take = adjacent & near
    return np.where(take, g, r), int(np.count_nonzero(take))


def attend(q, K, V, group: int):
    """out[h] = softmax(K[:, h // group] . q[h] / sqrt(D)) V[:, h // group]
    for one token; q [Hq, D], K and V [L, Hkv, D], all fp64."""
    hq, d = q.shape
    out = np.empty((hq, d))
    for hh in range(hq):
        g = hh // group
        sc = (K[:, g, :] @ q[hh]) / np.sqrt(d)
        p = np.exp(sc - sc.max())
        out[hh] = (p / p.sum()) @ V[:, g, :]
    return out


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

    After each ``step``, ``self.values`` maps (layer, name) to the fp64 value
    of each stored activation before its rounding (name in LAYER_ROUNDINGS,
    plus "v" for the appended values, copies of their qkv slice) and ``self.ties`` counts
    the decisions taken from the kernel.
    """

    def __init__(self, weights, layers: int, num_q_heads: int, num_kv_heads: int, eps: float, caches):
        self.w = weights
        self.layers = layers
        self.hq, self.hkv = num_q_heads, num_kv_heads
        self.eps = eps
        self.kv = [[(bf16_bits_to_f64(k).copy(), bf16_bits_to_f64(v).copy()) for (k, v) in seq] for seq in caches]
        self.values, self.ties = {}, {}

    def set_cache(self, s: int, l: int, k_bits, v_bits):
        """Replace sequence s's cached tokens of layer l ([L, Hkv, D] bf16 bits)."""
        self.kv[s][l] = (bf16_bits_to_f64(k_bits).copy(), bf16_bits_to_f64(v_bits).copy())

    def layer(self, l: int, x_bits, h_bits, seqs, tie=None, feed=None):
        """Layer l for one new token of each sequence in ``seqs``.

        x_bits, h_bits: the layer's input residual stream and its normalised
        form, bf16 bits [B, H]. The sequences' layer-l caches hold the tokens
        before this one; the token's k and v are appended. tie: optional dict
        name -> kernel bf16 bits, for the near-tie rule (module docstring).
        feed: optional dict name -> bf16 bits that replace the oracle's own
        stored value of that activation for everything after it (one op at a
        time against the kernel's own inputs). Returns (values, stored):
        dicts name -> fp64 before rounding, and name -> fp64 as stored; the
        stored "x_out" and "h_out" are the next layer's inputs.
        """
        w, eps, hq, hkv = self.w, self.eps, self.hq, self.hkv
        nk = bool(w.get("b_is_nk", False))
        bsz, d = len(seqs), 128
        group = hq // hkv
        tie, feed = tie or {}, feed or {}
        values, stored = {}, {}
        ties = self.ties

        def keep(name, u):
            values[name] = u
            if name in feed:
                s = bf16_bits_to_f64(feed[name])
            else:
                s, n = round_at(u, tie.get(name))
                ties[(l, name)] = ties.get((l, name), 0) + n
            stored[name] = s
            return bf16_bits_of(s)

        x = np.asarray(x_bits)
        h = np.asarray(h_bits)
        qkv = keep("qkv", mm(h, w["w_qkv"][l], b_is_nk=nk))
        pos = [len(self.kv[s][l][0]) for s in seqs]
        q, k, v = qknorm_rope(qkv, w["q_norm"][l], w["k_norm"][l], eps, w["cos"], w["sin"], pos, hq, hkv)
        keep("q", q)
        keep("k", k)
        # v is a copy of its slice of the stored qkv: its value before rounding
        # is that slice of qkv's
        values["v"] = values["qkv"].reshape(bsz, hq + 2 * hkv, d)[:, hq + hkv:]
        stored["v"] = bf16_bits_to_f64(feed["v"]) if "v" in feed else v
        att = np.empty((bsz, hq, d))
        for i, s in enumerate(seqs):
            K, V = self.kv[s][l]
            K = np.concatenate([K, stored["k"][i][None]])
            V = np.concatenate([V, stored["v"][i][None]])
            self.kv[s][l] = (K, V)
            att[i] = attend(stored["q"][i], K, V, group)
        att_b = keep("att", att.reshape(bsz, hq * d))
        o = keep("o", mm(att_b, w["w_o"][l], b_is_nk=nk))
        x_mid = keep("x_mid", bf16_bits_to_f64(x) + bf16_bits_to_f64(o))
        h_mid = keep("h_mid", rmsnorm(x_mid, w["w_post"][l], eps))
        gu = keep("gu", mm(h_mid, w["w_gu"][l], b_is_nk=nk))
        act = keep("act", silu_mul(gu))
        dn = keep("dn", mm(act, w["w_down"][l], b_is_nk=nk))
        x_out = keep("x_out", bf16_bits_to_f64(x_mid) + bf16_bits_to_f64(dn))
        w_next = w["w_in"][l + 1] if l + 1 < self.layers else w["w_final"]
        keep("h_out", rmsnorm(x_out, w_next, eps))
        return values, stored

    def step(self, tokens, seqs=None, tie=None):
        """Feed tokens[i] to sequence seqs[i] (default: all, in order); return
        fp64 logits [B, V]. tie: optional dict (layer, name) -> kernel bf16
        bits of this step's stored activations (near-tie rule); the name
        "h_in" of layer 0 is the first normalisation."""
        w, eps = self.w, self.eps
        nk = bool(w.get("b_is_nk", False))
        seqs = list(range(len(tokens))) if seqs is None else list(seqs)
        tie = tie or {}
        self.values, self.ties = {}, {}
        x = bf16_bits_of(round_bf16(embed(w["embed"], tokens)))
        u = rmsnorm(x, w["w_in"][0], eps)
        h, n = round_at(u, tie.get((0, "h_in")))
        self.values[(0, "h_in")], self.ties[(0, "h_in")] = u, n
        h = bf16_bits_of(h)
        for l in range(self.layers):
            lt = {name: b for (ll, name), b in tie.items() if ll == l}
            values, stored = self.layer(l, x, h, seqs, tie=lt)
            for name, val in values.items():
                self.values[(l, name)] = val
            x, h = bf16_bits_of(stored["x_out"]), bf16_bits_of(stored["h_out"])
        return addmm(w["b_lm"], h, w["w_lm"], b_is_nk=nk)
