"""One greedy decode step of a Qwen3-style model, end to end on the library.

The pages assess batch invariance by a token stream: temperature-0
completions of one prompt that agree for a long prefix and then fork,
because the batch a request lands in changes the kernels' reduction order
(readhandoff.com, agent-run reproducibility pinning, sections "What does
temperature zero actually guarantee?" and "Where the divergence showed
up"); the cost is measured on Qwen3-8B decoding ("Key takeaways"). This
module chains the library's kernels into that per-token computation so a
sequence's stream can be checked bit for bit across batch compositions.

Per layer (activations bf16, weights bf16 stored [K, N] or, with the
weights' "b_is_nk" flag, [N, K] as nn.Linear keeps them; fp32 accumulation):

    h = rmsnorm(x)                          bi_rmsnorm / bi_add_rmsnorm
    qkv = h @ W_qkv                         bi_mm
    q -> q_out; k, v -> paged cache         bi_qknorm_rope_append
    a = attention(q, cache)                 bi_decode_attention (split 256)
    x += a @ W_o ; h = rmsnorm(x)           bi_mm, bi_add_rmsnorm
    x += silu(g) * u @ W_down               bi_mm, bi_silu_mul, bi_mm
then logits = rmsnorm(x) @ W_lm + b_lm (bi_addmm, fp32), log-probabilities
and the greedy token (bi_log_softmax). Every arithmetic step runs in the HIP
kernels; torch only allocates and moves the few host-side plan integers
(context lengths, split offsets) to the device.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (bi_add_rmsnorm, bi_addmm, bi_decode_attention, bi_decode_plan, bi_decode_workspace_bytes, bi_embed,
               bi_log_softmax, bi_mm, bi_qknorm_rope_append, bi_rmsnorm, bi_silu_mul)

__all__ = ["Qwen3Shape", "QWEN3_8B", "Batch", "Decoder", "GraphStep"]


@dataclasses.dataclass(frozen=True)
class Qwen3Shape:
    hidden: int = 4096
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    intermediate: int = 12288
    vocab: int = 151936
    layers: int = 36
    eps: float = 1e-6
    page_size: int = 16
    split_tokens: int = 256


QWEN3_8B = Qwen3Shape()


@dataclasses.dataclass
class Batch:
    """The sequences of one step: their block tables (device int32
    [B, max_pages], into the decoder's page pool) and how many tokens each
    has cached before this step (host int32 [B])."""
    block_table: torch.Tensor
    lens: torch.Tensor


class Decoder:
    """Holds the weights and the paged KV cache (one page pool per layer).

    weights: dict of device tensors, bf16 unless noted: embed [V, H];
    lists over layers of w_in [H], w_qkv [H, (Hq + 2 Hkv) D], q_norm [D],
    k_norm [D], w_o [Hq D, H], w_post [H], w_gu [H, 2 I], w_down [I, H];
    w_final [H]; w_lm [H, V]; b_lm [V]; cos, sin fp32 [max_pos, D / 2].
    The matrices are given [K, N] as listed, or transposed ([N, K], the
    nn.Linear layout) when weights["b_is_nk"] is true.
    """

    def __init__(self, shape: Qwen3Shape, weights: dict, num_pages: int, device="cuda"):
        s = shape
        if s.num_q_heads * s.head_dim != s.hidden:
            raise ValueError("hidden must equal num_q_heads * head_dim")
        self.s, self.w = s, weights
        self.k_pages = [torch.empty((num_pages, s.num_kv_heads, s.page_size, s.head_dim), dtype=torch.bfloat16,
                                    device=device) for _ in range(s.layers)]
        # V pages d-major [P, Hkv, D, page], the layout bi_decode_attention reads
        self.v_pages = [torch.empty((num_pages, s.num_kv_heads, s.head_dim, s.page_size), dtype=torch.bfloat16,
                                    device=device) for _ in range(s.layers)]
        self.device = device

    def _layers(self, x, positions, lens_dev, offs_dev, total, ws, block_table, tap=None):
        """The kernels of one step after the embedding; returns (logits, log-probs, greedy tokens).

        tap: optional callable tap(layer, name, tensor), called in stream
        order right after each stored activation is produced (names: x_in and
        h_in of layer 0, then per layer qkv, q, att, o, x_mid, h_mid, gu, act, dn,
        x_out, h_out; the residual x is updated in place, so a tap that keeps
        a value must copy it). For tests that compare every step of the chain."""
        s, w = self.s, self.w
        nk = bool(w.get("b_is_nk", False))
        bsz = x.shape[0]
        h = bi_rmsnorm(x, w["w_in"][0], s.eps)
        if tap:
            tap(0, "x_in", x)
            tap(0, "h_in", h)
        for l in range(s.layers):
            qkv = bi_mm(h, w["w_qkv"][l], b_is_nk=nk, out_dtype=torch.bfloat16)
            q = bi_qknorm_rope_append(qkv, w["q_norm"][l], w["k_norm"][l], w["cos"], w["sin"], positions,
                                      block_table, self.k_pages[l], self.v_pages[l],
                                      num_q_heads=s.num_q_heads, num_kv_heads=s.num_kv_heads, eps=s.eps)
            a = bi_decode_attention(q, self.k_pages[l], self.v_pages[l], block_table, lens_dev, offs_dev, total,
                                    workspace=ws, out_dtype=torch.bfloat16, split_tokens=s.split_tokens,
                                    stream_kv=True)
            o = bi_mm(a.view(bsz, s.hidden), w["w_o"][l], b_is_nk=nk, out_dtype=torch.bfloat16)
            if tap:
                for name, t in (("qkv", qkv), ("q", q), ("att", a.view(bsz, s.hidden)), ("o", o)):
                    tap(l, name, t)
            h = bi_add_rmsnorm(x, o, w["w_post"][l], s.eps)
            if tap:
                tap(l, "x_mid", x)
                tap(l, "h_mid", h)
            gu = bi_mm(h, w["w_gu"][l], b_is_nk=nk, out_dtype=torch.bfloat16)
            act = bi_silu_mul(gu)
            dn = bi_mm(act, w["w_down"][l], b_is_nk=nk, out_dtype=torch.bfloat16)
            h = bi_add_rmsnorm(x, dn, w["w_in"][l + 1] if l + 1 < s.layers else w["w_final"], s.eps)
            if tap:
                for name, t in (("gu", gu), ("act", act), ("dn", dn), ("x_out", x), ("h_out", h)):
                    tap(l, name, t)
        logits = bi_addmm(w["b_lm"], h, w["w_lm"], b_is_nk=nk)
        logp, nxt = bi_log_softmax(logits)
        return logits, logp, nxt

    def graph(self, batch: Batch, max_steps: int) -> "GraphStep":
        """Capture one step of this batch as a HIP graph that can be replayed
        for up to max_steps successive steps (see GraphStep)."""
        return GraphStep(self, batch, max_steps)

    def step(self, tokens: torch.Tensor, batch: Batch, tap=None):
        """Run one token per sequence. tokens: device int64 [B]. Appends the
        tokens' k, v to the cache and advances batch.lens. Returns (fp32
        logits [B, V], fp32 log-probabilities [B, V], greedy tokens int64 [B]).
        tap: see _layers."""
        s, w = self.s, self.w
        bsz = tokens.shape[0]
        dev = self.device
        lens_after = batch.lens + 1
        if int(lens_after.max()) > batch.block_table.shape[1] * s.page_size:
            raise ValueError("a sequence has no page left for the new token")
        positions = batch.lens.to(dev, non_blocking=False)
        offs, total = bi_decode_plan(lens_after, s.split_tokens)
        lens_dev = lens_after.to(dev)
        offs_dev = offs.to(dev)
        ws = torch.empty(bi_decode_workspace_bytes(total, s.num_q_heads, s.head_dim), dtype=torch.uint8, device=dev)

        x = bi_embed(w["embed"], tokens)
        logits, logp, nxt = self._layers(x, positions, lens_dev, offs_dev, total, ws, batch.block_table, tap)
        batch.lens = lens_after
        return logits, logp, nxt


class GraphStep:
    """A decode step of one batch captured once and replayed step after step.

    A step launches ~10 kernels per layer; replaying them as one HIP graph
    removes the host launch cost between them. What changes from step to
    step lives in fixed device buffers that the host refreshes before each
    replay: the tokens (the previous replay writes its greedy tokens there),
    the positions, the context lengths and the split offsets. The attention
    launches cover an upper bound of the split count over max_steps steps;
    workgroups past the current count exit at once, so every replay does the
    same work as an eager step and gives the same bits.
    """

    def __init__(self, decoder: Decoder, batch: Batch, max_steps: int):
        s = decoder.s
        dev = decoder.device
        self.dec, self.batch, self.left = decoder, batch, max_steps
        bsz = batch.block_table.shape[0]
        if int((batch.lens + max_steps).max()) > batch.block_table.shape[1] * s.page_size:
            raise ValueError("the block table has no room for max_steps more tokens")
        lens_max = (batch.lens.to(torch.int64) + max_steps)
        self.bound = int(((lens_max + s.split_tokens - 1) // s.split_tokens).sum())
        self.tokens = torch.zeros(bsz, dtype=torch.int64, device=dev)
        self.positions = torch.zeros(bsz, dtype=torch.int32, device=dev)
        self.lens_dev = torch.ones(bsz, dtype=torch.int32, device=dev)
        self.offs_dev = torch.zeros(bsz + 1, dtype=torch.int32, device=dev)
        self._host = torch.empty(3 * bsz + 1, dtype=torch.int32, pin_memory=True)
        self.ws = torch.empty(bi_decode_workspace_bytes(self.bound, s.num_q_heads, s.head_dim), dtype=torch.uint8,
                              device=dev)
        self._set(batch.lens)  # valid contents for the capture's argument checks
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            x = bi_embed(decoder.w["embed"], self.tokens)
            self.logits, self.logp, nxt = decoder._layers(x, self.positions, self.lens_dev, self.offs_dev,
                                                          self.bound, self.ws, batch.block_table)
            self.tokens.copy_(nxt)

    def _set(self, lens: torch.Tensor):
        bsz = lens.shape[0]
        lens_after = lens + 1
        offs, _ = bi_decode_plan(lens_after, self.dec.s.split_tokens)
        h = self._host
        h[:bsz] = lens
        h[bsz:2 * bsz] = lens_after
        h[2 * bsz:] = offs
        self.positions.copy_(h[:bsz], non_blocking=True)
        self.lens_dev.copy_(h[bsz:2 * bsz], non_blocking=True)
        self.offs_dev.copy_(h[2 * bsz:], non_blocking=True)

    def run(self, tokens: torch.Tensor | None = None):
        """One step. tokens (device int64 [B]) for the first step; later steps
        take the previous step's greedy tokens. Returns the graph's (logits,
        log-probabilities, tokens) buffers, overwritten by the next replay."""
        if self.left <= 0:
            raise RuntimeError("captured for fewer steps: capture again")
        torch.cuda.current_stream().synchronize()  # the pinned staging buffer is reused
        if tokens is not None:
            self.tokens.copy_(tokens)
        self._set(self.batch.lens)
        self.g.replay()
        self.batch.lens = self.batch.lens + 1
        self.left -= 1
        return self.logits, self.logp, self.tokens
