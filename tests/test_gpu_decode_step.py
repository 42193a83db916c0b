"""The decode-step kernels and the end-to-end decode step, on the GPU.

Per kernel: parity with the fp64 oracle on the same seeded inputs (fp32
tolerances as for the other ops; bit-exact where the result is a copy or a
rounding both sides do in the same precision). End to end, on two layers of
the Qwen3-8B shape with the workload's weight draws: every stored activation,
the fp32 logits and the greedy token of the library's decode step against
``OracleDecoder`` (the whole chain from the same seeds, and each layer fed the
GPU's own layer input and cache), at the op tolerances; and one sequence's
logits, bit for bit, and greedy token stream in every batch composition --
the property whose absence the pages show as completions that fork after a
common prefix (readhandoff.com, agent-run reproducibility pinning, "Where the
divergence showed up").
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from helpers import ELEM_TOL, assert_close, bits, f32, same_bits
from oracle.decode_step import OracleDecoder

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def close_bf16(got, ref, what=""):
    """A bf16 output is one round-to-nearest of an fp32 value: relative error
    at most half a bf16 ulp, <= 2^-8 per element, so rel-Frobenius <= 2^-8;
    and the usual elementwise bound."""
    g = f32(got.float())
    fro, el = O.relative_frobenius(g, ref), O.elementwise_ratio(g, ref)
    assert fro <= 2.0 ** -8 and el <= ELEM_TOL, f"{what}: rel-Frobenius {fro:.3e}, elementwise {el:.3e}"


# ---------------------------------------------------------------- kernels
@pytest.mark.parametrize("m,n", [(1, 4096), (7, 4096), (64, 4104), (5, 20000)])
def test_add_rmsnorm_parity(lib, m, n):
    say(f"add_rmsnorm m={m} n={n}")
    x = S.normal_bf16((m, n), 1.0, seed=700 + m, device=DEV)
    d = S.normal_bf16((m, n), 1.0, seed=710 + m, device=DEV)
    w = S.uniform_bf16((n,), 0.5, 1.5, seed=720, device=DEV)
    x0 = x.clone()
    y = lib.bi_add_rmsnorm(x, d, w, 1e-6, out_dtype=torch.float32)
    # the residual: fp32 sum of the two bf16 values, rounded once (same precision as torch on the CPU)
    want_x = (x0.cpu().float() + d.cpu().float()).to(torch.bfloat16)
    assert same_bits(x.cpu(), want_x)
    ref_bits, ref_y = O.add_rmsnorm(bits(x0), bits(d), bits(w), 1e-6)
    assert np.abs(ref_bits.astype(np.int32) - bits(x).astype(np.int32)).max() <= 1  # <= 1 ulp from the exact sum
    assert_close(f32(y), O.rmsnorm(bits(x), bits(w), 1e-6), "add_rmsnorm vs rmsnorm(updated x)")
    assert_close(f32(y), ref_y, "add_rmsnorm vs oracle")
    # fused == unfused on the updated row, and the bf16 output is the RNE of the fp32 one
    assert same_bits(y, lib.bi_rmsnorm(x, w, 1e-6, out_dtype=torch.float32))
    x1 = x0.clone()
    yb = lib.bi_add_rmsnorm(x1, d, w, 1e-6)
    assert same_bits(yb.cpu(), y.cpu().to(torch.bfloat16)) and same_bits(x1, x)



def test_add_rmsnorm_row_shorter_than_a_chunk(lib):
    """n < 8: the row has no full 16-byte chunk, only the tail (rows padded to
    a stride of 8, as the alignment rule asks)."""
    m, n, ld = 3, 5, 8
    say("add_rmsnorm n=5")
    x = S.normal_bf16((m, ld), 1.0, seed=731, device=DEV)[:, :n]
    d = S.normal_bf16((m, ld), 1.0, seed=732, device=DEV)[:, :n]
    w = S.uniform_bf16((ld,), 0.5, 1.5, seed=733, device=DEV)[:n]
    x0 = x.clone()
    y = lib.bi_add_rmsnorm(x, d, w, 1e-6, out_dtype=torch.float32, out=torch.empty((m, ld), device=DEV)[:, :n])
    want_x = (x0.cpu().float() + d.cpu().float()).to(torch.bfloat16)
    assert same_bits(x.cpu(), want_x)
    assert_close(f32(y), O.add_rmsnorm(bits(x0), bits(d), bits(w), 1e-6)[1], "add_rmsnorm n=5 vs oracle")

def test_embed_is_an_exact_gather(lib):
    table = S.normal_bf16((1000, 4096), 1.0, seed=730, device=DEV)
    tok = torch.tensor([5, 999, 0, 5, -3, 1000, 123], dtype=torch.int64, device=DEV)
    out = lib.bi_embed(table, tok)
    for i, t in enumerate(tok.tolist()):
        if 0 <= t < 1000:
            assert same_bits(out[i], table[t])
        else:
            assert not out[i].any()


@pytest.mark.parametrize("m,n", [(1, 12288), (13, 12288), (4, 200)])
def test_silu_mul_parity(lib, m, n):
    gu = S.normal_bf16((m, 2 * n), 4.0, seed=740 + m, device=DEV)
    out = lib.bi_silu_mul(gu)
    ref = O.silu_mul(bits(gu))
    close_bf16(out, ref, "silu_mul")
    # the bf16 result is one rounding of the fp32 value: within half a bf16 ulp of the exact one,
    # plus the fp32 evaluation error
    got = f32(out.float()).astype(np.float64)
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
    assert np.all((rel <= 2.0 ** -8 + 1e-6) | (np.abs(ref) < 1e-30))


def _rope_case(b, hq, hkv, seed, max_pos=4096, pages=64, page=16):
    qkv = S.normal_bf16((b, (hq + 2 * hkv) * 128), 9.0, seed=seed, device=DEV)
    qw = S.uniform_bf16((128,), 0.5, 1.5, seed=seed + 1, device=DEV)
    kw = S.uniform_bf16((128,), 0.5, 1.5, seed=seed + 2, device=DEV)
    cos, sin = S.rope_tables(max_pos)
    g = torch.Generator().manual_seed(seed + 3)
    pos = torch.randint(0, 64 * page, (b,), generator=g, dtype=torch.int32)
    table = torch.randperm(pages, generator=g).to(torch.int32)[: b * 4].view(b, 4)
    return qkv, qw, kw, cos, sin, pos, table


def test_qknorm_rope_append_parity_and_cache_slots(lib):
    b, hq, hkv, page = 5, 32, 8, 16
    qkv, qw, kw, cos, sin, pos, table = _rope_case(b, hq, hkv, 750)
    pos = torch.tensor([0, 17, 63, 40, 5], dtype=torch.int32)  # within 4 pages of 16
    kp = torch.full((64, hkv, page, 128), 7.0, dtype=torch.bfloat16, device=DEV)  # sentinel
    vp = torch.full((64, hkv, 128, page), 7.0, dtype=torch.bfloat16, device=DEV)  # d-major
    q = lib.bi_qknorm_rope_append(qkv, qw, kw, cos.to(DEV), sin.to(DEV), pos.to(DEV), table.to(DEV), kp, vp,
                                  num_q_heads=hq, num_kv_heads=hkv, eps=1e-6)
    rq, rk, rv = O.qknorm_rope(bits(qkv), bits(qw), bits(kw), 1e-6, cos.numpy(), sin.numpy(), pos.numpy(), hq, hkv)
    close_bf16(q, rq, "q")
    touched = torch.zeros((64, page), dtype=torch.bool)
    for i in range(b):
        p, s = int(table[i, pos[i] // page]), int(pos[i] % page)
        touched[p, s] = True
        close_bf16(kp[p, :, s], rk[i], f"k of token {i}")
        assert same_bits(vp[p, :, :, s], qkv[i, (hq + hkv) * 128:].view(hkv, 128))
    sentinel = torch.full((hkv, 128), 7.0, dtype=torch.bfloat16)
    kc, vc = kp.cpu(), vp.cpu()
    for p in range(64):
        for s in range(page):
            if not touched[p, s]:
                assert same_bits(kc[p, :, s], sentinel) and same_bits(vc[p, :, :, s], sentinel)


def test_qknorm_rope_append_rejects_bad_positions_without_writing(lib):
    b, hq, hkv, page = 3, 8, 2, 16
    qkv, qw, kw, cos, sin, _, _ = _rope_case(b, hq, hkv, 760, max_pos=100)
    table = torch.tensor([[0, 1], [2, 3], [4, 99]], dtype=torch.int32)  # page 99 is outside the pool of 8
    pos = torch.tensor([100, -1, 20], dtype=torch.int32)  # past the table; negative; page 99
    kp = torch.full((8, hkv, page, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    vp = torch.full((8, hkv, 128, page), 3.0, dtype=torch.bfloat16, device=DEV)
    q = lib.bi_qknorm_rope_append(qkv, qw, kw, cos.to(DEV), sin.to(DEV), pos.to(DEV), table.to(DEV), kp, vp,
                                  num_q_heads=hq, num_kv_heads=hkv)
    assert not q.any()
    assert (kp == 3.0).all() and (vp == 3.0).all()


# ---------------------------------------------------------------- end to end
def make_weights(shape, layers, seed, device=DEV, max_pos=40000, qk_norm=(0.5, 1.5)):
    return S.qwen3_weights(shape.hidden, shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.intermediate,
                           shape.vocab, layers, seed, device=device, max_pos=max_pos, qk_norm=qk_norm)


def prompt_cache(shape, layers, length, seed):
    """A sequence's already-cached tokens (its prompt), per layer (K, V) bf16 [L, Hkv, D], from its seed."""
    return [(S.normal_bf16((length, shape.num_kv_heads, shape.head_dim), 1.0, seed=seed + 2 * l, device=DEV),
             S.normal_bf16((length, shape.num_kv_heads, shape.head_dim), 1.0, seed=seed + 2 * l + 1, device=DEV))
            for l in range(layers)]


def place(decoder, caches, lens, room, seed):
    """Block table with random physical pages for the given sequences (each
    with `room` free token slots), and their prompt caches written there."""
    from invariant_bi_mm_amd.decode import Batch
    ps = decoder.s.page_size
    need = [(L + room + ps - 1) // ps for L in lens]
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(decoder.k_pages[0].shape[0], generator=g)
    assert sum(need) <= len(perm)
    table = torch.zeros((len(lens), max(need)), dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    for b, (L, cache) in enumerate(zip(lens, caches)):
        if L == 0:
            continue
        t = torch.arange(L)
        pg, sl = table[b, t // ps].long().to(DEV), (t % ps).to(DEV)
        for l, (k, v) in enumerate(cache):
            decoder.k_pages[l][pg, :, sl] = k
            decoder.v_pages[l][pg, :, :, sl] = v  # d-major pages
    return Batch(block_table=table.to(DEV), lens=torch.tensor(lens, dtype=torch.int32))


def _np_weights(w):
    return {k: ([S.bf16_bits_numpy(t) for t in v] if isinstance(v, list) else
                v if not isinstance(v, torch.Tensor) else
                (S.bf16_bits_numpy(v) if v.dtype == torch.bfloat16 else v.cpu().numpy())) for k, v in w.items()}


def _gpu_cache(dec, batch, b, l, L):
    """Tokens 0..L-1 of sequence b in the GPU's layer-l cache, token-major bf16 bits [L, Hkv, D] (K, V)."""
    ps = dec.s.page_size
    t = torch.arange(L)
    pg, sl = batch.block_table[b, (t // ps).to(DEV)].long(), (t % ps).to(DEV)
    return bits(dec.k_pages[l][pg, :, sl]), bits(dec.v_pages[l][pg, :, :, sl])


class _Taps:
    """Copies of the stored activations of one GPU step, as bf16 bits, plus
    the k and v the step appended (read from the cache slots)."""

    def __init__(self):
        self.t = {}

    def __call__(self, l, name, tensor):
        self.t[(l, name)] = tensor.clone()

    def bits(self, dec, batch, lens_before):
        out = {key: bits(t) for key, t in self.t.items()}
        for l in range(dec.s.layers):
            kv = [_gpu_cache(dec, batch, b, l, L + 1) for b, L in enumerate(lens_before)]
            out[(l, "k")] = np.stack([k[-1] for k, _ in kv])
            out[(l, "v")] = np.stack([v[-1] for _, v in kv])
        out.update({(l, "q"): out[(l, "q")].reshape(len(lens_before), -1, 128) for l in range(dec.s.layers)})
        return out


def _check_activation(name, got_bits, ref, what):
    """A stored activation against the oracle's value before its rounding:
    bf16 values are one rounding of that value, so rel-Frobenius <= 2^-8 and
    the elementwise bound (v: its qkv slice's value)."""
    got = O.bf16_bits_to_f64(got_bits).reshape(ref.shape)
    fro, el = O.relative_frobenius(got, ref), O.elementwise_ratio(got, ref)
    assert fro <= 2.0 ** -8 and el <= ELEM_TOL, f"{what}: rel-Frobenius {fro:.3e}, elementwise {el:.3e}"
    return fro, el


def _check_greedy(nxt, ref_logits, what):
    """The greedy token against the oracle's logits (S8): equal to the oracle's
    argmax unless the oracle's top two are within the elementwise bound of
    each other, in which case any token of that near-tie set is correct."""
    for i in range(ref_logits.shape[0]):
        j, r = int(nxt[i]), ref_logits[i]
        top = r.max()
        near = np.flatnonzero(r >= top - ELEM_TOL * (abs(top) + 1.0))
        assert j in near, f"{what}: sequence {i} chose {j}, oracle {int(np.argmax(r))}"


QWEN_LENS = [1, 17, 300, 700]  # one page, a partial second page, two and three splits of 256


def _qwen_model(seed):
    from invariant_bi_mm_amd.decode import QWEN3_8B, Decoder
    import dataclasses
    shape = dataclasses.replace(QWEN3_8B, layers=2)
    w = make_weights(shape, 2, seed=seed, max_pos=2048)  # the workload's draws, q/k norm weights U(0.5, 1.5)
    caches = [prompt_cache(shape, 2, L, seed=seed + 100 + 10 * i) for i, L in enumerate(QWEN_LENS)]
    dec = Decoder(shape, w, num_pages=256)
    batch = place(dec, caches, QWEN_LENS, room=4, seed=seed + 200)
    npw = _np_weights(w)
    assert npw["b_is_nk"] is True  # the nn.Linear layout the decode step is benchmarked with
    ocaches = [[(S.bf16_bits_numpy(k), S.bf16_bits_numpy(v)) for (k, v) in c] for c in caches]
    return shape, dec, batch, npw, ocaches


def test_decode_step_chain_matches_oracle_qwen3_8b_shape(lib):
    """Two Qwen3-8B layers (hidden 4096, 32/8 heads, intermediate 12288,
    vocab 151936, the workload's weight draws) decoded for 3 teacher-forced
    tokens on the GPU and by OracleDecoder from the same seeds. Every stored
    activation of every layer is held to the bf16 tolerance against the
    oracle's value before its rounding, the fp32 logits to 1e-3 / 4e-3, and
    the greedy token to the oracle's choice. The oracle takes the kernel's
    rounding decision only at near-ties (within 1/8 ulp of a bf16 rounding
    midpoint, where fp32 and fp64 evaluation may fall on either side);
    nothing else of the GPU's reaches it."""
    from oracle.decode_step import OracleDecoder
    shape, dec, batch, npw, ocaches = _qwen_model(9000)
    orc = OracleDecoder(npw, 2, shape.num_q_heads, shape.num_kv_heads, shape.eps, ocaches)
    g = torch.Generator().manual_seed(9300)
    for step in range(3):
        tok = torch.randint(0, shape.vocab, (len(QWEN_LENS),), generator=g)
        lens_before = batch.lens.tolist()
        taps = _Taps()
        logits, _, nxt = dec.step(tok.to(DEV), batch, tap=taps)
        kb = taps.bits(dec, batch, lens_before)
        ref = orc.step(tok.numpy(), tie=kb)
        worst = 0.0
        for (l, name), u in orc.values.items():
            worst = max(worst, _check_activation(name, kb[(l, name)], u, f"step {step} layer {l} {name}")[1])
        fro, el = assert_close(f32(logits), ref, f"step {step} logits")
        _check_greedy(nxt.cpu(), ref, f"step {step}")
        say(f"step {step}: activations worst elementwise {worst:.2e}; logits rel-Frobenius {fro:.2e}, "
            f"elementwise {el:.2e}; near-tie decisions taken from the kernel {sum(orc.ties.values())}")


def test_decode_step_layerwise_teacher_forced_qwen3_8b_shape(lib):
    """Each layer of a GPU decode step against OracleDecoder's layer fed the
    GPU's own layer input (residual stream and its normalised form) and the
    cache the GPU holds: every output of the layer (the appended k and v, the
    new residual stream and its normalised form, and every activation in
    between) at the bf16 tolerance, near-tie rule as in the chain test. Then
    each op alone: the layer fed every GPU activation, so each op's output is
    compared with the oracle's op on the op's own GPU inputs. And the fp32
    logits against the oracle's LM head on the GPU's last normalised state."""
    from oracle.decode_step import LAYER_ROUNDINGS, OracleDecoder
    shape, dec, batch, npw, ocaches = _qwen_model(9050)
    g = torch.Generator().manual_seed(9350)
    for step in range(2):
        tok = torch.randint(0, shape.vocab, (len(QWEN_LENS),), generator=g)
        lens_before = batch.lens.tolist()
        caches = [[_gpu_cache(dec, batch, b, l, L) for l in range(2)] for b, L in enumerate(lens_before)]
        taps = _Taps()
        logits, _, nxt = dec.step(tok.to(DEV), batch, tap=taps)
        kb = taps.bits(dec, batch, lens_before)
        assert np.array_equal(kb[(0, "x_in")], O.bf16_bits_of(O.embed(npw["embed"], tok.numpy())))
        for l in range(2):
            x_in = kb[(0, "x_in")] if l == 0 else kb[(l - 1, "x_out")]
            h_in = kb[(0, "h_in")] if l == 0 else kb[(l - 1, "h_out")]
            mine = {name: kb[(l, name)] for name in LAYER_ROUNDINGS[1:] + ("v",)}
            for mode in ("layer", "op"):
                orc = OracleDecoder(npw, 2, shape.num_q_heads, shape.num_kv_heads, shape.eps, caches)
                if mode == "layer":
                    vals, _ = orc.layer(l, x_in, h_in, list(range(len(QWEN_LENS))), tie=mine)
                else:
                    vals, _ = orc.layer(l, x_in, h_in, list(range(len(QWEN_LENS))), feed=mine)
                worst = max(_check_activation(name, mine[name], vals[name], f"step {step} layer {l} {mode} {name}")[1]
                            for name in vals)
                say(f"step {step} layer {l} ({mode}): worst elementwise {worst:.2e}, "
                    f"near-tie decisions {sum(orc.ties.values())}")
        ref = O.addmm(npw["b_lm"], kb[(1, "h_out")], npw["w_lm"], b_is_nk=True)
        fro, el = assert_close(f32(logits), ref, f"step {step} logits")
        _check_greedy(nxt.cpu(), ref, f"step {step}")
        assert nxt.cpu().tolist() == O.argmax(f32(logits)).tolist()


def test_decode_token_stream_is_batch_invariant_qwen3_8b_shape(lib):
    """One sequence, greedy, 6 tokens, inside three batch compositions."""
    from invariant_bi_mm_amd.decode import QWEN3_8B, Decoder
    import dataclasses
    layers = 2
    shape = dataclasses.replace(QWEN3_8B, layers=layers)
    w = make_weights(shape, layers, seed=9500)
    target_len, steps = 700, 6
    target = prompt_cache(shape, layers, target_len, seed=9600)
    dec = Decoder(shape, w, num_pages=8192)
    runs = []
    for comp, (bsz, pos, seed) in enumerate([(1, 0, 1), (8, 3, 2), (33, 32, 3)]):
        lens = S.context_lens(bsz, seed=9700 + seed, hi=4096).tolist()
        lens[pos] = target_len
        caches = [prompt_cache(shape, layers, L, seed=9800 + 100 * seed + 7 * b) if b != pos else target
                  for b, L in enumerate(lens)]
        batch = place(dec, caches, lens, room=steps + 1, seed=9900 + seed)
        g = torch.Generator().manual_seed(10000 + seed)
        tok = torch.randint(0, shape.vocab, (bsz,), generator=g)
        tok[pos] = 42
        tok = tok.to(DEV)
        stream, rows = [], []
        for _ in range(steps):
            logits, logp, nxt = dec.step(tok, batch)
            rows.append((logits[pos].clone(), logp[pos].clone()))
            stream.append(int(nxt[pos]))
            tok = nxt.clone()
        say(f"composition {comp}: batch {bsz}, position {pos}: stream {stream}")
        runs.append((stream, rows))
    for stream, rows in runs[1:]:
        assert stream == runs[0][0]
        for (l0, p0), (l1, p1) in zip(runs[0][1], rows):
            assert same_bits(l0, l1) and same_bits(p0, p1)


def test_per_token_kernels_are_batch_invariant(lib):
    """A fixed row through add_rmsnorm, silu_mul, embed and the q/k prologue alone and inside
    batches of other random rows, at several positions: identical bytes."""
    n = 4096
    row_x = S.normal_bf16((1, n), 1.0, seed=800, device=DEV)
    row_d = S.normal_bf16((1, n), 1.0, seed=801, device=DEV)
    row_gu = S.normal_bf16((1, 2 * 12288), 4.0, seed=802, device=DEV)
    w = S.uniform_bf16((n,), 0.5, 1.5, seed=803, device=DEV)
    x1 = row_x.clone()
    y1 = lib.bi_add_rmsnorm(x1, row_d, w)
    s1 = lib.bi_silu_mul(row_gu)
    table = S.normal_bf16((5000, n), 1.0, seed=804, device=DEV)
    e1 = lib.bi_embed(table, torch.tensor([4321], dtype=torch.int64, device=DEV))
    for m in (2, 7, 64, 300):
        for pos in (0, m // 2, m - 1):
            x = S.normal_bf16((m, n), 1.0, seed=810 + m, device=DEV)
            d = S.normal_bf16((m, n), 1.0, seed=820 + m, device=DEV)
            gu = S.normal_bf16((m, 2 * 12288), 4.0, seed=830 + m, device=DEV)
            x[pos], d[pos], gu[pos] = row_x[0], row_d[0], row_gu[0]
            y = lib.bi_add_rmsnorm(x, d, w)
            assert same_bits(y[pos], y1[0]) and same_bits(x[pos], x1[0])
            assert same_bits(lib.bi_silu_mul(gu)[pos], s1[0])
            tok = torch.randint(0, 5000, (m,), generator=torch.Generator().manual_seed(m)).to(DEV)
            tok[pos] = 4321
            assert same_bits(lib.bi_embed(table, tok)[pos], e1[0])


def test_graph_replay_equals_eager_steps(lib):
    """The decode step captured once as a HIP graph and replayed step after step (eager host work and
    a synchronisation between replays) gives every step's logits and tokens the eager step's bits,
    also across a step where a sequence's split count grows under the same capture."""
    from invariant_bi_mm_amd.decode import Decoder, Qwen3Shape
    shape = Qwen3Shape(hidden=1024, num_q_heads=8, num_kv_heads=2, intermediate=3072, vocab=8192, layers=2)
    w = make_weights(shape, 2, seed=9400, max_pos=1024)
    lens = [254, 17, 300]  # sequence 0 reaches a second split at its third new token
    caches = [prompt_cache(shape, 2, L, seed=9410 + 10 * i) for i, L in enumerate(lens)]
    runs = []
    for mode in ("eager", "graph"):
        dec = Decoder(shape, w, num_pages=64)
        batch = place(dec, caches, lens, room=6, seed=9420)
        tok = torch.tensor([5, 77, 8000], dtype=torch.int64, device=DEV)
        outs = []
        gs = dec.graph(batch, 5) if mode == "graph" else None
        for i in range(5):
            if gs is None:
                logits, _, nxt = dec.step(tok, batch)
                tok = nxt
            else:
                logits, _, nxt = gs.run(tok if i == 0 else None)
            outs.append((logits.clone(), nxt.clone()))
        runs.append(outs)
    for i, ((l0, n0), (l1, n1)) in enumerate(zip(*runs)):
        assert same_bits(l0, l1) and same_bits(n0, n1), f"step {i}"
