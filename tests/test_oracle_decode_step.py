"""Pins for the oracle's decode-step functions (round_bf16, embed,
add_rmsnorm, silu_mul, qknorm_rope, OracleDecoder), against closed forms,
independent formulas and invariants. CPU only.

Each pin is chosen so a plausible slip fails it: rounding ties to the wrong
side, gate and up swapped, the rotation's sign or pairing wrong, the norm
applied with the wrong weight, a residual dropped, a head mapped to the
wrong kv head.
"""
import math

import numpy as np
import pytest

import oracle as O
from oracle.decode_step import OracleDecoder
from helpers import d_major


def bits(x):
    f = np.asarray(x, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f)
    return b


def rand_bf16(rng, shape, scale=1.0):
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------------------ round_bf16
def test_round_bf16_ties_and_exact_values():
    one = 1.0
    ulp = 2.0 ** -7  # bf16 spacing in [1, 2)
    got = O.round_bf16([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, one + 3 * ulp / 4, -(one + ulp / 2),
                        2.0 ** 100 * (one + ulp / 2), 3.0, 0.0])
    assert list(got) == [1.0, 1.0 + 2 * ulp, 1.0, 1.0 + ulp, -1.0, 2.0 ** 100, 3.0, 0.0]
    assert O.round_bf16([3.4e38])[0] == math.inf and O.round_bf16([-3.4e38])[0] == -math.inf


def test_round_bf16_matches_integer_rounding_of_fp32():
    # an independent definition: RNE on the fp32 bit pattern (add 0x7fff plus the
    # kept lsb, drop 16 bits), valid for finite fp32 values
    rng = np.random.default_rng(0)
    f = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    ref = (r << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(O.round_bf16(f.astype(np.float64)), ref)
    assert np.array_equal(O.bf16_bits_of(ref), r.astype(np.uint16))


# ------------------------------------------------------------------ embed
def test_embed_gathers_rows_and_zeroes_bad_tokens():
    table = bits(np.arange(5 * 8, dtype=np.float32).reshape(5, 8))
    out = O.embed(table, [3, 0, 7, -1, 3])
    assert np.array_equal(out[0], np.arange(24, 32)) and np.array_equal(out[1], np.arange(8))
    assert not out[2].any() and not out[3].any() and np.array_equal(out[4], out[0])


# ------------------------------------------------------------------ add_rmsnorm
def test_add_rmsnorm_zero_delta_is_rmsnorm_and_residual_is_rounded():
    rng = np.random.default_rng(1)
    x, w = rand_bf16(rng, (3, 64)), rand_bf16(rng, (64,))
    xb, y = O.add_rmsnorm(x, np.zeros_like(x), w, 1e-6)
    assert np.array_equal(xb, x) and np.allclose(y, O.rmsnorm(x, w, 1e-6), rtol=0, atol=0)
    # constant rows: x = 1, d = 2^-8 (a tie: 1 + 2^-8 rounds to even, 1.0) and d = 0.75
    xb, y = O.add_rmsnorm(bits(np.ones((2, 16))), bits(np.array([[2.0 ** -8] * 16, [0.75] * 16])),
                          bits(np.full(16, 2.0)), 0.0)
    assert np.array_equal(O.bf16_bits_to_f64(xb), np.array([[1.0] * 16, [1.75] * 16]))
    assert np.allclose(y, 2.0)  # w * c / |c| with eps = 0


# ------------------------------------------------------------------ silu_mul
def test_silu_mul_closed_forms_and_gate_up_order():
    g = np.array([[0.0, 1.0, -1.0, 20.0, -20.0, 2.0]], dtype=np.float32)
    u = np.array([[5.0, 1.0, 1.0, 1.0, 1.0, 0.5]], dtype=np.float32)
    out = O.silu_mul(bits(np.concatenate([g, u], axis=1)))[0]
    sig1 = 1.0 / (1.0 + math.exp(-1.0))
    assert out[0] == 0.0
    assert math.isclose(out[1], sig1, rel_tol=1e-15)
    assert math.isclose(out[1] - out[2], 1.0, rel_tol=1e-15)  # silu(x) - silu(-x) = x
    assert math.isclose(out[3], 20.0, rel_tol=1e-8) and abs(out[4]) < 1e-7
    assert math.isclose(out[5], 0.5 * 2.0 / (1.0 + math.exp(-2.0)), rel_tol=1e-15)


# ------------------------------------------------------------------ qknorm_rope
def _qkv(rng, b, hq, hkv):
    return rand_bf16(rng, (b, (hq + 2 * hkv) * 128))


def test_qknorm_rope_identity_rotation_is_per_head_rmsnorm():
    rng = np.random.default_rng(2)
    hq, hkv = 4, 1
    qkv = _qkv(rng, 2, hq, hkv)
    qw, kw = rand_bf16(rng, (128,)), rand_bf16(rng, (128,))
    cos, sin = np.ones((4, 64)), np.zeros((4, 64))
    q, k, v = O.qknorm_rope(qkv, qw, kw, 1e-6, cos, sin, [0, 3], hq, hkv)
    heads = O.bf16_bits_to_f64(qkv).reshape(2, hq + 2 * hkv, 128)
    for b in range(2):
        for h in range(hq):
            assert np.allclose(q[b, h], O.rmsnorm(O.bf16_bits_of(heads[b, h])[None], qw, 1e-6)[0], rtol=1e-14)
        assert np.allclose(k[b, 0], O.rmsnorm(O.bf16_bits_of(heads[b, hq])[None], kw, 1e-6)[0], rtol=1e-14)
        assert np.array_equal(v[b, 0], heads[b, hq + 1])


def test_qknorm_rope_one_hot_closed_form_and_sign():
    # x = e_j (q head 0), w = 1: t_j = 1 / sqrt(1/128 + eps); rotation by a
    # sends (t, 0) at pair (j, j+64) to (t cos a, t sin a) and (0, t) at pair
    # (j-64, j) to (-t sin a, t cos a)
    hq, hkv, eps = 4, 1, 1e-6
    t = 1.0 / math.sqrt(1.0 / 128 + eps)
    a = 0.7
    cos, sin = np.full((2, 64), math.cos(a)), np.full((2, 64), math.sin(a))
    ones = bits(np.ones(128))
    for j in (5, 70):
        x = np.zeros((1, (hq + 2 * hkv) * 128), dtype=np.float32)
        x[0, j] = 1.0
        q, _, _ = O.qknorm_rope(bits(x), ones, ones, eps, cos, sin, [1], hq, hkv)
        want = np.zeros(128)
        if j < 64:
            want[j], want[j + 64] = t * math.cos(a), t * math.sin(a)
        else:
            want[j - 64], want[j] = -t * math.sin(a), t * math.cos(a)
        assert np.allclose(q[0, 0], want, rtol=0, atol=1e-13)


def test_qknorm_rope_composes_and_preserves_pair_norms():
    rng = np.random.default_rng(3)
    hq, hkv = 4, 1
    qkv = _qkv(rng, 1, hq, hkv)
    ones = bits(np.ones(128))
    ang = rng.uniform(-3, 3, 64)
    tab = lambda p: (np.cos(p * ang)[None].repeat(4, 0), np.sin(p * ang)[None].repeat(4, 0))  # noqa: E731
    c1, s1 = tab(1.0)
    c2, s2 = tab(2.0)
    q1, _, _ = O.qknorm_rope(qkv, ones, ones, 0.0, c1, s1, [0], hq, hkv)
    q2, _, _ = O.qknorm_rope(qkv, ones, ones, 0.0, c2, s2, [0], hq, hkv)
    q0, _, _ = O.qknorm_rope(qkv, ones, ones, 0.0, np.ones((1, 64)), np.zeros((1, 64)), [0], hq, hkv)
    # rotating the once-rotated vector by the same angles again equals rotating by twice the angles
    r = q1[0, 2]
    twice = np.concatenate([r[:64] * c1[0] - r[64:] * s1[0], r[64:] * c1[0] + r[:64] * s1[0]])
    assert np.allclose(twice, q2[0, 2], rtol=0, atol=1e-12)
    pn = lambda z: z[:64] ** 2 + z[64:] ** 2  # noqa: E731
    assert np.allclose(pn(q1[0, 1]), pn(q0[0, 1]), rtol=1e-12)


# ------------------------------------------------------------------ decode step
def _tiny_weights(rng, layers=1, hq=4, hkv=1, inter=64, vocab=32, max_pos=16, zero_blocks=False):
    hdim = hq * 128
    r = lambda *s, sc=0.05: rand_bf16(rng, s, sc)  # noqa: E731
    w = {"embed": r(vocab, hdim, sc=1.0), "w_in": [r(hdim, sc=1.0) for _ in range(layers)],
         "w_qkv": [r(hdim, (hq + 2 * hkv) * 128) for _ in range(layers)],
         "q_norm": [r(128, sc=1.0) for _ in range(layers)], "k_norm": [r(128, sc=1.0) for _ in range(layers)],
         "w_o": [r(hq * 128, hdim) for _ in range(layers)], "w_post": [r(hdim, sc=1.0) for _ in range(layers)],
         "w_gu": [r(hdim, 2 * inter) for _ in range(layers)], "w_down": [r(inter, hdim) for _ in range(layers)],
         "w_final": r(hdim, sc=1.0), "w_lm": r(hdim, vocab), "b_lm": r(vocab, sc=0.1)}
    ang = np.arange(max_pos)[:, None] * (1e6 ** (-np.arange(64) / 64.0))[None]
    w["cos"], w["sin"] = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    if zero_blocks:
        w["w_o"] = [np.zeros_like(x) for x in w["w_o"]]
        w["w_down"] = [np.zeros_like(x) for x in w["w_down"]]
    return w


def test_decoder_with_silent_blocks_is_norm_then_head():
    # with W_o = W_down = 0 the residual stream stays the embedding, so the
    # logits are rmsnorm(embed(token), w_final) @ W_lm + b (rounded where the
    # model rounds); this pins the residual wiring and the final norm
    rng = np.random.default_rng(4)
    w = _tiny_weights(rng, layers=2, zero_blocks=True)
    caches = [[(rand_bf16(rng, (3, 1, 128)), rand_bf16(rng, (3, 1, 128))) for _ in range(2)] for _ in range(2)]
    dec = OracleDecoder(w, 2, 4, 1, 1e-6, caches)
    got = dec.step(np.array([5, 9]))
    x = O.bf16_bits_of(O.embed(w["embed"], [5, 9]))
    h = O.bf16_bits_of(O.round_bf16(O.rmsnorm(x, w["w_final"], 1e-6)))
    assert np.allclose(got, O.addmm(w["b_lm"], h, w["w_lm"]), rtol=1e-14, atol=0)
    assert all(len(dec.kv[s][l][0]) == 4 for s in range(2) for l in range(2))  # one token appended


def test_decoder_rows_are_independent_and_one_token_cache_attends_to_itself():
    rng = np.random.default_rng(5)
    w = _tiny_weights(rng, layers=1)
    caches = [[(rand_bf16(rng, (L, 1, 128)), rand_bf16(rng, (L, 1, 128)))] for L in (0, 6)]
    both = OracleDecoder(w, 1, 4, 1, 1e-6, caches).step(np.array([1, 2]))
    alone = OracleDecoder(w, 1, 4, 1, 1e-6, caches[1:]).step(np.array([2]))
    assert np.array_equal(both[1], alone[0])
    # an empty prompt cache: attention over the single new token returns its own v
    d1 = OracleDecoder(w, 1, 4, 1, 1e-6, caches[:1])
    x = O.bf16_bits_of(O.embed(w["embed"], [1]))
    h = O.bf16_bits_of(O.round_bf16(O.rmsnorm(x, w["w_in"][0], 1e-6)))
    qkv = O.bf16_bits_of(O.round_bf16(O.mm(h, w["w_qkv"][0])))
    d1.step(np.array([1]))
    assert np.array_equal(d1.kv[0][0][1][0, 0], O.bf16_bits_to_f64(qkv)[0, 5 * 128:6 * 128])



def test_decoder_nn_linear_layout_gives_the_same_logits():
    # the same model with every matrix stored transposed ([N, K], nn.Linear's
    # layout) and the b_is_nk flag set must decode to the same logits: pins
    # that the oracle applies the flag to every projection and the LM head
    rng = np.random.default_rng(6)
    w = _tiny_weights(rng, layers=2)
    wt = dict(w, b_is_nk=True)
    for k in ("w_qkv", "w_o", "w_gu", "w_down"):
        wt[k] = [np.ascontiguousarray(x.T) for x in w[k]]
    wt["w_lm"] = np.ascontiguousarray(w["w_lm"].T)
    caches = [[(rand_bf16(rng, (L, 1, 128)), rand_bf16(rng, (L, 1, 128))) for _ in range(2)] for L in (2, 7)]
    a, b = OracleDecoder(w, 2, 4, 1, 1e-6, caches), OracleDecoder(wt, 2, 4, 1, 1e-6, caches)
    for toks in ([3, 11], [30, 0]):
        la, lb = a.step(np.array(toks)), b.step(np.array(toks))
        assert np.allclose(la, lb, rtol=1e-12, atol=1e-12)
    # [K, N] weights flagged [N, K] are rejected (q+kv's inner dimension no longer matches)
    with pytest.raises(ValueError):
        OracleDecoder(dict(w, b_is_nk=True), 2, 4, 1, 1e-6, caches).step(np.array([3, 11]))

# ------------------------------------------------------------------ near-tie rounding decisions
def test_round_at_takes_the_kernel_neighbour_only_at_near_ties():
    from oracle.decode_step import TIE_WINDOW, round_at
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    mid = 1.0 + ulp / 2                   # midpoint between 1 and 1 + ulp
    w = TIE_WINDOW * ulp
    one, up = bits(np.array([1.0])), bits(np.array([1.0 + ulp]))
    # on the midpoint: RNE gives 1.0 (even); a kernel that stored 1 + ulp is adopted
    got, n = round_at(np.array([mid]), up)
    assert got[0] == 1.0 + ulp and n == 1
    # just above the midpoint, inside the window: RNE gives 1 + ulp; the kernel's 1.0 is adopted
    got, n = round_at(np.array([mid + w / 2]), one)
    assert got[0] == 1.0 and n == 1
    # outside the window the oracle's own rounding stands
    got, n = round_at(np.array([mid + 2 * w]), one)
    assert got[0] == 1.0 + ulp and n == 0
    # a kernel value that is not the other neighbour is never adopted, even on a midpoint
    got, n = round_at(np.array([mid]), bits(np.array([1.0 + 2 * ulp])))
    assert got[0] == 1.0 and n == 0
    got, n = round_at(np.array([mid]), bits(np.array([-(1.0 + ulp)])))
    assert got[0] == 1.0 and n == 0
    # agreeing values, and no kernel values at all, give plain round_bf16
    u = np.random.default_rng(8).standard_normal(1000) * 7
    r = O.round_bf16(u)
    assert np.array_equal(round_at(u, O.bf16_bits_of(r))[0], r) and np.array_equal(round_at(u)[0], r)
    # negative values: the midpoint between -1 and -(1 + ulp)
    got, n = round_at(np.array([-mid]), bits(np.array([-(1.0 + ulp)])))
    assert got[0] == -(1.0 + ulp) and n == 1


def test_decoder_layer_feed_and_tie_with_its_own_values_change_nothing():
    """Feeding a layer its own stored activations, or offering its own
    roundings as the kernel's, reproduces the plain step bit for bit and
    takes no decision from outside; feeding a different value changes what
    follows (the feed is used)."""
    from oracle.decode_step import LAYER_ROUNDINGS
    rng = np.random.default_rng(9)
    w = _tiny_weights(rng, layers=2, max_pos=32)
    caches = [[(rand_bf16(rng, (L, 1, 128)), rand_bf16(rng, (L, 1, 128))) for _ in range(2)] for L in (3, 20)]
    toks = np.array([4, 17])
    plain = OracleDecoder(w, 2, 4, 1, 1e-6, caches)
    ref = plain.step(toks)
    vals = dict(plain.values)
    own = {key: O.bf16_bits_of(O.round_bf16(v)) for key, v in vals.items() if key[1] != "v"}
    tied = OracleDecoder(w, 2, 4, 1, 1e-6, caches)
    assert np.array_equal(tied.step(toks, tie=own), ref) and sum(tied.ties.values()) == 0
    assert {name for (_, name) in vals} == set(LAYER_ROUNDINGS) | {"v"}
    # layer 1 alone from the stored layer-0 outputs, fed its own activations: same values
    x1, h1 = own[(0, "x_out")], own[(0, "h_out")]
    for feed in ({}, {name: b for (l, name), b in own.items() if l == 1}):
        d = OracleDecoder(w, 2, 4, 1, 1e-6, caches)
        d.kv = [[plain.kv[s][0], (plain.kv[s][1][0][:-1], plain.kv[s][1][1][:-1])] for s in range(2)]
        v1, st1 = d.layer(1, x1, h1, [0, 1], feed=feed)
        for name in LAYER_ROUNDINGS[1:]:
            assert np.array_equal(v1[name], vals[(1, name)]), name
    # a fed activation replaces the oracle's own downstream
    d = OracleDecoder(w, 2, 4, 1, 1e-6, caches)
    d.kv = [[plain.kv[s][0], (plain.kv[s][1][0][:-1], plain.kv[s][1][1][:-1])] for s in range(2)]
    bent = own[(1, "o")].copy()
    bent[0, 0] ^= 0x40
    v1, _ = d.layer(1, x1, h1, [0, 1], feed={"o": bent})
    assert not np.array_equal(v1["x_mid"], vals[(1, "x_mid")])


# ------------------------------------------------------------------ prefill attention
def _paged(rng, lens, hkv=1, page=16):
    pages = sum((L + page - 1) // page for L in lens)
    perm = rng.permutation(pages)
    table = np.zeros((len(lens), max((L + page - 1) // page for L in lens)), dtype=np.int32)
    off = 0
    for b, L in enumerate(lens):
        n = (L + page - 1) // page
        table[b, :n] = perm[off:off + n]
        off += n
    return rand_bf16(rng, (pages, hkv, page, 128)), rand_bf16(rng, (pages, hkv, page, 128)), table


def test_prefill_first_token_sees_only_itself_and_rows_equal_decode():
    rng = np.random.default_rng(6)
    kp, vp, table = _paged(rng, [40, 300])
    q_seq, q_pos = [0, 0, 0, 1, 1], [0, 17, 39, 255, 299]
    q = rand_bf16(rng, (5, 4, 128))
    out = O.prefill_attention(q, kp, d_major(vp), table, q_seq, q_pos, 128 ** -0.5)
    v0 = O.bf16_bits_to_f64(vp[table[0, 0], 0, 0])
    for h in range(4):
        assert np.array_equal(out[0, h], v0)  # softmax over one token is exactly 1
    # each row is the decode attention of its sequence truncated to p + 1 tokens
    for r in range(5):
        one = O.decode_attention(q[r:r + 1], kp, d_major(vp), table[q_seq[r]:q_seq[r] + 1], [q_pos[r] + 1], 128 ** -0.5)
        assert np.allclose(out[r], one[0], rtol=1e-13, atol=1e-13)


def test_prefill_brute_force_causal_mask():
    # two tokens, scores a and b: row 1 = (e^a v0 + e^b v1) / (e^a + e^b), computed with fsum
    rng = np.random.default_rng(7)
    kp, vp, table = _paged(rng, [2])
    q = rand_bf16(rng, (2, 4, 128))
    out = O.prefill_attention(q, kp, d_major(vp), table, [0, 0], [0, 1], 0.125)
    K = O.bf16_bits_to_f64(kp[table[0, 0], 0, :2])
    V = O.bf16_bits_to_f64(vp[table[0, 0], 0, :2])
    qq = O.bf16_bits_to_f64(q)
    for h in range(4):
        s = [0.125 * math.fsum(qq[1, h] * K[t]) for t in range(2)]
        w = [math.exp(x - max(s)) for x in s]
        want = [math.fsum([w[0] * V[0, d], w[1] * V[1, d]]) / math.fsum(w) for d in range(128)]
        assert np.allclose(out[1, h], want, rtol=1e-13, atol=1e-14)
        assert np.array_equal(out[0, h], V[0])
