"""Pins for the fp64 oracle, checked against things other than itself:
hand-derived fixtures, closed forms, invariants, and brute force with
correctly rounded sums (math.fsum) on tiny inputs. CPU only.

Each group is chosen so that a plausible slip in the oracle (a transposed
operand, a wrong index, a dropped term, a missing scale) fails at least one
test; ``test_pins_catch_planted_mistakes`` plants such slips in copies of the
oracle's functions and checks the pins notice.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from helpers import d_major

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    """fp64/fp32 values that are exactly representable in bf16 -> uint16 bits
    (truncation is exact for such values; asserted)."""
    f = np.asarray(x, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    back = (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, f), "value not exactly representable in bf16"
    return b


def rand_bf16(rng, shape, scale=1.0):
    """Random bf16 bit patterns with values scale*N(0,1) (truncated to bf16)."""
    f = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- decoding
def test_bf16_decode_known_patterns():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x0000 = +0, 0x8000 = -0, 0x7F80 = +inf,
    # 0x0001 = smallest bf16 subnormal = 2^-133.
    b = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049], dtype=np.uint16)
    v = O.bf16_bits_to_f64(b)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0 and v[4] == math.inf
    assert math.copysign(1.0, v[3]) == -1.0
    assert v[5] == 2.0 ** -133
    assert v[6] == 3.140625  # 0x4049 = 1.5703125 * 2
    with pytest.raises(TypeError):
        O.bf16_bits_to_f64(np.zeros(3, dtype=np.int32))


# ----------------------------------------------------------------- mm/addmm
def test_mm_textbook_fixture():
    d = load("mm_textbook_2x3x2.json")
    A, B, C = bits(d["A"]), bits(d["B_kn"]), np.array(d["C"], float)
    assert np.array_equal(O.mm(A, B), C)
    # the same product with B stored [N, K]
    Bt = bits(np.array(d["B_kn"], float).T)
    assert np.array_equal(O.mm(A, Bt, b_is_nk=True), C)


def test_addmm_fixture():
    d = load("addmm_hand_2x2x2.json")
    out = O.addmm(bits(d["bias"]), bits(d["A"]), bits(d["B_kn"]), beta=d["beta"], alpha=d["alpha"])
    assert np.array_equal(out, np.array(d["out"], float))
    # fp32 bias path gives the same
    out2 = O.addmm(np.array(d["bias"], np.float32), bits(d["A"]), bits(d["B_kn"]),
                   beta=d["beta"], alpha=d["alpha"])
    assert np.array_equal(out2, out)


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (3, 5, 7), (7, 2, 11), (12, 9, 16), (5, 13, 4)])
@pytest.mark.parametrize("b_is_nk", [False, True])
def test_mm_brute_force_fsum(m, n, k, b_is_nk):
    rng = np.random.default_rng(1000 * m + 10 * n + k)
    A = rand_bf16(rng, (m, k))
    B = rand_bf16(rng, (n, k) if b_is_nk else (k, n))
    a = O.bf16_bits_to_f64(A)
    b = O.bf16_bits_to_f64(B)
    got = O.mm(A, B, b_is_nk=b_is_nk)
    for i in range(m):
        for j in range(n):
            terms = [a[i, kk] * (b[j, kk] if b_is_nk else b[kk, j]) for kk in range(k)]
            exact = math.fsum(terms)  # bf16*bf16 products are exact in fp64
            bound = 1e-12 * math.fsum(abs(t) for t in terms) + 1e-300
            assert abs(got[i, j] - exact) <= bound


def test_mm_identity_and_scaled_permutation_exact():
    rng = np.random.default_rng(7)
    A = rand_bf16(rng, (9, 16))
    I = bits(np.eye(16))
    assert np.array_equal(O.mm(A, I), O.bf16_bits_to_f64(A))
    # B = 2^-3 * P (permutation): C = A[:, perm^-1] / 8 exactly
    perm = rng.permutation(16)
    P = np.zeros((16, 16))
    P[np.arange(16), perm] = 0.125
    C = O.mm(A, bits(P))
    a = O.bf16_bits_to_f64(A)
    expect = np.empty_like(a)
    expect[:, perm] = a * 0.125
    assert np.array_equal(C, expect)


def test_mm_ones_gives_k():
    for k in (1, 3, 512, 4096):
        C = O.mm(bits(np.ones((2, k))), bits(np.ones((k, 3))))
        assert np.all(C == k)


def test_mm_rejects_mismatched_inner():
    with pytest.raises(ValueError):
        O.mm(bits(np.ones((2, 3))), bits(np.ones((4, 2))))


def test_addmm_zero_a_gives_bias():
    rng = np.random.default_rng(3)
    bias = rand_bf16(rng, (17,))
    out = O.addmm(bias, bits(np.zeros((4, 8))), rand_bf16(rng, (8, 17)))
    assert np.array_equal(out, np.broadcast_to(O.bf16_bits_to_f64(bias), (4, 17)))


# ----------------------------------------------------------------- rmsnorm
def test_rmsnorm_hand_cases():
    # x=[3,4], w=[1,2], eps=0: mean(x^2) = 12.5
    y = O.rmsnorm(bits([[3, 4]]), bits([1, 2]), 0.0)
    r = math.sqrt(12.5)
    assert abs(y[0, 0] - 3 / r) < 1e-15 and abs(y[0, 1] - 2 * 4 / r) < 1e-15
    # x = ones(4), eps = 0.5: y = 1/sqrt(1.5)
    y = O.rmsnorm(bits([[1, 1, 1, 1]]), bits([1, 1, 1, 1]), 0.5)
    assert np.allclose(y, 1 / math.sqrt(1.5), rtol=0, atol=1e-15)


@pytest.mark.parametrize("c", [0.0, 1.0, -0.5, 3.0, 2.0 ** -6])
def test_rmsnorm_constant_row_closed_form(c):
    rng = np.random.default_rng(11)
    n, eps = 4096, 1e-6
    w = rand_bf16(rng, (n,))
    y = O.rmsnorm(bits(np.full((1, n), c)), w, eps)
    expect = O.bf16_bits_to_f64(w) * c / math.sqrt(c * c + eps)
    assert np.allclose(y[0], expect, rtol=1e-14, atol=0)


def test_rmsnorm_brute_force_and_scale():
    rng = np.random.default_rng(12)
    X = rand_bf16(rng, (3, 37))
    W = rand_bf16(rng, (37,))
    x, w = O.bf16_bits_to_f64(X), O.bf16_bits_to_f64(W)
    y = O.rmsnorm(X, W, 1e-6)
    for i in range(3):
        r = 1.0 / math.sqrt(math.fsum(v * v for v in x[i]) / 37 + 1e-6)
        for j in range(37):
            assert abs(y[i, j] - w[j] * x[i, j] * r) <= 1e-14 * abs(w[j] * x[i, j] * r) + 1e-300
    # scaling x by 2^k leaves y unchanged when eps = 0
    y1 = O.rmsnorm(X, W, 0.0)
    y2 = O.rmsnorm(bits(x * 8.0), W, 0.0)
    assert np.allclose(y1, y2, rtol=1e-14, atol=0)


# ----------------------------------------------------------------- mean
def test_mean_fixture_and_closed_forms():
    d = load("mean_hand.json")
    for case in d["cases"]:
        assert np.array_equal(O.mean(bits(case["x"])), np.array(case["y"]))
        assert np.array_equal(O.mean(np.array(case["x"], np.float32)), np.array(case["y"]))
    for c in (1.5, -3.25, 0.0):
        assert O.mean(bits(np.full((2, 4096), c)))[1] == c


# ----------------------------------------------------------------- log_softmax
def test_log_softmax_hand_case():
    y = O.log_softmax(np.array([[1.0, 2.0, 3.0]], np.float32))
    lse = math.log(math.exp(1) + math.exp(2) + math.exp(3))
    assert np.allclose(y[0], [1 - lse, 2 - lse, 3 - lse], rtol=0, atol=1e-15)


def test_log_softmax_exp_sums_to_one():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((4, 151936)) * 2.0).astype(np.float32)
    y = O.log_softmax(x)
    for i in range(4):
        assert abs(math.fsum(np.exp(y[i])) - 1.0) <= 1e-12


def test_log_softmax_closed_forms():
    n = 151936
    y = O.log_softmax(np.full((1, n), 0.7, np.float32))
    assert np.allclose(y, -math.log(n), rtol=0, atol=1e-12)
    # one-hot: x0 = delta, rest 0 -> y0 = -log(1 + (n-1) e^-delta), yj = y0 - delta
    for delta in (0.5, 5.0, 30.0):
        x = np.zeros((1, n), np.float32)
        x[0, 0] = delta
        y = O.log_softmax(x)
        y0 = -math.log1p((n - 1) * math.exp(-delta))
        assert abs(y[0, 0] - y0) < 1e-12
        assert abs(y[0, 5] - (y0 - delta)) < 1e-12
    # two entries: y0 = -log(1 + e^(b - a))
    y = O.log_softmax(np.array([[1.0, 4.0]], np.float32))
    assert abs(y[0, 0] + math.log1p(math.exp(3.0))) < 1e-15


def test_log_softmax_shift_invariant():
    rng = np.random.default_rng(6)
    x = rng.integers(-40, 40, size=(3, 1000)).astype(np.float32) / 4
    assert np.allclose(O.log_softmax(x), O.log_softmax(x + np.float32(17.0)), rtol=0, atol=1e-12)


# ----------------------------------------------------------------- argmax
def test_argmax_planted_and_ties():
    x = np.zeros((4, 151936), np.float32)
    x[0, 12345] = 9.0
    x[1, 7] = 3.0
    x[1, 150000] = 3.0          # tie: lowest index wins
    x[2, :] = -1.0
    x[2, 151935] = -0.5         # max at the last column
    # row 3 all zeros: index 0
    assert O.argmax(x).tolist() == [12345, 7, 151935, 0]
    with pytest.raises(TypeError):
        O.argmax(x.astype(np.float64))


# ----------------------------------------------------------------- attention
def paged(rng, lens, hkv, d, page, scale=1.0):
    """Random K/V caches with a random physical page permutation."""
    pages_per = [(L + page - 1) // page for L in lens]
    total = sum(pages_per)
    perm = rng.permutation(total)
    table = np.zeros((len(lens), max(pages_per)), np.int32)
    off = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[off:off + n]
        off += n
    K = rand_bf16(rng, (total, hkv, page, d), scale)
    V = rand_bf16(rng, (total, hkv, page, d), scale)
    return K, V, table


def test_attention_single_token_returns_v0():
    rng = np.random.default_rng(21)
    hq, hkv, d, page = 8, 2, 16, 4
    K, V, table = paged(rng, [1, 1], hkv, d, page)
    q = rand_bf16(rng, (2, hq, d))
    out = O.decode_attention(q, K, d_major(V), table, [1, 1], scale=0.25)
    for b in range(2):
        for h in range(hq):
            v0 = O.bf16_bits_to_f64(V[table[b, 0], h // (hq // hkv), 0])
            assert np.array_equal(out[b, h], v0)


def test_attention_zero_query_is_mean_of_v():
    rng = np.random.default_rng(22)
    hq, hkv, d, page, L = 4, 2, 8, 4, 11
    K, V, table = paged(rng, [L], hkv, d, page)
    q = bits(np.zeros((1, hq, d)))
    out = O.decode_attention(q, K, d_major(V), table, [L], scale=1.0)
    for h in range(hq):
        g = h // 2
        v = np.stack([O.bf16_bits_to_f64(V[table[0, t // page], g, t % page]) for t in range(L)])
        assert np.allclose(out[0, h], v.mean(axis=0), rtol=1e-14, atol=1e-15)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(23)
    hq, hkv, d, page = 4, 1, 4, 2
    lens = [1, 2, 3, 4]
    K, V, table = paged(rng, lens, hkv, d, page)
    q = rand_bf16(rng, (4, hq, d))
    scale = 1 / math.sqrt(d)
    out = O.decode_attention(q, K, d_major(V), table, lens, scale)
    qq = O.bf16_bits_to_f64(q)
    for b, L in enumerate(lens):
        for h in range(hq):
            ks = [O.bf16_bits_to_f64(K[table[b, t // page], 0, t % page]) for t in range(L)]
            vs = [O.bf16_bits_to_f64(V[table[b, t // page], 0, t % page]) for t in range(L)]
            sc = [scale * math.fsum(qq[b, h, i] * k[i] for i in range(d)) for k in ks]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = math.fsum(e)
            for i in range(d):
                ref = math.fsum(e[t] * vs[t][i] for t in range(L)) / z
                assert abs(out[b, h, i] - ref) <= 1e-13 * (abs(ref) + 1)


def test_attention_two_token_closed_form_pins_scale():
    # K0 = 0, K1 = e_0 * 2, q = e_0 * 3: scores 0 and 6*scale;
    # out = (v0 + e^(6 scale) v1) / (1 + e^(6 scale)).
    hq, hkv, d, page = 1, 1, 4, 16
    K = np.zeros((1, hkv, page, d))
    K[0, 0, 1, 0] = 2.0
    V = np.zeros((1, hkv, page, d))
    V[0, 0, 0, :] = [1, 2, 3, 4]
    V[0, 0, 1, :] = [-1, 0, 0.5, 8]
    q = np.zeros((1, hq, d))
    q[0, 0, 0] = 3.0
    scale = 0.125
    out = O.decode_attention(bits(q), bits(K), d_major(bits(V)), np.zeros((1, 1), np.int32), [2], scale)
    e = math.exp(6 * scale)
    expect = (np.array([1, 2, 3, 4]) + e * np.array([-1, 0, 0.5, 8])) / (1 + e)
    assert np.allclose(out[0, 0], expect, rtol=1e-15, atol=1e-15)


def test_attention_gqa_head_map_and_page_gather():
    # V of kv head g is the constant token index t + 64 g in every dim (exact in
    # bf16); K is zero except token t* which gets a huge score, so
    # out = t* + 64 * g(h).
    rng = np.random.default_rng(24)
    hq, hkv, d, page, L = 8, 4, 8, 4, 23
    tstar = 13
    pages = (L + page - 1) // page
    perm = rng.permutation(pages)
    table = perm[None, :].astype(np.int32)
    K = np.zeros((pages, hkv, page, d))
    V = np.zeros((pages, hkv, page, d))
    for t in range(L):
        p = perm[t // page]
        for g in range(hkv):
            V[p, g, t % page, :] = t + 64 * g
    K[perm[tstar // page], :, tstar % page, 0] = 64.0
    q = np.zeros((1, hq, d))
    q[0, :, 0] = 64.0
    out = O.decode_attention(bits(q), bits(K), d_major(bits(V)), table, [L], scale=1.0)
    for h in range(hq):
        assert np.allclose(out[0, h], tstar + 64 * (h // 2), rtol=0, atol=1e-9)


def test_attention_split_form_equals_single_pass():
    rng = np.random.default_rng(25)
    hq, hkv, d, page = 8, 2, 32, 16
    lens = [1, 255, 256, 257, 700, 1024]
    K, V, table = paged(rng, lens, hkv, d, page)
    q = rand_bf16(rng, (len(lens), hq, d))
    a = O.decode_attention(q, K, d_major(V), table, lens, 1 / math.sqrt(d))
    for split in (16, 256):
        b = O.decode_attention_split(q, K, d_major(V), table, lens, 1 / math.sqrt(d), split)
        assert O.relative_frobenius(b, a) < 1e-13
        assert np.max(np.abs(b - a)) < 1e-13


def test_split_counts():
    assert O.decode_split_counts([1, 255, 256, 257, 32768], 256).tolist() == [1, 1, 1, 2, 128]


# ----------------------------------------------------------------- comparators
def test_comparators():
    ref = np.array([3.0, 4.0])
    assert O.relative_frobenius(ref, ref) == 0.0
    assert abs(O.relative_frobenius(ref + np.array([0.3, 0.4]), ref) - 0.1) < 1e-15
    assert O.relative_frobenius(np.zeros(2), np.zeros(2)) == 0.0
    assert abs(O.elementwise_ratio(np.array([1.5]), np.array([1.0])) - 0.25) < 1e-15


# ----------------------------------------------------------------- the pins bite
def test_pins_catch_planted_mistakes():
    """Plant plausible slips in copies of oracle functions (on the CPU) and
    check that the pins above reject each one."""
    d = load("mm_textbook_2x3x2.json")
    A, B, C = bits(d["A"]), bits(d["B_kn"]), np.array(d["C"], float)

    def mm_transposed_b(a_bits, b_bits, b_is_nk=False):  # forgets the layout flag
        return O.bf16_bits_to_f64(a_bits) @ O.bf16_bits_to_f64(b_bits)
    Bt = bits(np.array(d["B_kn"], float).T)
    with pytest.raises(ValueError):
        mm_transposed_b(A, Bt, True)  # shape error surfaces immediately
    assert not np.array_equal(O.mm(A, B)[:, ::-1], C)  # a column-index slip changes C

    def rms_sum_not_mean(x_bits, w_bits, eps):
        x, w = O.bf16_bits_to_f64(x_bits), O.bf16_bits_to_f64(w_bits)
        return w * x / np.sqrt(np.sum(x * x, axis=1) + eps)[:, None]
    y = rms_sum_not_mean(bits([[3, 4]]), bits([1, 2]), 0.0)
    assert abs(y[0, 0] - 3 / math.sqrt(12.5)) > 1e-3

    def rms_eps_outside(x_bits, w_bits, eps):
        x, w = O.bf16_bits_to_f64(x_bits), O.bf16_bits_to_f64(w_bits)
        return w * x / (np.sqrt(np.mean(x * x, axis=1)) + eps)[:, None]
    y = rms_eps_outside(bits([[1, 1, 1, 1]]), bits([1, 1, 1, 1]), 0.5)
    assert abs(y[0, 0] - 1 / math.sqrt(1.5)) > 1e-3

    def lsm_no_log(x):
        x = x.astype(np.float64)
        m = x.max(1, keepdims=True)
        return x - m - np.sum(np.exp(x - m), 1, keepdims=True)
    y = lsm_no_log(np.array([[1.0, 2.0, 3.0]], np.float32))
    lse = math.log(math.exp(1) + math.exp(2) + math.exp(3))
    assert abs(y[0, 0] - (1 - lse)) > 1e-3

    def attn_wrong_group(q_bits, Kp, Vp, table, lens, scale):
        # maps head h to kv head h % Hkv instead of h // (Hq/Hkv)
        q = O.bf16_bits_to_f64(q_bits)
        out = np.zeros(q.shape)
        hkv = Kp.shape[1]
        for b in range(q.shape[0]):
            for h in range(q.shape[1]):
                k = O.gather_kv(Kp, table, lens[b], h % hkv, b)
                v = O.gather_kv(Vp, table, lens[b], h % hkv, b, d_major=True)
                s = scale * (k @ q[b, h])
                p = np.exp(s - s.max())
                out[b, h] = p @ v / p.sum()
        return out
    hq, hkv, dd, page, L = 8, 4, 8, 4, 5
    K = np.zeros((2, hkv, page, dd))
    V = np.zeros((2, hkv, page, dd))
    for g in range(hkv):
        V[:, g] = 64 * g
    q = np.zeros((1, hq, dd))
    table = np.array([[0, 1]], np.int32)
    good = O.decode_attention(bits(q), bits(K), d_major(bits(V)), table, [L], 1.0)
    bad = attn_wrong_group(bits(q), bits(K), d_major(bits(V)), table, [L], 1.0)
    assert np.allclose(good[0, 1], 0.0) and not np.allclose(bad[0, 1], 0.0)
