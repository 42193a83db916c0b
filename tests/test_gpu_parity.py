"""GPU parity: every kernel against the fp64 oracle, through the C ABI.

fp32 outputs must meet relative Frobenius <= 1e-3 and elementwise
|err| <= 4e-3 (|ref| + 1). bf16 outputs cannot meet the Frobenius bound
against an unrounded oracle (a single round-to-nearest of N(0,1) data to bf16
alone gives ~1.7e-3), so they are checked as bitwise equal to torch's
round-to-nearest-even of the same kernel's fp32 output, plus the elementwise
bound against the unrounded oracle. Argmax indices are compared exactly on
the same fp32 logits.

Small cases are compared element by element; the full-size shapes are
compared on sampled rows/columns the oracle can afford, in the launch
configuration the benchmark times.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from helpers import assert_close, bits, d_major, f32, rne_bf16, same_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("m", [1, 2, 3, 8, 16])
def test_mm_smoke_config(lib, m):
    """X[M,512] ~ N(0,1), W[512,512] ~ N(0,1/512): the small smoke case."""
    say(f"mm smoke m={m}")
    x = S.rows_with_fixed_row(m, 512, 1.0, fixed_seed=1, other_seed=100 + m).to(DEV)
    w = S.normal_bf16((512, 512), 1 / 512, seed=2).to(DEV)
    c = lib.bi_mm(x, w)
    ref = O.mm(bits(x), bits(w))
    assert_close(f32(c), ref, f"mm m={m}")
    cb = lib.bi_mm(x, w, out_dtype=torch.bfloat16)
    assert same_bits(cb, rne_bf16(c)), "bf16 output is not RNE of the fp32 output"
    assert O.elementwise_ratio(f32(cb.float()), ref) <= 4e-3


@pytest.mark.parametrize("b_is_nk", [False, True])
@pytest.mark.parametrize("m,n,k", [(300, 200, 264), (129, 136, 520), (1, 8, 8), (257, 384, 64), (77, 1000, 1032)])
def test_mm_ragged_tiles(lib, m, n, k, b_is_nk):
    """Sizes that span several tiles with ragged M, N and K tails."""
    if not b_is_nk and n % 8:
        pytest.skip("B [k, n] needs n % 8 == 0")
    say(f"mm ragged m={m} n={n} k={k} nk={b_is_nk}")
    a = S.normal_bf16((m, k), 1.0, seed=m * 7 + k).to(DEV)
    b = S.normal_bf16((n, k) if b_is_nk else (k, n), 1.0 / k, seed=n * 13 + k).to(DEV)
    c = lib.bi_mm(a, b, b_is_nk=b_is_nk)
    assert_close(f32(c), O.mm(bits(a), bits(b), b_is_nk=b_is_nk), "mm ragged")


@pytest.mark.parametrize("b_is_nk", [False, True])
def test_mm_wide_skinny_tiles_ragged(lib, b_is_nk):
    """The 96-column skinny tiles on a width that is not a multiple of 96 (or
    32) and a ragged K: against the oracle, and bit for bit against the
    fixed-tile mode (256x256 tiles) for the same rows."""
    n, k = 20008, 1032
    w = S.normal_bf16((n, k) if b_is_nk else (k, n), 1.0 / k, seed=81, device=DEV)
    for m in (1, 33, 64):
        cfg = lib.bi_gemm_config(m, n, k, b_is_nk)
        say(f"wide skinny m={m} n={n} k={k} nk={b_is_nk} cfg={cfg}")
        assert cfg[1] == 96, cfg
        a = S.normal_bf16((m, k), 1.0, seed=82 + m, device=DEV)
        c = lib.bi_mm(a, w, b_is_nk=b_is_nk)
        cols = np.r_[0:40, n // 2 - 20:n // 2 + 20, n - 72:n]
        wb = bits(w)
        ref = O.mm(bits(a), wb[cols] if b_is_nk else wb[:, cols], b_is_nk=b_is_nk)
        assert_close(f32(c)[:, cols], ref, "wide skinny vs oracle")
        fixed = lib.bi_gemm(a, w, b_is_nk=b_is_nk, fixed_tile=True)
        assert same_bits(c, fixed)


def test_mm_layouts_agree_bitwise(lib):
    """B stored [K,N] and the same B stored [N,K] give identical bits: the
    layout changes only how B reaches LDS, not the arithmetic."""
    say("mm layouts")
    a = S.normal_bf16((200, 512), 1.0, seed=5).to(DEV)
    b = S.normal_bf16((512, 384), 1 / 512, seed=6).to(DEV)
    c1 = lib.bi_mm(a, b)
    c2 = lib.bi_mm(a, b.t().contiguous(), b_is_nk=True)
    assert same_bits(c1, c2)


def test_mm_strided_operands(lib):
    """Row strides larger than the rows (sub-views of wider buffers)."""
    say("mm strided")
    big_a = S.normal_bf16((70, 520), 1.0, seed=8).to(DEV)
    big_b = S.normal_bf16((264, 208), 1 / 256, seed=9).to(DEV)
    a = big_a[:, :256]
    b = big_b[:256, :200]
    out_big = torch.full((70, 216), 7.0, device=DEV)
    out = out_big[:, :200]
    lib.bi_mm(a, b, out=out)
    assert_close(f32(out), O.mm(bits(a), bits(b)), "mm strided")
    assert torch.all(out_big[:, 200:] == 7.0), "wrote outside the output view"


def test_mm_identity_and_ones_exact(lib):
    say("mm identity")
    a = S.normal_bf16((130, 256), 1.0, seed=10).to(DEV)
    eye = torch.eye(256, dtype=torch.bfloat16, device=DEV)
    assert same_bits(lib.bi_mm(a, eye), a.float())
    assert same_bits(lib.bi_mm(a, eye, out_dtype=torch.bfloat16), a)
    ones_a = torch.ones((5, 4096), dtype=torch.bfloat16, device=DEV)
    ones_b = torch.ones((4096, 64), dtype=torch.bfloat16, device=DEV)
    assert torch.all(lib.bi_mm(ones_a, ones_b) == 4096.0)


def test_mm_k_zero_and_empty(lib):
    say("mm empty")
    a = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    b = torch.empty((0, 16), dtype=torch.bfloat16, device=DEV)
    c = torch.full((5, 16), 3.0, device=DEV)
    lib.bi_mm(a, b, out=c)
    assert torch.all(c == 0)
    e = lib.bi_mm(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV),
                  torch.ones((64, 8), dtype=torch.bfloat16, device=DEV))
    assert e.shape == (0, 8)
    # k == 0 at a size whose k > 0 form takes the 256x384 tile (no k mask in
    # its loads): the table must keep such a call on a masked kernel
    for nk in (False, True):
        m, n = 1024, 24576
        assert lib.bi_gemm_config(m, n, 0, nk)[1] != 384 and lib.bi_gemm_config(m, n, 64, nk)[1] == 384
        a = torch.empty((m, 0), dtype=torch.bfloat16, device=DEV)
        b = torch.empty((n, 0) if nk else (0, n), dtype=torch.bfloat16, device=DEV)
        c = torch.full((m, n), 3.0, device=DEV)
        lib.bi_mm(a, b, out=c, b_is_nk=nk)
        assert torch.all(c == 0)


QWEN = [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)]


@pytest.mark.parametrize("b_is_nk", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("k,n", QWEN)
@pytest.mark.parametrize("m", [1, 512, 4096])
def test_mm_qwen_shapes_sampled(lib, k, n, m, b_is_nk):
    """Full-size projection GEMMs (weights ~N(0,0.02)), sampled rows, the
    weight stored [K,N] (the benchmark's layout) or [N,K] (the decode
    step's)."""
    say(f"mm qwen k={k} n={n} m={m} b_is_nk={b_is_nk}")
    a = S.normal_bf16((m, k), 1.0, seed=20 + m, device=DEV)
    w = S.normal_bf16((k, n), 0.02, seed=30 + n + k, device=DEV)
    c = lib.bi_mm(a, w.t().contiguous(), b_is_nk=True) if b_is_nk else lib.bi_mm(a, w)
    rows = sorted({0, m - 1, m // 2, (m * 7) // 11})
    ref = O.mm(bits(a[rows]), bits(w))
    assert_close(f32(c[rows]), ref, f"qwen k={k} n={n} m={m}")


def test_addmm_small_and_alpha_beta(lib):
    say("addmm small")
    a = S.normal_bf16((70, 256), 1.0, seed=40).to(DEV)
    b = S.normal_bf16((256, 136), 1 / 256, seed=41).to(DEV)
    bias = S.normal_bf16((136,), 0.1, seed=42).to(DEV)
    c = lib.bi_addmm(bias, a, b)
    assert_close(f32(c), O.addmm(bits(bias), bits(a), bits(b)), "addmm")
    c2 = lib.bi_addmm(bias.float(), a, b, beta=0.5, alpha=2.0)
    assert_close(f32(c2), O.addmm(f32(bias.float()), bits(a), bits(b), beta=0.5, alpha=2.0), "addmm a/b")
    cb = lib.bi_addmm(bias, a, b, out_dtype=torch.bfloat16)
    assert same_bits(cb, rne_bf16(c))
    # A = 0 gives beta * bias exactly
    z = lib.bi_addmm(bias, torch.zeros_like(a), b)
    assert same_bits(z, bias.float().expand(70, 136).contiguous())


def test_addmm_lm_head_then_log_softmax(lib):
    """LM head (X[M,4096], W[4096,151936] ~N(0,0.02), bias ~N(0,0.1)) then
    log_softmax + argmax, sampled columns/rows."""
    m, k, n = 32, 4096, 151936
    say("lm head chain")
    x = S.normal_bf16((m, k), 1.0, seed=50, device=DEV)
    w = S.normal_bf16((k, n), 0.02, seed=51, device=DEV)
    bias = S.normal_bf16((n,), 0.1, seed=52, device=DEV)
    logits = lib.bi_addmm(bias, x, w)
    rows = [0, 13, 31]
    cols = np.sort(np.random.default_rng(0).choice(n, 2048, replace=False))
    colst = torch.from_numpy(cols).to(DEV)
    ref = O.addmm(bits(bias[colst]), bits(x[rows]), bits(w[:, colst]))
    assert_close(f32(logits[rows][:, colst]), ref, "lm head")
    lp, am = lib.bi_log_softmax(logits)
    # op-level: log_softmax and argmax on the GPU logits against the oracle
    lg = f32(logits[rows])
    assert_close(f32(lp[rows]), O.log_softmax(lg), "log_softmax of lm head")
    assert am[rows].cpu().tolist() == O.argmax(lg).tolist()


def test_addmm_lm_head_benchmark_size_sampled(lib):
    """The benchmark's LM head (X[256,4096], W[4096,151936], bias; its seeded
    inputs) in its own launch configuration: at M = 256 the first 131072
    columns run on 256x256 tiles and the rest on 256x128 tiles, so the
    sampled columns come from both parts."""
    m, k, n, split = 256, 4096, 151936, 131072
    say("lm head 256 x 151936")
    x = S.normal_bf16((m, k), 1.0, seed=4000, device=DEV)
    w = S.normal_bf16((k, n), 0.02, seed=4001, device=DEV)
    bias = S.normal_bf16((n,), 0.1, seed=4002, device=DEV)
    logits = lib.bi_addmm(bias, x, w)
    rows = [0, 101, 255]
    g = np.random.default_rng(1)
    cols = np.unique(np.concatenate([g.choice(split, 1024, replace=False),
                                     split + g.choice(n - split, 1024, replace=False), [split - 1, split, n - 1]]))
    colst = torch.from_numpy(cols).to(DEV)
    ref = O.addmm(bits(bias[colst]), bits(x[rows]), bits(w[:, colst]))
    assert_close(f32(logits[rows][:, colst]), ref, "lm head 256 rows")


# ------------------------------------------------------------------ reductions
@pytest.mark.parametrize("m", [1, 7, 64, 513, 2048])
def test_rmsnorm(lib, m):
    say(f"rmsnorm m={m}")
    x = S.normal_bf16((m, 4096), 1.0, seed=60 + m).to(DEV)
    w = S.uniform_bf16((4096,), 0.5, 1.5, seed=61).to(DEV)
    y = lib.bi_rmsnorm(x, w, 1e-6, out_dtype=torch.float32)
    ref = O.rmsnorm(bits(x), bits(w), 1e-6)
    assert_close(f32(y), ref, f"rmsnorm m={m}")
    yb = lib.bi_rmsnorm(x, w, 1e-6, out_dtype=torch.bfloat16)
    assert same_bits(yb, rne_bf16(y)), "bf16 RMSNorm is not RNE of its fp32 output"
    assert O.elementwise_ratio(f32(yb.float()), ref) <= 4e-3


@pytest.mark.parametrize("n", [4100, 5, 8, 13, 20000, 4096 * 5])
def test_rmsnorm_other_widths(lib, n):
    """Widths with a tail (n % 8 != 0), tiny rows and rows past the register
    cache (streaming variant)."""
    say(f"rmsnorm n={n}")
    ld = (n + 7) // 8 * 8
    buf = S.normal_bf16((9, ld), 1.0, seed=n).to(DEV)
    x = buf[:, :n]
    w = S.uniform_bf16((ld,), 0.5, 1.5, seed=n + 1).to(DEV)[:n]
    y = lib.bi_rmsnorm(x, w, 1e-6, out_dtype=torch.float32, out=torch.empty((9, ld), device=DEV)[:, :n])
    assert_close(f32(y), O.rmsnorm(bits(x), bits(w), 1e-6), f"rmsnorm n={n}")


def test_rmsnorm_constant_rows(lib):
    say("rmsnorm const")
    n = 4096
    x = torch.tensor([0.0, 1.0, -0.5, 3.0], dtype=torch.bfloat16).repeat_interleave(n).view(4, n).to(DEV)
    w = S.uniform_bf16((n,), 0.5, 1.5, seed=62).to(DEV)
    y = lib.bi_rmsnorm(x, w, 1e-6, out_dtype=torch.float32)
    assert torch.all(y[0] == 0)
    assert_close(f32(y), O.rmsnorm(bits(x), bits(w), 1e-6), "rmsnorm const")


@pytest.mark.parametrize("m", [1, 7, 64, 513, 2048])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_mean(lib, m, dt):
    say(f"mean m={m} {dt}")
    x = S.normal_f32((m, 4096), 1.0, seed=70 + m).to(dt).to(DEV)
    y = lib.bi_mean(x)
    ref = O.mean(bits(x) if dt == torch.bfloat16 else f32(x))
    assert_close(f32(y), ref, "mean")


def test_mean_constant_rows_exact_and_tails(lib):
    say("mean const")
    vals = [1.5, -3.25, 0.0, 7.0]
    x = torch.tensor(vals, dtype=torch.bfloat16).repeat_interleave(4096).view(4, 4096).to(DEV)
    assert lib.bi_mean(x).cpu().tolist() == vals
    for n in (1, 5, 4099, 30000):
        ld = (n + 7) // 8 * 8
        xb = S.normal_bf16((3, ld), 1.0, seed=n).to(DEV)[:, :n]
        assert_close(f32(lib.bi_mean(xb)), O.mean(bits(xb)), f"mean n={n}")


@pytest.mark.parametrize("m", [1, 7, 64])
def test_log_softmax(lib, m):
    say(f"log_softmax m={m}")
    x = S.normal_f32((m, 151936), 4.0, seed=80 + m).to(DEV)
    y, am = lib.bi_log_softmax(x)
    xc = f32(x)
    assert_close(f32(y), O.log_softmax(xc), f"log_softmax m={m}")
    assert am.cpu().tolist() == O.argmax(xc).tolist()
    # sum exp(y) = 1 per row (fp64 sum of the fp32 outputs)
    s = np.exp(f32(y).astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(s - 1.0) < 1e-4)



def test_log_softmax_benchmark_size_sampled(lib):
    """The benchmark's 2048 x 151936 log_softmax + argmax (its inputs, same
    seed and launch), sampled rows against the oracle."""
    say("log_softmax 2048 x 151936")
    x = S.normal_f32((2048, 151936), 4.0, seed=1002, device=DEV)
    y, am = lib.bi_log_softmax(x)
    rows = [0, 1, 777, 1024, 2047]
    xc = f32(x[rows])
    assert_close(f32(y[rows]), O.log_softmax(xc), "log_softmax 2048 rows")
    assert am[rows].cpu().tolist() == O.argmax(xc).tolist()
    del x, y

def test_log_softmax_edges(lib):
    say("log_softmax edges")
    n = 1003
    ld = 1004
    buf = S.normal_f32((6, ld), 1.0, seed=90).to(DEV)
    x = buf[:, :n]
    x[0] = 0.7                              # constant row: -log n
    x[1, 10] = 50.0                         # unique max
    x[2, 5] = 9.0
    x[2, 900] = 9.0                         # tie: lowest index
    x[3, n - 1] = 80.0                      # max in the tail (n % 4 != 0)
    y, am = lib.bi_log_softmax(x, out=torch.empty((6, ld), device=DEV)[:, :n])
    xc = f32(x)
    assert_close(f32(y), O.log_softmax(xc), "log_softmax edges")
    assert am.cpu().tolist() == O.argmax(xc).tolist()
    assert am[2].item() == 5 and am[3].item() == n - 1
    assert abs(y[0, 0].item() + math.log(n)) < 1e-5
    y1, none = lib.bi_log_softmax(x[:1].contiguous(), want_argmax=False)
    assert none is None and same_bits(y1, y[:1])


def assert_close_masked(got, ref, what):
    """Parity where the reference holds -inf (masked logits give -inf
    log-probabilities): those positions must be -inf exactly, the rest meet
    the usual tolerance."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    neg = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), neg), f"{what}: -inf positions differ"
    assert np.isfinite(got[~neg]).all(), f"{what}: non-finite values where the oracle is finite"
    assert_close(got[~neg], ref[~neg], what)


@pytest.mark.parametrize("n", [1003, 151936])
def test_log_softmax_masked_rows(lib, n):
    """Rows with -inf entries (banned tokens, a grammar mask): a masked first
    chunk, a masked prefix longer than what a thread keeps in registers, all
    but one entry masked, a masked tail with n % 4 != 0, and a scattered
    mask. The fp64 oracle gives finite log-probabilities for the unmasked
    entries and -inf for the masked ones; so must the kernel."""
    say(f"log_softmax masked rows n={n}")
    m = 6
    ld = (n + 3) // 4 * 4  # rows start 16-byte aligned
    x = S.normal_f32((m, ld), 4.0, seed=95 + n).to(DEV)[:, :n]
    ninf = float("-inf")
    x[0, :4] = ninf                                  # one leading 16-byte chunk
    x[1, : min(n - 1, 70000)] = ninf                 # a long masked prefix
    x[2, :] = ninf
    x[2, n // 3] = 1.5                               # all but one entry masked
    x[3, n - 3:] = ninf                              # masked tail (n % 4 != 0 for 1003)
    g = torch.Generator().manual_seed(96)
    x[4, torch.rand(n, generator=g) < 0.3] = ninf     # scattered
    x[5, 4096:8192] = ninf                           # a block in the middle
    y, am = lib.bi_log_softmax(x, out=torch.empty((m, ld), device=DEV)[:, :n])
    xc = f32(x)
    ref = O.log_softmax(xc)
    assert_close_masked(f32(y), ref, f"masked log_softmax n={n}")
    assert am.cpu().tolist() == O.argmax(xc).tolist()
    assert float(y[2, n // 3]) == 0.0 and am[2].item() == n // 3
    # a row has the same bits alone and in a batch, and in a batch large enough
    # for the one-workgroup-per-row form (the six rows above use the other form)
    y0, _ = lib.bi_log_softmax(x[4:5].contiguous())
    assert same_bits(y0, y[4:5])
    big = torch.empty((80, ld), device=DEV)
    big[:, :n] = S.normal_f32((80, n), 4.0, seed=97).to(DEV)
    big[70:76, :n] = x
    yb, ab = lib.bi_log_softmax(big[:, :n], out=torch.empty((80, ld), device=DEV)[:, :n])
    assert same_bits(yb[70:76], y) and same_bits(ab[70:76], am)


# ------------------------------------------------------------------ decode attention
def make_decode(lens, seed, hkv=8, hq=32, d=128, page=16):
    lens_t = torch.tensor(lens, dtype=torch.int32)
    table, npages = S.paged_kv_layout(lens_t, page, seed=seed)
    q = S.normal_bf16((len(lens), hq, d), 1.0, seed=seed + 1)
    kp = S.normal_bf16((npages, hkv, page, d), 1.0, seed=seed + 2)
    vp = d_major(S.normal_bf16((npages, hkv, page, d), 1.0, seed=seed + 3))
    return lens_t, table, q, kp, vp


def run_decode(lib, lens_t, table, q, kp, vp, out_dtype=torch.float32):
    offs, total = lib.bi_decode_plan(lens_t)
    return lib.bi_decode_attention(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t.to(DEV),
                                   offs.to(DEV), total, out_dtype=out_dtype)


def test_decode_attention_lengths(lib):
    lens = [1, 15, 16, 17, 255, 256, 257, 1000, 4097]
    say("decode lengths", lens)
    lens_t, table, q, kp, vp = make_decode(lens, seed=100)
    out = run_decode(lib, lens_t, table, q, kp, vp)
    ref = O.decode_attention(bits(q), bits(kp), bits(vp), table.numpy(), lens, 128 ** -0.5)
    assert_close(f32(out), ref, "decode")
    outb = run_decode(lib, lens_t, table, q, kp, vp, torch.bfloat16)
    assert same_bits(outb, rne_bf16(out))


def test_decode_attention_single_token_is_v0(lib):
    say("decode L=1")
    lens_t, table, q, kp, vp = make_decode([1, 1, 1], seed=110)
    out = run_decode(lib, lens_t, table, q, kp, vp)
    for b in range(3):
        for h in range(32):
            v0 = vp[table[b, 0], h // 4, :, 0].float()
            assert same_bits(out[b, h].cpu(), v0)


def test_decode_attention_config_batch(lib):
    """A log-uniform batch (lengths in [1, 32768]), sampled sequences."""
    lens_t = S.context_lens(64, seed=120)
    say("decode batch64 total tokens", int(lens_t.sum()))
    table, npages = S.paged_kv_layout(lens_t, 16, seed=121)
    q = S.normal_bf16((64, 32, 128), 1.0, seed=122, device=DEV)
    kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=123, device=DEV)
    vp = d_major(S.normal_bf16((npages, 8, 16, 128), 1.0, seed=124, device=DEV))
    offs, total = lib.bi_decode_plan(lens_t)
    out = lib.bi_decode_attention(q, kp, vp, table.to(DEV), lens_t.to(DEV), offs.to(DEV), total)
    seqs = [0, 1, int(torch.argmax(lens_t)), int(torch.argmin(lens_t)), 63]
    ref = O.decode_attention(bits(q), bits(kp), bits(vp), table.numpy(), lens_t.numpy(), 128 ** -0.5, seqs=seqs)
    assert_close(f32(out[seqs]), ref[seqs], "decode batch")


def test_decode_attention_benchmark_batch_sampled(lib):
    """The benchmark's decode attention (B = 256, lengths log-uniform in
    [1, 32768], its seeds and launch), sampled sequences against the oracle."""
    lens_t = S.context_lens(256, seed=5000)
    say("decode batch256 total tokens", int(lens_t.sum()))
    table, npages = S.paged_kv_layout(lens_t, 16, seed=5001)
    q = S.normal_bf16((256, 32, 128), 1.0, seed=5002, device=DEV)
    kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=5003, device=DEV)
    vp = S.normal_bf16((npages, 8, 128, 16), 1.0, seed=5004, device=DEV)  # d-major, as the benchmark draws it
    offs, total = lib.bi_decode_plan(lens_t)
    out = lib.bi_decode_attention(q, kp, vp, table.to(DEV), lens_t.to(DEV), offs.to(DEV), total)
    seqs = [0, 100, int(torch.argmax(lens_t)), int(torch.argmin(lens_t)), 255]
    ref = O.decode_attention(bits(q), bits(kp), bits(vp), table.numpy(), lens_t.numpy(), 128 ** -0.5, seqs=seqs)
    assert_close(f32(out[seqs]), ref[seqs], "decode batch 256")
    # the streaming hint changes how K/V are loaded, not what is computed
    out_nt = lib.bi_decode_attention(q, kp, vp, table.to(DEV), lens_t.to(DEV), offs.to(DEV), total, stream_kv=True)
    assert same_bits(out_nt, out)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_decode_attention_unaligned_out_same_bits(lib, dt):
    """out need only be aligned to its element size: an output that starts
    one element past a 16-byte boundary (written element by element) gets
    the bits of an aligned one (written as whole 4-element vectors)."""
    lens_t, table, q, kp, vp = make_decode([1, 300, 700], seed=130)
    say("decode unaligned out", dt)
    aligned = run_decode(lib, lens_t, table, q, kp, vp, dt)
    offs, total = lib.bi_decode_plan(lens_t)
    buf = torch.full((1 + 3 * 32 * 128,), 7.0, dtype=dt, device=DEV)
    out = buf[1:].view(3, 32, 128)
    assert out.data_ptr() % 16 != 0
    lib.bi_decode_attention(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t.to(DEV), offs.to(DEV), total,
                            out=out)
    assert same_bits(out, aligned)
    assert buf[0].item() == 7.0


def test_decode_attention_inconsistent_device_offsets_stay_in_bounds(lib):
    """Device-side lengths and offsets are the caller's: the host cannot read
    them. Offsets that give one sequence a split its length does not reach
    (and a sequence with fewer splits than its length needs) leave those
    workgroups with nothing to do; every access stays inside the buffers and
    the sequences whose splits are consistent keep their exact bits."""
    lens = [300, 5, 40]
    say("decode inconsistent offsets", lens)
    lens_t, table, q, kp, vp = make_decode(lens, seed=130)
    good = run_decode(lib, lens_t, table, q, kp, vp)
    bad_offs = torch.tensor([0, 2, 4, 5], dtype=torch.int32)  # sequence 1 (5 tokens) given 2 splits
    ws = torch.zeros(lib.bi_decode_workspace_bytes(5, 32, 128), dtype=torch.uint8, device=DEV)
    out = lib.bi_decode_attention(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), lens_t.to(DEV),
                                  bad_offs.to(DEV), 5, workspace=ws)
    torch.cuda.synchronize()
    assert same_bits(out[0], good[0]) and same_bits(out[2], good[2])


def test_binding_checks_output_shapes(lib):
    """A caller's output buffer must have the shape the kernel writes."""
    a = S.normal_bf16((4, 64), 1.0, seed=140, device=DEV)
    w = S.normal_bf16((64, 32), 1.0, seed=141, device=DEV)
    with pytest.raises(ValueError, match="shape"):
        lib.bi_mm(a, w, out=torch.empty((4, 16), device=DEV))
    with pytest.raises(ValueError, match="shape"):
        lib.bi_mean(a, out=torch.empty(3, device=DEV))
    with pytest.raises(ValueError, match="CUDA"):
        lib.bi_mm(a, w.cpu())
