"""Batch invariance, bit for bit, through the C ABI.

The property -- the defect the pages describe is a kernel whose result for
one sequence changes with the size of the batch it is computed in
(readhandoff.com, agent-run reproducibility pinning, "What does temperature
zero actually guarantee?") -- is checked directly by memcmp, with no oracle: a fixed row
computed alone (M = 1) must have the same bytes inside every batch size, at
every position, whatever the other rows hold (random, zeros, huge, NaN/Inf),
and on every repeated run. A negative control runs the same harness on
torch's own kernels and reports how many rows change.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from helpers import assert_close, bits, d_major, digest, f32, same_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def with_row(m, k, row, pos, seed, fill="random", dtype=torch.bfloat16):
    """[m, k] on the GPU with `row` at `pos` and the other rows per `fill`."""
    if fill == "random":
        x = S.normal_f32((m, k), 1.0, seed=seed, device=DEV)
    elif fill == "zeros":
        x = torch.zeros((m, k), device=DEV)
    elif fill == "huge":
        x = torch.full((m, k), 3.0e38, device=DEV)
    elif fill == "nan":
        x = torch.full((m, k), float("nan"), device=DEV)
        x[:, ::3] = float("inf")
    x = x.to(dtype)
    x[pos] = row
    return x


# ------------------------------------------------------------------ GEMM
def gemm_sweep(lib, k, n, ms, b_is_nk=False, out_dtype=torch.float32, var=0.02, positions=None):
    w = S.normal_bf16((n, k) if b_is_nk else (k, n), var, seed=7 + n + k, device=DEV)
    row = S.normal_bf16((1, k), 1.0, seed=11, device=DEV)[0]
    ref = lib.bi_mm(row[None], w, b_is_nk=b_is_nk, out_dtype=out_dtype)[0].clone()
    bad = []
    for m in ms:
        for pos in (positions(m) if positions else sorted({0, m - 1, (m * 5) // 7})):
            x = with_row(m, k, row, pos, seed=1000 + m)
            c = lib.bi_mm(x, w, b_is_nk=b_is_nk, out_dtype=out_dtype)
            if not same_bits(c[pos], ref):
                bad.append((m, pos))
    return bad


def test_mm_smoke_every_m_up_to_4096(lib):
    """K = N = 512 smoke shape, every M = 1..4096: row 0 fixed, others random."""
    w = S.normal_bf16((512, 512), 1 / 512, seed=2, device=DEV)
    row = S.normal_bf16((1, 512), 1.0, seed=1, device=DEV)[0]
    ref = lib.bi_mm(row[None], w)[0].clone()
    refb = lib.bi_mm(row[None], w, out_dtype=torch.bfloat16)[0].clone()
    say("mm every M 1..4096")
    # one big random block; each M uses its first M rows (row 0 fixed)
    big = S.normal_bf16((4096, 512), 1.0, seed=3, device=DEV)
    big[0] = row
    outs = torch.empty((4096, 512), device=DEV)
    bad = []
    for m in range(1, 4097):
        c = lib.bi_mm(big[:m], w, out=outs[:m])
        if m % 512 == 0 or m < 4:
            torch.cuda.synchronize()
        if not torch.equal(c[0].view(torch.int32), ref.view(torch.int32)):
            bad.append(m)
    assert not bad, f"row 0 changed at M = {bad[:20]}"
    cb = lib.bi_mm(big, w, out_dtype=torch.bfloat16)
    assert same_bits(cb[0], refb)


def test_mm_smoke_every_position_in_tile(lib):
    """The fixed row at every position 0..TM-1 of a tile (and in the next
    tiles), for each tile configuration the shape takes: MFMA lane placement
    must not change its bits."""
    w = S.normal_bf16((512, 512), 1 / 512, seed=2, device=DEV)
    row = S.normal_bf16((1, 512), 1.0, seed=1, device=DEV)[0]
    ref = lib.bi_mm(row[None], w)[0].clone()
    cfgs = {}
    for m in range(1, 600):
        cfgs.setdefault(lib.bi_gemm_config(m, 512, 512), m)
    assert len(cfgs) >= 2, cfgs
    bad = []
    for cfg in cfgs:
        tm = cfg[0]
        m = next(mm for mm in range(2 * tm + 3, 0, -1) if lib.bi_gemm_config(mm, 512, 512) == cfg)
        say(f"every position: config {cfg}, m={m}")
        base = S.normal_bf16((m, 512), 1.0, seed=4, device=DEV)
        for pos in range(m):
            x = base.clone()
            x[pos] = row
            c = lib.bi_mm(x, w)
            if not same_bits(c[pos], ref):
                bad.append((cfg, m, pos))
    assert not bad, f"row changed at {bad[:20]}"


@pytest.mark.parametrize("fill", ["zeros", "huge", "nan"])
def test_mm_adversarial_other_rows(lib, fill):
    w = S.normal_bf16((512, 512), 1 / 512, seed=2, device=DEV)
    row = S.normal_bf16((1, 512), 1.0, seed=1, device=DEV)[0]
    ref = lib.bi_mm(row[None], w)[0].clone()
    for m in (2, 33, 200):
        for pos in (0, m - 1):
            x = with_row(m, 512, row, pos, seed=0, fill=fill)
            assert same_bits(lib.bi_mm(x, w)[pos], ref), (fill, m, pos)


ALL_CONFIGS = {(32, 32, 64, 3), (64, 32, 64, 4), (32, 96, 64, 5), (64, 96, 64, 8), (64, 128, 64, 6), (128, 128, 64, 10),
               (128, 128, 64, 4), (256, 256, 64, 8), (256, 384, 64, 8)}
# (n, k): a ragged K (a 64-tail) on three widths, and whole k tiles where the
# 256x384 tile (K a multiple of 64, N of 384) can be chosen
CONFIG_SHAPES = [(4096, 1032), (6144, 1032), (24576, 1032), (6144, 1024), (24576, 1024)]


@pytest.mark.parametrize("b_is_nk", [False, True])
@pytest.mark.parametrize("n,k", CONFIG_SHAPES)
def test_mm_every_tile_configuration_same_bits(lib, b_is_nk, n, k):
    """A row's addmm output is the same, bit for bit, at an M of each tile
    configuration the shape takes (skinny 32 or 64 rows, the 64x128 and
    128x128 rings, 128x128, 256x256, 256x384), at the first and last row, for
    fp32 and bf16 outputs, with a ragged K (a 64-tail) or whole k tiles -- and
    it matches the oracle."""
    first = {}
    for m in range(1, 4097):
        first.setdefault(lib.bi_gemm_config(m, n, k, b_is_nk), m)
    say(f"configs for k={k} n={n} nk={b_is_nk}: {first}")
    assert len(first) >= 4, first
    w = S.normal_bf16((n, k) if b_is_nk else (k, n), 1 / k, seed=71, device=DEV)
    bias = S.normal_bf16((n,), 0.1, seed=72, device=DEV)
    row = S.normal_bf16((1, k), 1.0, seed=73, device=DEV)[0]
    for od in (torch.float32, torch.bfloat16):
        ref = lib.bi_addmm(bias, row[None], w, b_is_nk=b_is_nk, out_dtype=od, beta=0.5, alpha=1.5)[0].clone()
        if od == torch.float32:
            want = 0.5 * O.bf16_bits_to_f64(bits(bias)) + 1.5 * O.mm(bits(row[None]), bits(w), b_is_nk=b_is_nk)[0]
            assert_close(f32(ref[None]), want[None], "addmm row vs oracle")
        for cfg, m0 in first.items():
            for m in sorted({m0, m0 + 1, m0 + cfg[0] + 3}):
                if lib.bi_gemm_config(m, n, k, b_is_nk) != cfg:
                    continue
                for pos in (0, m - 1):
                    x = with_row(m, k, row, pos, seed=900 + m)
                    c = lib.bi_addmm(bias, x, w, b_is_nk=b_is_nk, out_dtype=od, beta=0.5, alpha=1.5)
                    assert same_bits(c[pos], ref), (cfg, m, pos, od)


def test_every_tile_configuration_is_exercised(lib):
    """The shapes of the test above take every configuration of the table between them."""
    seen = {lib.bi_gemm_config(m, n, k, nk) for n, k in CONFIG_SHAPES for nk in (False, True)
            for m in range(1, 4097)}
    assert seen == ALL_CONFIGS, seen


@pytest.mark.parametrize("b_is_nk", [False, True])
@pytest.mark.parametrize("m,k,n,slab,second", [(4096, 1032, 6144, 2048, 128), (4096, 1032, 6136, 2048, 128),
                                                (769, 4096, 151936, 131072, 128), (256, 4096, 151936, 131072, 256)])
def test_mm_column_split_same_bits(lib, b_is_nk, m, k, n, slab, second):
    """A GEMM in two launches over its columns: a 256x256 GEMM whose last
    round over the CUs would be part-empty runs its leftover columns as
    256x128 tiles (N = 6136: the last of them ragged, 120 columns), and a wide
    one (the LM head at M = 256) its first columns as 256x384 tiles in whole
    rounds and the rest as 256x256 tiles. Each column block of its output
    must have the bits of the same block computed on its own (other plans),
    for fp32 and bf16 outputs with a bias, and sampled rows of the second
    launch's columns match the oracle."""
    plan = lib.bi_gemm_plan(m, n, k, b_is_nk)
    assert len(plan) == 2 and plan[1][:2] == (256, second), plan
    w = S.normal_bf16((n, k) if b_is_nk else (k, n), 1 / k, seed=81, device=DEV)
    bias = S.normal_bf16((n,), 0.1, seed=82, device=DEV)
    a = S.normal_bf16((m, k), 1.0, seed=83, device=DEV)
    for od in (torch.float32, torch.bfloat16):
        full = lib.bi_addmm(bias, a, w, b_is_nk=b_is_nk, out_dtype=od, beta=0.5, alpha=1.5)
        for c0 in range(0, n, slab):
            c1 = min(n, c0 + slab)
            ws = w[c0:c1] if b_is_nk else w[:, c0:c1]
            part = lib.bi_addmm(bias[c0:c1], a, ws, b_is_nk=b_is_nk, out_dtype=od, beta=0.5, alpha=1.5)
            assert same_bits(full[:, c0:c1], part), (od, c0)
        if od == torch.float32:  # sampled rows of the second launch's columns against the oracle
            rows, ct = [0, m // 2 + 1, m - 1], plan[1][4]
            wt = w[ct:] if b_is_nk else w[:, ct:]
            want = 0.5 * O.bf16_bits_to_f64(bits(bias[ct:]))[None] + 1.5 * O.mm(bits(a[rows]), bits(wt), b_is_nk=b_is_nk)
            assert_close(f32(full[rows][:, ct:]), want, "split addmm rows vs oracle")
        del full, part



QWEN = [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)]


@pytest.mark.parametrize("k,n", QWEN)
def test_mm_qwen_shapes_invariant(lib, k, n):
    """Qwen3-8B projection shapes: config Ms, tile boundaries, random Ms."""
    rng = np.random.default_rng(k + n)
    ms = {1, 2, 8, 64, 65, 256, 257, 512, 4096, *rng.integers(2, 4097, size=4).tolist()}
    # the tile boundaries of every configuration the shape takes, and the Ms where the configuration changes
    prev = None
    for m in range(1, 4097):
        cfg = lib.bi_gemm_config(m, n, k)
        if cfg != prev:
            ms |= {m - 1, m}
            prev = cfg
    for tm in {lib.bi_gemm_config(m, n, k)[0] for m in (1, 64, 512, 4096)}:
        ms |= {tm - 1, tm, tm + 1, 2 * tm + 1}
    ms = sorted(x for x in ms if 1 <= x <= 4096)
    say(f"qwen invariance k={k} n={n} ms={ms}")
    bad = gemm_sweep(lib, k, n, ms)
    assert not bad, bad


def test_mm_nk_layout_and_bf16_invariant(lib):
    bad = gemm_sweep(lib, 4096, 4096, [1, 7, 129, 1000], b_is_nk=True)
    assert not bad, bad
    bad = gemm_sweep(lib, 4096, 4096, [1, 7, 129, 1000], out_dtype=torch.bfloat16)
    assert not bad, bad


def test_addmm_lm_head_invariant(lib):
    k, n = 4096, 151936
    w = S.normal_bf16((k, n), 0.02, seed=51, device=DEV)
    bias = S.normal_bf16((n,), 0.1, seed=52, device=DEV)
    row = S.normal_bf16((1, k), 1.0, seed=53, device=DEV)[0]
    ref = lib.bi_addmm(bias, row[None], w)[0].clone()
    lp_ref, am_ref = lib.bi_log_softmax(ref[None].contiguous())
    for m in (32, 256):
        say(f"lm head invariance m={m}")
        x = with_row(m, k, row, m // 3, seed=54 + m)
        logits = lib.bi_addmm(bias, x, w)
        assert same_bits(logits[m // 3], ref)
        lp, am = lib.bi_log_softmax(logits)
        assert same_bits(lp[m // 3], lp_ref[0]) and am[m // 3].item() == am_ref[0].item()


def test_mm_repeat_100(lib):
    x = S.normal_bf16((512, 4096), 1.0, seed=60, device=DEV)
    w = S.normal_bf16((4096, 4096), 0.02, seed=61, device=DEV)
    first = lib.bi_mm(x, w)
    h = digest(first)
    for _ in range(99):
        assert same_bits(lib.bi_mm(x, w), first)
    say("mm sha256", h)


# ------------------------------------------------------------------ reductions
def test_rows_reductions_invariant(lib):
    n = 4096
    w = S.uniform_bf16((n,), 0.5, 1.5, seed=61, device=DEV)
    row = S.normal_bf16((1, n), 1.0, seed=62, device=DEV)[0]
    ref_y = lib.bi_rmsnorm(row[None], w, 1e-6)[0].clone()
    ref_yf = lib.bi_rmsnorm(row[None], w, 1e-6, out_dtype=torch.float32)[0].clone()
    ref_mean = lib.bi_mean(row[None])[0].clone()
    for m in (1, 2, 7, 64, 513, 2048):
        for fill in ("random", "zeros", "huge", "nan"):
            for pos in sorted({0, m - 1, m // 2}):
                x = with_row(m, n, row, pos, seed=63 + m, fill=fill)
                assert same_bits(lib.bi_rmsnorm(x, w, 1e-6)[pos], ref_y), ("rmsnorm", m, fill, pos)
                assert same_bits(lib.bi_rmsnorm(x, w, 1e-6, out_dtype=torch.float32)[pos], ref_yf)
                assert same_bits(lib.bi_mean(x)[pos], ref_mean), ("mean", m, fill, pos)


def test_log_softmax_invariant(lib):
    n = 151936
    row = S.normal_f32((1, n), 4.0, seed=70, device=DEV)[0]
    ref_y, ref_a = lib.bi_log_softmax(row[None].contiguous())
    for m in (1, 7, 64, 513):
        for fill in ("random", "zeros", "nan"):
            pos = (m * 3) // 5
            x = with_row(m, n, row, pos, seed=71 + m, fill=fill, dtype=torch.float32)
            y, a = lib.bi_log_softmax(x)
            assert same_bits(y[pos], ref_y[0]), (m, fill)
            assert a[pos].item() == ref_a[0].item()


def test_reductions_repeat_100(lib):
    x = S.normal_bf16((2048, 4096), 1.0, seed=80, device=DEV)
    w = S.uniform_bf16((4096,), 0.5, 1.5, seed=81, device=DEV)
    lg = S.normal_f32((64, 151936), 4.0, seed=82, device=DEV)
    y0, m0 = lib.bi_rmsnorm(x, w, 1e-6), lib.bi_mean(x)
    l0, a0 = lib.bi_log_softmax(lg)
    for _ in range(99):
        assert same_bits(lib.bi_rmsnorm(x, w, 1e-6), y0)
        assert same_bits(lib.bi_mean(x), m0)
        l1, a1 = lib.bi_log_softmax(lg)
        assert same_bits(l1, l0) and same_bits(a1, a0)


# ------------------------------------------------------------------ decode attention
def test_decode_batch_composition_invariant(lib):
    """A sequence's output is the same bytes alone, in batches of other
    sequences, at other batch positions and with other page placements."""
    hq, hkv, d, page = 32, 8, 128, 16
    target_len = 5000
    qx = S.normal_bf16((hq, d), 1.0, seed=90)
    kx = S.normal_bf16((target_len, hkv, d), 1.0, seed=91)   # the target's tokens
    vx = S.normal_bf16((target_len, hkv, d), 1.0, seed=92)

    def batch(other_lens, pos, seed):
        lens = list(other_lens)
        lens.insert(pos, target_len)
        lens_t = torch.tensor(lens, dtype=torch.int32)
        table, npages = S.paged_kv_layout(lens_t, page, seed=seed)
        kp = S.normal_bf16((npages, hkv, page, d), 1.0, seed=seed + 1)
        vp = S.normal_bf16((npages, hkv, page, d), 1.0, seed=seed + 2)
        for t in range(target_len):              # place the target's tokens
            p = table[pos, t // page]
            kp[p, :, t % page] = kx[t]
            vp[p, :, t % page] = vx[t]
        q = S.normal_bf16((len(lens), hq, d), 1.0, seed=seed + 3)
        q[pos] = qx
        offs, total = lib.bi_decode_plan(lens_t)
        out = lib.bi_decode_attention(q.to(DEV), kp.to(DEV), d_major(vp).to(DEV), table.to(DEV), lens_t.to(DEV),
                                      offs.to(DEV), total)
        return out[pos].cpu()

    ref = batch([], 0, seed=200)
    cases = [([1], 1, 210), ([300, 7, 32768], 2, 220), (S.context_lens(63, seed=5).tolist(), 40, 230),
             ([5000] * 3, 0, 240)]
    for others, pos, seed in cases:
        say(f"decode composition B={len(others) + 1} pos={pos}")
        assert same_bits(batch(others, pos, seed), ref), (len(others), pos)


def test_decode_repeat_100(lib):
    lens_t = S.context_lens(32, seed=300)
    table, npages = S.paged_kv_layout(lens_t, 16, seed=301)
    q = S.normal_bf16((32, 32, 128), 1.0, seed=302, device=DEV)
    kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=303, device=DEV)
    vp = d_major(S.normal_bf16((npages, 8, 16, 128), 1.0, seed=304, device=DEV))
    offs, total = lib.bi_decode_plan(lens_t)
    args = (q, kp, vp, table.to(DEV), lens_t.to(DEV), offs.to(DEV), total)
    first = lib.bi_decode_attention(*args)
    for _ in range(99):
        assert same_bits(lib.bi_decode_attention(*args), first)


# ------------------------------------------------------------------ negative control
def test_harness_detects_one_flipped_bit():
    a = torch.randn(64)
    b = a.clone()
    b.view(torch.int32)[17] ^= 1
    assert not same_bits(a, b) and same_bits(a, a.clone())


def test_negative_control_torch_kernels(lib):
    """The same harness on torch's own (non-invariant) kernels. The count is
    reported, not asserted: whether a vendor library changes its reduction
    with M is its own business; the test only shows the harness can see it."""
    k, n = 4096, 4096
    w = S.normal_bf16((k, n), 0.02, seed=7, device=DEV)
    row = S.normal_bf16((1, k), 1.0, seed=11, device=DEV)[0]
    ref = (row[None] @ w)[0].float()
    changed = []
    for m in (2, 8, 64, 512, 4096):
        x = with_row(m, k, row, 0, seed=m)
        if not same_bits((x @ w)[0].float(), ref):
            changed.append(m)
    lg = S.normal_f32((1, 151936), 4.0, seed=3, device=DEV)
    ref_l = torch.log_softmax(lg, dim=-1)[0]
    lchanged = []
    for m in (2, 64, 513):
        x = with_row(m, 151936, lg[0], 0, seed=m, dtype=torch.float32)
        if not same_bits(torch.log_softmax(x, dim=-1)[0], ref_l):
            lchanged.append(m)
    say(f"negative control: torch.mm row 0 changed at M={changed}; log_softmax at M={lchanged}")
