"""Exhaustive batch-invariance sweep on the shapes whose tile configuration
changes with M.

The defect the pages describe is a kernel whose result for one sequence
changes with the size of the batch it is computed in (readhandoff.com,
agent-run reproducibility pinning, "What does temperature zero actually
guarantee?"); the property wanted is outputs that do not depend on the batch
size ("Batch-invariant inference kernels (Thinking Machines) -- Evidence &
limits", "Rubric assessment"). The GEMM picks its tile configuration from
(M, N, K), and on the Qwen3-8B projection shapes that choice changes up to
eight times between M = 1 and 4096 (the LM head's also splits its last
columns onto 256x128 tiles from M = 192). So every M = 1..4096 is run on each
of the projection shapes, both weight layouts, fp32 and bf16 outputs:

* a fixed row, placed at positions 0, M - 1 and a seeded p, must have the
  bytes it has at M = 1;
* the other rows are fresh for every M (a seeded offset into a large random
  block);
* the fixed-tile mode (one configuration for every M) must give the whole
  output the same bytes as the table.

Then the LM head (addmm, log_softmax, argmax) at every M = 1..256. The
configurations visited are printed. Comparisons are accumulated on the GPU
and read once at the end of each case.
"""
import numpy as np
import pytest
import torch

import synthetic as S

pytestmark = pytest.mark.gpu
DEV = "cuda"

QWEN = [(4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)]


def say(*a):
    print(*a, flush=True)


def as_int(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def positions(rng, mmax):
    """Per M = 1..mmax: (offset into the random block, [0, M - 1, p])."""
    offs = rng.integers(0, 8192, size=mmax)
    ps = np.array([rng.integers(0, m) for m in range(1, mmax + 1)])
    pos = np.stack([np.zeros(mmax, dtype=np.int64), np.arange(mmax), ps], axis=1)
    return offs.tolist(), torch.from_numpy(pos).to(DEV)


def plan_key(lib, m, n, k, nk):
    return tuple(p[:4] for p in lib.bi_gemm_plan(m, n, k, nk))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("b_is_nk", [False, True], ids=["kn", "nk"])
@pytest.mark.parametrize("k,n", QWEN, ids=[f"k{k}_n{n}" for k, n in QWEN])
def test_mm_every_m_qwen_shape(lib, k, n, b_is_nk, out_dtype):
    seed = 40000 + k + n + (7 if b_is_nk else 0)
    rng = np.random.default_rng(seed)
    w = S.normal_bf16((n, k) if b_is_nk else (k, n), 0.02, seed=seed + 1, device=DEV)
    row = S.normal_bf16((1, k), 1.0, seed=seed + 2, device=DEV)[0]
    ref = as_int(lib.bi_mm(row[None], w, b_is_nk=b_is_nk, out_dtype=out_dtype)[0].clone())
    big = S.normal_bf16((8192 + 4096, k), 1.0, seed=seed + 3, device=DEV)
    out = torch.empty((4096, n), dtype=out_dtype, device=DEV)
    outf = torch.empty_like(out)
    bad = torch.zeros((4096, 3), dtype=torch.bool, device=DEV)
    fixed_bad = torch.zeros(4096, dtype=torch.bool, device=DEV)
    offs, pos = positions(rng, 4096)
    plans = {}
    say(f"every M: k={k} n={n} b_is_nk={b_is_nk} out={out_dtype}")
    for m in range(1, 4097):
        x = big[offs[m - 1]:offs[m - 1] + m].clone()
        p = pos[m - 1]
        x[p] = row
        c = lib.bi_mm(x, w, b_is_nk=b_is_nk, out_dtype=out_dtype, out=out[:m])
        bad[m - 1] = (as_int(c[p]) != ref).any(dim=1)
        cf = lib.bi_gemm(x, w, b_is_nk=b_is_nk, out_dtype=out_dtype, fixed_tile=True, out=outf[:m])
        fixed_bad[m - 1] = (as_int(cf) != as_int(c)).any()
        plans.setdefault(plan_key(lib, m, n, k, b_is_nk), []).append(m)
        if m % 1024 == 0:
            torch.cuda.synchronize()
            say(f"  M up to {m}: {int(bad.sum())} changed rows, {int(fixed_bad.sum())} fixed-tile differences")
    for key, ms in plans.items():
        say(f"  launches {key}: M = {ms[0]}..{ms[-1]} ({len(ms)} values)")
    say(f"  fixed-tile configuration: {lib.bi_gemm_plan(1, n, k, b_is_nk, fixed_tile=True)}")
    changed = bad.nonzero().tolist()
    assert not changed, f"fixed row changed at (M - 1, position slot) {changed[:20]}"
    diff = fixed_bad.nonzero().flatten().tolist()
    assert not diff, f"fixed-tile mode differs from the table at M - 1 = {diff[:20]}"
    assert len(plans) >= 4


@pytest.mark.parametrize("b_is_nk", [False, True], ids=["kn", "nk"])
def test_lm_head_every_m_up_to_256(lib, b_is_nk):
    """addmm + log_softmax + argmax of the LM head (K = 4096, N = 151936) at
    every M = 1..256: the fixed row's logits, log-probabilities and greedy
    token at positions 0, M - 1 and p equal its M = 1 results, and the
    fixed-tile mode gives the same logits."""
    k, n = 4096, 151936
    seed = 41000 + (7 if b_is_nk else 0)
    rng = np.random.default_rng(seed)
    w = S.normal_bf16((n, k) if b_is_nk else (k, n), 0.02, seed=seed + 1, device=DEV)
    bias = S.normal_bf16((n,), 0.1, seed=seed + 2, device=DEV)
    row = S.normal_bf16((1, k), 1.0, seed=seed + 3, device=DEV)[0]
    ref = lib.bi_addmm(bias, row[None], w, b_is_nk=b_is_nk)
    ref_lp, ref_am = lib.bi_log_softmax(ref)
    ref, ref_lp = as_int(ref[0].clone()), as_int(ref_lp[0].clone())
    big = S.normal_bf16((8192 + 256, k), 1.0, seed=seed + 4, device=DEV)
    logits = torch.empty((256, n), device=DEV)
    logits_f = torch.empty_like(logits)
    lp = torch.empty_like(logits)
    am = torch.empty(256, dtype=torch.int64, device=DEV)
    bad = torch.zeros((256, 3, 3), dtype=torch.bool, device=DEV)
    fixed_bad = torch.zeros(256, dtype=torch.bool, device=DEV)
    offs, pos = positions(rng, 256)
    plans = {}
    say(f"LM head every M: b_is_nk={b_is_nk}")
    for m in range(1, 257):
        x = big[offs[m - 1]:offs[m - 1] + m].clone()
        p = pos[m - 1]
        x[p] = row
        c = lib.bi_addmm(bias, x, w, b_is_nk=b_is_nk, out=logits[:m])
        y, a = lib.bi_log_softmax(c, out=lp[:m], argmax=am[:m])
        bad[m - 1, :, 0] = (as_int(c[p]) != ref).any(dim=1)
        bad[m - 1, :, 1] = (as_int(y[p]) != ref_lp).any(dim=1)
        bad[m - 1, :, 2] = a[p] != ref_am[0]
        cf = lib.bi_gemm(x, w, bias, b_is_nk=b_is_nk, fixed_tile=True, out=logits_f[:m])
        fixed_bad[m - 1] = (as_int(cf) != as_int(c)).any()
        plans.setdefault(plan_key(lib, m, n, k, b_is_nk), []).append(m)
    torch.cuda.synchronize()
    for key, ms in plans.items():
        say(f"  launches {key}: M = {ms[0]}..{ms[-1]} ({len(ms)} values)")
    changed = bad.nonzero().tolist()
    assert not changed, f"fixed row changed at (M - 1, slot, [logits, log-probs, argmax]) {changed[:20]}"
    diff = fixed_bad.nonzero().flatten().tolist()
    assert not diff, f"fixed-tile mode differs from the table at M - 1 = {diff[:20]}"


@pytest.mark.parametrize("n,ms", [(8203, range(1, 2049)), (151936, list(range(1, 257)) + [511, 512, 1024, 2048])],
                         ids=["n8203_every_m", "n151936"])
def test_log_softmax_forms_same_bits_every_m(lib, n, ms):
    """log_softmax + argmax gives each of a row's 16 wave partials a
    workgroup of its own for small M (three launches) and gives each row one
    workgroup otherwise; both forms compute the same partials and merge them
    in the same order. A fixed row at positions 0, M - 1 and p, other rows
    fresh per M: its log-probabilities and greedy token have the bytes they
    have at M = 1, at every M listed (n = 8203: a partial last unit)."""
    ld = (n + 3) // 4 * 4
    ms = list(ms)
    mmax = max(ms)
    rng = np.random.default_rng(n)
    row = S.normal_f32((1, n), 4.0, seed=42000 + n, device=DEV)[0]
    r1 = torch.zeros((1, ld), device=DEV)[:, :n]  # rows 16-byte aligned
    r1.copy_(row[None])
    y1, a1 = lib.bi_log_softmax(r1, out=torch.empty((1, ld), device=DEV)[:, :n])
    ref, ref_a = as_int(y1[0].clone()), int(a1[0])
    nblk = min(8192, 4 * mmax)
    big = S.normal_f32((nblk + mmax, ld), 4.0, seed=42100 + n, device=DEV)
    ybuf = torch.empty((mmax, ld), device=DEV)
    abuf = torch.empty(mmax, dtype=torch.int64, device=DEV)
    bad = torch.zeros((len(ms), 3, 2), dtype=torch.bool, device=DEV)
    offs = rng.integers(0, nblk, size=len(ms)).tolist()
    pos = torch.from_numpy(np.array([[0, m - 1, rng.integers(0, m)] for m in ms])).to(DEV)
    say(f"log_softmax every M: n={n}, {len(ms)} values of M up to {mmax}")
    for i, m in enumerate(ms):
        x = big[offs[i]:offs[i] + m].clone()
        p = pos[i]
        x[p, :n] = row
        y, a = lib.bi_log_softmax(x[:, :n], out=ybuf[:m, :n], argmax=abuf[:m])
        bad[i, :, 0] = (as_int(y[p]) != ref).any(dim=1)
        bad[i, :, 1] = a[p] != ref_a
        if (i + 1) % 256 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    changed = bad.nonzero().tolist()
    assert not changed, f"(index into M list, slot, [log-probs, argmax]) {changed[:20]}"
