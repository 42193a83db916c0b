"""Prefill / extend attention on the GPU.

A chunk token at position p must get exactly the bits a decode step with
p + 1 cached tokens gives it: same 256-token split boundaries, same
per-split arithmetic, same combine. Checked directly (prefill vs decode
bitwise), together with parity against the fp64 causal-attention oracle,
independence from how a prompt is chunked, and from the other sequences in
the batch (the chunked-prefill form of the batch dependence the pages trace
to attention: readhandoff.com, agent-run reproducibility pinning, "What does
temperature zero actually guarantee?").
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from helpers import assert_close, bits, d_major, f32, same_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"
HQ, HKV, D, PAGE = 32, 8, 128, 16


def say(*a):
    print(*a, flush=True)


def cache_for(total_lens, seed):
    """Pages for sequences of the given total lengths (cache already holding every token)."""
    lens = torch.tensor(total_lens, dtype=torch.int32)
    table, npages = S.paged_kv_layout(lens, PAGE, seed=seed)
    kp = S.normal_bf16((npages, HKV, PAGE, D), 1.0, seed=seed + 1, device=DEV)
    vp = d_major(S.normal_bf16((npages, HKV, PAGE, D), 1.0, seed=seed + 2, device=DEV))
    return table, kp, vp


def prefill(lib, q, kp, vp, table, chunk, ctx, out_dtype=torch.float32):
    q_pos, q_offs, work, sizes = lib.bi_prefill_plan(torch.tensor(chunk), torch.tensor(ctx))
    out = lib.bi_prefill_attention(q, kp, vp, table.to(DEV), q_pos.to(DEV), q_offs.to(DEV), work.to(DEV), sizes,
                                   out_dtype=out_dtype)
    return out, q_pos


def decode_rows(lib, q, kp, vp, table, seq_of_row, pos, out_dtype=torch.float32):
    """Each chunk row as its own decode step: context length pos + 1, its sequence's block-table row."""
    tb = table[torch.as_tensor(seq_of_row)].contiguous()
    lens = (torch.as_tensor(pos) + 1).to(torch.int32)
    offs, total = lib.bi_decode_plan(lens)
    return lib.bi_decode_attention(q, kp, vp, tb.to(DEV), lens.to(DEV), offs.to(DEV), total, out_dtype=out_dtype)


def test_prefill_parity_with_oracle(lib):
    chunk, ctx = [3, 40, 9], [0, 230, 500]  # crosses split 1 (256) and split 2 (512)
    table, kp, vp = cache_for([c + n for c, n in zip(ctx, chunk)], seed=6000)
    q = S.normal_bf16((sum(chunk), HQ, D), 1.0, seed=6010, device=DEV)
    out, q_pos = prefill(lib, q, kp, vp, table, chunk, ctx)
    seq = np.repeat(np.arange(3), chunk)
    ref = O.prefill_attention(bits(q), bits(kp), bits(vp), table.numpy(), seq, q_pos.numpy(), D ** -0.5)
    assert_close(f32(out), ref, "prefill vs oracle")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("chunk,ctx", [([1, 300, 17, 600], [0, 0, 255, 1000]),
                                       # rows of 8 and 9 splits around position 2048, and of 17 and 33
                                       ([40, 8, 5], [2030, 4200, 8190])],
                         ids=["up_to_7_splits", "8_to_33_splits"])
def test_prefill_equals_decode_bitwise(lib, out_dtype, chunk, ctx):
    table, kp, vp = cache_for([c + n for c, n in zip(ctx, chunk)], seed=6100)
    q = S.normal_bf16((sum(chunk), HQ, D), 1.0, seed=6110, device=DEV)
    out, q_pos = prefill(lib, q, kp, vp, table, chunk, ctx, out_dtype)
    seq = np.repeat(np.arange(len(chunk)), chunk)
    dec = decode_rows(lib, q, kp, vp, table, seq, q_pos, out_dtype)
    diff = [r for r in range(sum(chunk)) if not same_bits(out[r], dec[r])]
    say(f"rows differing from decode: {len(diff)} of {sum(chunk)}")
    assert not diff


def test_prefill_independent_of_chunking_and_batch(lib):
    prompt = 700
    table, kp, vp = cache_for([prompt, 900, 50], seed=6200)
    q_all = S.normal_bf16((prompt, HQ, D), 1.0, seed=6210, device=DEV)
    whole, _ = prefill(lib, q_all, kp, vp, table[:1], [prompt], [0])
    # the same prompt in three chunks (each call sees the cache as it would then be: rows attend only up to
    # their own position, so later tokens already in the cache are never read)
    parts, start = [], 0
    for n in (100, 333, 267):
        o, _ = prefill(lib, q_all[start:start + n].contiguous(), kp, vp, table[:1], [n], [start])
        parts.append(o)
        start += n
    assert same_bits(torch.cat(parts), whole)
    # the middle chunk inside a batch with two other sequences' chunks, before and after it
    q_other1 = S.normal_bf16((64, HQ, D), 1.0, seed=6220, device=DEV)
    q_other2 = S.normal_bf16((50, HQ, D), 1.0, seed=6230, device=DEV)
    qb = torch.cat([q_other1, q_all[100:433], q_other2]).contiguous()
    tb = torch.stack([table[1], table[0], table[2]])
    ob, _ = prefill(lib, qb, kp, vp, tb, [64, 333, 50], [836, 100, 0])
    assert same_bits(ob[64:64 + 333], parts[1])


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_prefill_unaligned_out_same_bits(lib, dt):
    """An output one element past a 16-byte boundary (element stores) gets
    the bits of an aligned one (vector stores)."""
    chunk, ctx = [40, 9], [230, 500]
    table, kp, vp = cache_for([c + n for c, n in zip(ctx, chunk)], seed=6200)
    q = S.normal_bf16((sum(chunk), HQ, D), 1.0, seed=6210, device=DEV)
    aligned, _ = prefill(lib, q, kp, vp, table, chunk, ctx, dt)
    q_pos, q_offs, work, sizes = lib.bi_prefill_plan(torch.tensor(chunk), torch.tensor(ctx))
    buf = torch.full((1 + sum(chunk) * HQ * D,), 7.0, dtype=dt, device=DEV)
    out = buf[1:].view(sum(chunk), HQ, D)
    assert out.data_ptr() % 16 != 0
    lib.bi_prefill_attention(q, kp, vp, table.to(DEV), q_pos.to(DEV), q_offs.to(DEV), work.to(DEV), sizes, out=out)
    say("prefill unaligned out", dt)
    assert same_bits(out, aligned)
    assert buf[0].item() == 7.0


def test_prefill_inconsistent_plan_stays_in_bounds(lib):
    """The plan's arrays live on the device, where the host cannot check them: work items whose row
    range, sequence, split or pages do not fit the buffers, and split offsets past the workspace, are
    skipped by the kernels (their rows' values are then unspecified), never followed outside the buffers.
    A correct call afterwards still gives decode's bits."""
    chunk, ctx = [40, 9, 30], [200, 500, 700]  # 2 + 2 + 3 work items
    table, kp, vp = cache_for([c + n for c, n in zip(ctx, chunk)], seed=6300)
    q = S.normal_bf16((sum(chunk), HQ, D), 1.0, seed=6310, device=DEV)
    q_pos, q_offs, work, sizes = lib.bi_prefill_plan(torch.tensor(chunk), torch.tensor(ctx))
    rows, total, n_work = sizes
    bad = work.clone()
    assert n_work >= 5
    bad[0, 0] = -5                 # row before the first
    bad[1, 2] = 1_000_000          # sequence past the batch
    bad[2, 1] = 1000               # more rows than an item holds
    bad[3, 3] = 100_000            # a split no row of the item sees
    bad[4, 0], bad[4, 1] = rows - 1, 5  # rows past the last
    bad_offs = q_offs.clone()
    bad_offs[3] = 1 << 30          # a row whose split slots lie past the workspace
    out = lib.bi_prefill_attention(q, kp, vp, table.to(DEV), q_pos.to(DEV), bad_offs.to(DEV), bad.to(DEV), sizes)
    torch.cuda.synchronize()
    assert out.shape == (rows, HQ, D)
    good, pos = prefill(lib, q, kp, vp, table, chunk, ctx)
    seq = np.repeat(np.arange(len(chunk)), chunk)
    dec = decode_rows(lib, q, kp, vp, table, seq, pos)
    assert all(same_bits(good[r], dec[r]) for r in range(rows))


def test_prefill_large_workspace_equals_decode_bitwise(lib):
    """A workspace of 2 GiB or more takes the split kernel's plain-store path (smaller ones use buffer
    stores through one 32-bit-addressed resource): 2048 chunk tokens at positions 16384.. see 65-72
    splits each, ~140k split slots, a 2.3 GB workspace. Sampled rows have decode's bits."""
    chunk, ctx = [2048], [16384]
    table, kp, vp = cache_for([ctx[0] + chunk[0]], seed=6400)
    q = S.normal_bf16((chunk[0], HQ, D), 1.0, seed=6410, device=DEV)
    q_pos, q_offs, work, sizes = lib.bi_prefill_plan(torch.tensor(chunk), torch.tensor(ctx))
    rows, total, n_work = sizes
    need = lib.bi_decode_workspace_bytes(total, HQ, D)
    say(f"split slots {total}, workspace {need / 2**30:.2f} GiB")
    assert need >= 2 ** 31
    out = lib.bi_prefill_attention(q, kp, vp, table.to(DEV), q_pos.to(DEV), q_offs.to(DEV), work.to(DEV), sizes)
    rng = np.random.default_rng(6420)
    sample = np.unique(np.concatenate([[0, 1, 255, 256, rows - 1], rng.integers(0, rows, 59)]))
    dec = decode_rows(lib, q[sample].contiguous(), kp, vp, table, np.zeros(len(sample), dtype=np.int64),
                      q_pos[sample])
    diff = [int(r) for k, r in enumerate(sample) if not same_bits(out[r], dec[k])]
    say(f"sampled rows differing from decode: {len(diff)} of {len(sample)}")
    assert not diff
