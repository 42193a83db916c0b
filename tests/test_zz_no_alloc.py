"""bi_decode_attention_noalloc: decode attention with the library's own
scratch for the split partials, for callers that cannot allocate.

Through the C ABI it must give the bytes bi_decode_attention gives with a
caller's workspace (the same kernels), on two calls in a row, the second
with a smaller batch (the scratch still holds the first call's partials),
match the oracle, and refuse a call whose partials exceed the scratch
without launching anything.
"""
import pytest
import torch

import oracle as O
import synthetic as S
from helpers import assert_close, bits, f32, same_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def _case(lib, lens, seed):
    lens_t = torch.tensor(lens, dtype=torch.int32)
    table, npages = S.paged_kv_layout(lens_t, 16, seed=seed)
    q = S.normal_bf16((len(lens), 32, 128), 1.0, seed=seed + 1, device=DEV)
    kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=seed + 2, device=DEV)
    vp = S.normal_bf16((npages, 8, 128, 16), 1.0, seed=seed + 3, device=DEV)  # d-major value pages
    offs, total = lib.bi_decode_plan(lens_t)
    return lens_t, table, q, kp, vp, offs, total


def test_noalloc_decode_attention_equals_workspace_entry_point(lib):
    for lens, seed in (([4097, 1, 300, 32768, 255, 17, 9000, 2048], 60100), ([700, 3], 60200)):
        lens_t, table, q, kp, vp, offs, total = _case(lib, lens, seed)
        need = lib.bi_decode_workspace_bytes(total, 32, 128)
        say(f"noalloc: batch {len(lens)}, {total} splits, {need} bytes of partials")
        assert need <= lib.BI_DECODE_NOALLOC_MAX_BYTES
        args = (q, kp, vp, table.to(DEV), lens_t.to(DEV), offs.to(DEV), total)
        for od in (torch.float32, torch.bfloat16):
            ref = lib.bi_decode_attention(*args, out_dtype=od)
            out = torch.full_like(ref, float("nan"))
            lib.bi_decode_attention_noalloc(*args, out)
            torch.cuda.synchronize()
            assert same_bits(out, ref), (lens, od)
            if od == torch.float32:
                seqs = [0, len(lens) - 1]
                want = O.decode_attention(bits(q), bits(kp), bits(vp), table.numpy(), lens_t.numpy(), 128 ** -0.5,
                                          seqs=seqs)
                assert_close(f32(out[seqs]), want[seqs], "noalloc vs oracle")


def test_noalloc_refuses_partials_beyond_the_scratch(lib):
    """32 sequences of 32768 tokens: 4096 splits of 32 heads need more than
    the scratch holds; the call is refused before anything is launched (no
    cache is read: the pages passed are never touched)."""
    bsz, max_pages = 32, 2048
    lens_t = torch.full((bsz,), 32768, dtype=torch.int32)
    offs, total = lib.bi_decode_plan(lens_t)
    assert lib.bi_decode_workspace_bytes(total, 32, 128) > lib.BI_DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((bsz, 32, 128), dtype=torch.bfloat16, device=DEV)
    kp = torch.zeros((1, 8, 16, 128), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros((1, 8, 128, 16), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((bsz, max_pages), dtype=torch.int32, device=DEV)
    out = torch.full((bsz, 32, 128), 7.0, device=DEV)
    with pytest.raises(lib.BiError) as e:
        lib.bi_decode_attention_noalloc(q, kp, vp, table, lens_t.to(DEV), offs.to(DEV), total, out)
    assert e.value.name == "BI_ERR_WORKSPACE" and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
