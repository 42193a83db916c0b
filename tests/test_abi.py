"""C-ABI library tests that need no GPU: the library loads, exports every
symbol include/bi.h declares, rejects invalid arguments with the documented
status before any HIP call, treats empty batches as no-ops, and the host
plan is right. Also: only one HIP runtime is mapped after loading it."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bi.h")

OK, NULL, SHAPE, STRIDE, ALIGN, DTYPE, WORKSPACE, UNSUPPORTED, HIP = range(9)
A16 = 0x10000   # fake, 16-byte aligned device address (never dereferenced:
A2 = 0x10002    # every call below fails validation or is a no-op)


@pytest.fixture(scope="module")
def bi():
    import invariant_bi_mm_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(bi):
    names = declared_functions()
    assert {"bi_mm", "bi_addmm", "bi_rmsnorm", "bi_mean", "bi_log_softmax", "bi_decode_plan",
            "bi_decode_workspace_bytes", "bi_decode_attention", "bi_status_string",
            "bi_last_error_message", "bi_gemm_config", "bi_add_rmsnorm", "bi_embed", "bi_silu_mul",
            "bi_qknorm_rope_append", "bi_prefill_plan", "bi_prefill_attention"} <= set(names)
    raw = ctypes.CDLL(bi.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), f"{n} declared in bi.h but not exported"


def test_single_hip_runtime_mapped(bi):
    maps = open("/proc/self/maps").read()
    hips = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(hips) == 1, hips


def test_status_strings(bi):
    texts = [bi.bi_status_string(s) for s in range(9)]
    assert len(set(texts)) == 9 and texts[0] == "BI_OK"
    assert "unknown" in bi.bi_status_string(99)


def mm(bi, a=A16, lda=512, b=A16, ldb=512, nk=0, c=A16, ldc=512, dt=1, m=4, n=512, k=512):
    return bi.lib.bi_mm(a, lda, b, ldb, nk, c, ldc, dt, m, n, k, None)


def test_mm_validation(bi):
    assert mm(bi, m=-1) == SHAPE
    assert mm(bi, dt=7) == DTYPE
    assert mm(bi, c=None) == NULL
    assert mm(bi, a=None) == NULL
    assert mm(bi, lda=100) == STRIDE
    assert mm(bi, ldc=511) == STRIDE
    assert mm(bi, ldb=500, nk=1) == STRIDE
    assert mm(bi, k=12, lda=16, ldb=512) == UNSUPPORTED            # k % 8
    assert mm(bi, n=12, ldb=16, ldc=16) == UNSUPPORTED             # n % 8 with B [k, n]
    assert mm(bi, a=A2) == ALIGN
    assert mm(bi, lda=516) == ALIGN
    assert mm(bi, c=A2 + 1) == ALIGN
    assert "aligned" in bi.bi_last_error_message()
    assert mm(bi, lda=1 << 24) == UNSUPPORTED                      # tile byte range >= 2^31
    assert mm(bi, lda=100) == STRIDE and "lda" in bi.bi_last_error_message()
    # no-ops: nothing launched, so fine without a GPU
    assert mm(bi, m=0) == OK and bi.bi_last_error_message() == ""
    assert mm(bi, n=0, m=5) == OK
    assert mm(bi, m=0, a=None, b=None, c=None) == OK


def test_addmm_validation(bi):
    f = bi.lib.bi_addmm
    assert f(None, 0, 1.0, 1.0, A16, 512, A16, 512, 0, A16, 512, 1, 4, 512, 512, None) == NULL
    assert f(A16, 9, 1.0, 1.0, A16, 512, A16, 512, 0, A16, 512, 1, 4, 512, 512, None) == DTYPE
    assert f(A2 + 1, 0, 1.0, 1.0, A16, 512, A16, 512, 0, A16, 512, 1, 4, 512, 512, None) == ALIGN
    assert f(A16, 0, 1.0, 1.0, A16, 512, A16, 512, 0, A16, 512, 1, 0, 512, 512, None) == OK


def test_rowreduce_validation(bi):
    L = bi.lib
    assert L.bi_rmsnorm(A16, 4096, A16, 1e-6, A16, 4096, 0, -1, 4096, None) == SHAPE
    assert L.bi_rmsnorm(A16, 4096, A16, 1e-6, A16, 4096, 0, 3, 0, None) == SHAPE
    assert L.bi_rmsnorm(A16, 4096, None, 1e-6, A16, 4096, 0, 3, 4096, None) == NULL
    assert L.bi_rmsnorm(A16, 4000, A16, 1e-6, A16, 4096, 0, 3, 4096, None) == STRIDE
    assert L.bi_rmsnorm(A16, 4100, A16, 1e-6, A16, 4096, 0, 3, 4096, None) == ALIGN
    assert L.bi_rmsnorm(A16, 4096, A16, 1e-6, A16, 4100, 0, 3, 4096, None) == ALIGN     # bf16 y needs ldy%8
    assert L.bi_rmsnorm(A16, 4096, A16, 1e-6, A16, 4096, 5, 3, 4096, None) == DTYPE
    assert L.bi_rmsnorm(None, 4096, None, 1e-6, None, 4096, 0, 0, 4096, None) == OK
    assert L.bi_mean(A16, 0, 4096, A16, 3, 0, None) == SHAPE
    assert L.bi_mean(A16, 3, 4096, A16, 3, 4096, None) == DTYPE
    assert L.bi_mean(A16, 1, 4098, A16, 3, 4096, None) == ALIGN
    assert L.bi_mean(None, 0, 4096, A16, 3, 4096, None) == NULL
    assert L.bi_mean(None, 0, 4096, None, 0, 4096, None) == OK
    assert L.bi_log_softmax(A16, 151936, A16, 151936, None, 2, 0, None) == SHAPE
    assert L.bi_log_softmax(A16, 151930, A16, 151936, None, 2, 151936, None) == STRIDE
    assert L.bi_log_softmax(A16, 151936, A16, 151936, A2, 2, 151936, None) == ALIGN
    assert L.bi_log_softmax(None, 151936, A16, 151936, None, 2, 151936, None) == NULL
    assert L.bi_log_softmax(None, 151936, None, 151936, None, 0, 151936, None) == OK


def test_rmsnorm_f32_out_ldy_multiple_of_4_is_not_misaligned(bi):
    # validation for fp32 y accepts ldy % 4 == 0; confirm by a call that then
    # fails on something else checked later (nothing is launched)
    L = bi.lib
    assert L.bi_rmsnorm(A16, 4096, A16, 1e-6, A2, 4100, 1, 3, 4096, None) == ALIGN  # y misaligned


def attn(bi, **kw):
    args = dict(q=A16, k=A16, v=A16, bt=A16, maxp=2048, lens=A16, offs=A16, total=256, batch=2, hq=32, hkv=8,
                d=128, page=16, split=256, scale=0.088, ws=A16, wsb=1 << 30, out=A16, dt=1, flags=0)
    args.update(kw)
    a = args
    return bi.lib.bi_decode_attention(a["q"], a["k"], a["v"], a["bt"], a["maxp"], a["lens"], a["offs"], a["total"],
                                      a["batch"], a["hq"], a["hkv"], a["d"], a["page"], a["split"], a["scale"],
                                      a["ws"], a["wsb"], a["out"], a["dt"], a["flags"], None)


def test_decode_validation(bi):
    assert attn(bi, d=64) == UNSUPPORTED
    assert attn(bi, page=32) == UNSUPPORTED
    assert attn(bi, flags=2) == UNSUPPORTED
    assert attn(bi, split=128) == UNSUPPORTED
    assert attn(bi, hq=16) == UNSUPPORTED
    assert attn(bi, batch=1 << 23, total=1 << 23) == UNSUPPORTED  # work items of a launch past 2^32
    assert attn(bi, dt=3) == DTYPE
    assert attn(bi, batch=-1) == SHAPE
    assert attn(bi, q=None) == NULL
    assert attn(bi, total=1) == SHAPE            # fewer splits than sequences
    assert attn(bi, total=10**6) == SHAPE        # more than max_pages allows
    assert attn(bi, wsb=100) == WORKSPACE
    assert attn(bi, ws=None) == WORKSPACE
    assert attn(bi, q=A2) == ALIGN
    assert attn(bi, batch=0, q=None, k=None) == OK


def test_decode_step_kernels_validation(bi):
    L = bi.lib
    # bi_add_rmsnorm(x, ldx, d, ldd, w, eps, y, ldy, y_dtype, m, n, stream)
    ar = lambda **k: L.bi_add_rmsnorm(k.get("x", A16), k.get("ldx", 64), k.get("d", A16), k.get("ldd", 64),  # noqa
                                      k.get("w", A16), 1e-6, k.get("y", A16), k.get("ldy", 64), k.get("dt", 0),
                                      k.get("m", 2), k.get("n", 64), None)
    assert ar(m=-1) == SHAPE and ar(dt=5) == DTYPE and ar(n=0) == SHAPE and ar(d=None) == NULL
    assert ar(ldd=32) == STRIDE and ar(ldd=68) == ALIGN and ar(d=A2) == ALIGN and ar(m=0, x=None) == OK
    # bi_embed(table, ld, vocab, tokens, out, ldo, m, n, stream)
    em = lambda **k: L.bi_embed(k.get("t", A16), k.get("ld", 64), k.get("v", 100), k.get("tok", A16),  # noqa
                                k.get("o", A16), k.get("ldo", 64), k.get("m", 3), k.get("n", 64), None)
    assert em(v=-1) == SHAPE and em(v=0) == SHAPE and em(tok=None) == NULL and em(ld=32) == STRIDE
    assert em(n=60, ld=64, ldo=64) == ALIGN and em(tok=A2 + 4 - 2) == ALIGN and em(m=0, t=None) == OK
    # bi_silu_mul(gu, ldg, out, ldo, m, n, stream)
    sm = lambda **k: L.bi_silu_mul(k.get("gu", A16), k.get("ldg", 128), k.get("o", A16), k.get("ldo", 64),  # noqa
                                   k.get("m", 2), k.get("n", 64), None)
    assert sm(m=-2) == SHAPE and sm(o=None) == NULL and sm(ldg=64) == STRIDE and sm(n=60, ldg=120, ldo=64) == ALIGN
    assert sm(m=70000) == UNSUPPORTED and sm(m=0, gu=None) == OK
    # bi_qknorm_rope_append(qkv, ldqkv, qw, kw, eps, cos, sin, max_pos, pos, bt, max_pages, num_pages,
    #                       kp, vp, q_out, batch, hq, hkv, head_dim, page_size, stream)
    def qr(**k):
        return L.bi_qknorm_rope_append(k.get("qkv", A16), k.get("ld", 6144), A16, A16, 1e-6, A16, A16,
                                       k.get("max_pos", 4096), A16, A16, k.get("max_pages", 8), k.get("pages", 64),
                                       A16, A16, k.get("q_out", A16), k.get("b", 2), k.get("hq", 32),
                                       k.get("hkv", 8), k.get("d", 128), k.get("page", 16), None)
    assert qr(b=-1) == SHAPE and qr(d=64) == UNSUPPORTED and qr(page=0) == UNSUPPORTED
    assert qr(q_out=None) == NULL and qr(ld=6000) == STRIDE and qr(pages=0) == SHAPE
    assert qr(qkv=A2 + 1) == ALIGN and qr(b=0, qkv=None) == OK


def test_prefill_plan_rows_offsets_and_work_cover_every_visible_split(bi):
    import numpy as np
    chunk = torch.tensor([3, 20, 0, 5, 17, 1], dtype=torch.int32)
    ctx = torch.tensor([0, 250, 7, 510, 0, 1000], dtype=torch.int32)
    q_pos, q_offs, work, (rows, total, n_work) = bi.bi_prefill_plan(chunk, ctx)
    assert rows == int(chunk.sum()) and q_offs.shape[0] == rows + 1 and int(q_offs[-1]) == total
    seq = np.repeat(np.arange(len(chunk)), chunk.numpy())
    want_pos = np.concatenate([np.arange(c, c + n) for c, n in zip(ctx.tolist(), chunk.tolist())])
    assert np.array_equal(q_pos.numpy(), want_pos)
    nsplit = (want_pos + 256) // 256
    assert np.array_equal(np.diff(q_offs.numpy()), nsplit)
    seen = {}
    for r0, nr, b, sp in work.tolist():
        assert 1 <= nr <= 128 and np.all(seq[r0:r0 + nr] == b)                      # one sequence per item
        assert np.array_equal(want_pos[r0:r0 + nr], np.arange(want_pos[r0], want_pos[r0] + nr))
        assert want_pos[r0 + nr - 1] >= 256 * sp                                   # its last row sees the split
        for r in range(r0, r0 + nr):
            if want_pos[r] >= 256 * sp:
                assert (r, sp) not in seen
                seen[(r, sp)] = True
    assert len(seen) == total  # every (row, visible split) exactly once
    # sizes-only call, and errors
    sizes = (ctypes.c_int64 * 3)()
    L = bi.lib
    cl, cb = chunk.contiguous(), ctx.contiguous()
    assert L.bi_prefill_plan(cl.data_ptr(), cb.data_ptr(), 6, 256, None, None, None, sizes) == OK
    assert tuple(sizes) == (rows, total, n_work)
    assert L.bi_prefill_plan(cl.data_ptr(), cb.data_ptr(), 6, 0, None, None, None, sizes) == SHAPE
    assert L.bi_prefill_plan(cl.data_ptr(), cb.data_ptr(), 6, 256, None, None, None, None) == NULL
    assert L.bi_prefill_plan(cl.data_ptr(), cb.data_ptr(), 6, 256, A16, None, None, sizes) == NULL
    bad = torch.tensor([-1], dtype=torch.int32)
    assert L.bi_prefill_plan(bad.data_ptr(), cb.data_ptr(), 1, 256, None, None, None, sizes) == SHAPE


def test_prefill_attention_validation(bi):
    def pa(**k):
        return bi.lib.bi_prefill_attention(A16, A16, A16, A16, k.get("max_pages", 4), A16, A16, A16,
                                           k.get("n_work", 3), k.get("rows", 10), k.get("total", 12), k.get("b", 2),
                                           k.get("hq", 32), k.get("hkv", 8), k.get("d", 128), 16, k.get("split", 256),
                                           0.088, k.get("ws", A16), k.get("wsb", 1 << 30), k.get("out", A16),
                                           k.get("dt", 1), None)
    assert pa(rows=-1) == SHAPE and pa(dt=3) == DTYPE and pa(d=64) == UNSUPPORTED and pa(split=128) == UNSUPPORTED
    assert pa(hq=16) == UNSUPPORTED and pa(out=None) == NULL and pa(n_work=0) == SHAPE
    assert pa(rows=1 << 22, total=1 << 22) == UNSUPPORTED  # the combine's work items past 2^32
    assert pa(total=5) == SHAPE and pa(wsb=100) == WORKSPACE and pa(ws=A2) == ALIGN and pa(rows=0, out=None) == OK


def test_decode_plan_and_workspace(bi):
    offs, total = bi.bi_decode_plan(torch.tensor([1, 255, 256, 257, 32768], dtype=torch.int32))
    assert offs.tolist() == [0, 1, 2, 3, 5, 133] and total == 133
    offs, total = bi.bi_decode_plan(torch.tensor([], dtype=torch.int32))
    assert offs.tolist() == [0] and total == 0
    with pytest.raises(bi.BiError):
        bi.bi_decode_plan(torch.tensor([3, 0], dtype=torch.int32))
    assert bi.lib.bi_decode_plan(None, 2, 256, None) == -1
    assert bi.lib.bi_decode_plan(None, 1, 0, None) == -1
    assert bi.bi_decode_workspace_bytes(133, 32, 128) == 133 * 32 * 130 * 4
    assert bi.bi_decode_workspace_bytes(-1, 32, 128) == 0


def test_plan_split_count_depends_on_length_only(bi):
    # the split offsets of a batch are the prefix sums of per-sequence counts,
    # each ceil(L/256) whatever the neighbours
    lens = torch.tensor([300, 7, 4096, 1, 257], dtype=torch.int32)
    offs, total = bi.bi_decode_plan(lens)
    counts = (offs[1:] - offs[:-1]).tolist()
    assert counts == [2, 1, 16, 1, 2] and total == 22
    offs2, _ = bi.bi_decode_plan(lens.flip(0))
    assert (offs2[1:] - offs2[:-1]).tolist() == counts[::-1]


def test_gemm_config_table(bi):
    """The configuration is a pure function of (m, n, k, layout) from a small
    set; every member computes each element with the same chain (the GPU
    tests compare rows across the Ms that select different members)."""
    seen = set()
    for n, k in [(512, 512), (6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288), (151936, 4096)]:
        for m in (1, 31, 32, 33, 64, 65, 256, 512, 2048, 4096):
            for nk in (False, True):
                cfg = bi.bi_gemm_config(m, n, k, nk)
                assert cfg == bi.bi_gemm_config(m, n, k, nk)
                assert cfg in {(32, 32, 64, 3), (64, 32, 64, 4), (32, 96, 64, 5), (64, 96, 64, 8), (64, 128, 64, 6),
                               (128, 128, 64, 10), (128, 128, 64, 4), (256, 256, 64, 8), (256, 384, 64, 8)}, cfg
                seen.add(cfg)
    assert len(seen) == 9
    # small batches of the projection shapes take the skinny tiles, M = 4096 a full-width one
    assert bi.bi_gemm_config(1, 4096, 4096)[1] == 32 and bi.bi_gemm_config(64, 4096, 12288)[1] == 32
    assert bi.bi_gemm_config(1, 24576, 4096) == (32, 96, 64, 5) and bi.bi_gemm_config(64, 24576, 4096) == (64, 96, 64, 8)
    assert bi.bi_gemm_config(4096, 4096, 4096)[1] == 256 and bi.bi_gemm_config(1, 151936, 4096)[1] == 128
    # 256x384 only where K and N are whole tiles and its tiles make whole rounds of 256
    assert bi.bi_gemm_config(4096, 24576, 4096)[1] == 384 and bi.bi_gemm_config(4096, 6144, 4096)[1] == 384
    assert bi.bi_gemm_config(1024, 24576, 4096)[1] == 384 and bi.bi_gemm_config(1280, 24576, 4096)[1] == 256
    assert bi.bi_gemm_config(4096, 6144, 4104)[1] != 384 and bi.bi_gemm_config(3840, 6144, 4096)[1] != 384
    # its loads carry no k mask, so never for k == 0 (where A and B may be NULL)
    assert bi.bi_gemm_config(4096, 24576, 0)[1] != 384
    with pytest.raises(bi.BiError):
        bi.bi_gemm_config(-1, 4, 4, False)
    assert bi.lib.bi_gemm_config(1, 4, 4, 0, None) == NULL


def test_binding_rejects_bad_python_args(bi):
    with pytest.raises(TypeError):
        bi.bi_mm(torch.zeros(2, 8), torch.zeros(8, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        bi.bi_mm(torch.zeros(2, 8, dtype=torch.bfloat16), torch.zeros(16, 8, dtype=torch.bfloat16))


def test_binding_refuses_host_tensors_before_any_launch(bi):
    """A host pointer handed to a kernel is a GPU memory fault: every wrapper
    checks that its tensors are GPU tensors (and shapes that size the kernels'
    reads and writes) before it launches, so these raise here, without a GPU.
    The decode plan's split offsets come back on the host; passing them
    unmoved is the case that matters most."""
    bf = torch.bfloat16
    a, w = torch.zeros(4, 64, dtype=bf), torch.zeros(64, 32, dtype=bf)
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_mm(a, w)
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_addmm(torch.zeros(32, dtype=bf), a, w)
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_rmsnorm(a, torch.ones(64, dtype=bf))
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_mean(a)
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_log_softmax(torch.zeros(2, 64))
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_add_rmsnorm(a.clone(), a, torch.ones(64, dtype=bf))
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_embed(torch.zeros(10, 64, dtype=bf), torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_silu_mul(torch.zeros(2, 64, dtype=bf))
    lens = torch.tensor([5, 300], dtype=torch.int32)
    offs, total = bi.bi_decode_plan(lens)
    assert offs.device.type == "cpu" and total == 3
    q = torch.zeros(2, 32, 128, dtype=bf)
    kp = torch.zeros(4, 8, 16, 128, dtype=bf)
    vp = torch.zeros(4, 8, 128, 16, dtype=bf)
    bt = torch.zeros(2, 32, dtype=torch.int32)
    with pytest.raises(ValueError, match="CUDA"):
        bi.bi_decode_attention(q, kp, vp, bt, lens, offs, total)
    # shapes that size the kernels' accesses are checked too
    with pytest.raises(ValueError, match="split_offsets"):
        bi.bi_decode_attention(q, kp, vp, bt, lens, offs[:2], total)
    with pytest.raises(ValueError, match="block_table"):
        bi.bi_decode_attention(q, kp, vp, bt[:1], lens, offs, total)


def test_gemm_plan_and_fixed_tile_mode(bi):
    """bi_gemm_plan reports the launches: the M-keyed table changes its tile
    with M and splits the LM head's columns at M = 256; the fixed-tile mode
    uses one configuration per (N, K, layout) for every M and never splits."""
    plan = bi.bi_gemm_plan(769, 151936, 4096)
    assert len(plan) == 2 and plan[0][:4] == (256, 256, 64, 8) and plan[1][:2] == (256, 128)
    assert plan[0][4] == 0 and plan[1][4] % 256 == 0 and 0 < plan[1][4] < 151936
    # the LM head at M = 256: 256x384 tiles in one whole round over the CUs, the rest on 256x256
    plan = bi.bi_gemm_plan(256, 151936, 4096)
    assert len(plan) == 2 and plan[0][:4] == (256, 384, 64, 8) and plan[1][:4] == (256, 256, 64, 8)
    assert plan[1][4] == 256 * 384
    # not with a sparse last row of tiles (256x256 skips rows past M, 256x384 multiplies them)
    assert len(bi.bi_gemm_plan(300, 151936, 4096)) == 1
    for n, k in ((6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288), (151936, 4096), (512, 512)):
        for nk in (False, True):
            table = {bi.bi_gemm_plan(m, n, k, nk)[0][:4] for m in range(1, 4097, 7)}
            fixed = {tuple(bi.bi_gemm_plan(m, n, k, nk, fixed_tile=True)) for m in range(1, 4097, 7)}
            assert len(fixed) == 1 and len(next(iter(fixed))) == 1, (n, k, fixed)
            assert len(table) >= 2, (n, k, table)
    assert bi.bi_gemm_plan(8, 512, 512, fixed_tile=True)[0][:4] == (128, 128, 64, 4)
    # the first entry of the plan is what bi_gemm_config reports
    for m in (1, 64, 65, 512, 4096):
        assert bi.bi_gemm_plan(m, 6144, 4096)[0][:4] == bi.bi_gemm_config(m, 6144, 4096)
    out, cnt = (ctypes.c_int32 * 10)(), ctypes.c_int32()
    assert bi.lib.bi_gemm_plan(4, 512, 512, 0, 2, out, ctypes.byref(cnt)) == UNSUPPORTED
    assert bi.lib.bi_gemm_plan(-1, 512, 512, 0, 0, out, ctypes.byref(cnt)) == SHAPE
    assert bi.lib.bi_gemm_plan(4, 512, 512, 0, 0, None, ctypes.byref(cnt)) == NULL
    # bi_gemm validates like bi_mm/bi_addmm, plus the flags
    g = lambda flags=0, bias=None, m=4: bi.lib.bi_gemm(bias, 0, 1.0, 1.0, A16, 512, A16, 512, 0, A16, 512, 1,  # noqa: E731
                                                       m, 512, 512, flags, None)
    assert g(flags=4) == UNSUPPORTED and g(flags=1, m=-1) == SHAPE and g(bias=0x10001) == ALIGN
    assert g(m=0) == OK and g(flags=1, m=0) == OK


def test_qwen_shapes_walk_every_gemm_configuration(bi):
    """Over M = 1..4096 the four Qwen3-8B projection shapes (either layout)
    take every configuration of the tile table between them, and the LM head
    over M = 1..256 the split into 256x384 and 256x256 launches: so the
    every-M GPU sweeps on those shapes run them all. (The 256x128 column
    split has its own GPU test, test_mm_column_split_same_bits.)"""
    table = {(32, 32, 64, 3), (64, 32, 64, 4), (32, 96, 64, 5), (64, 96, 64, 8), (64, 128, 64, 6), (128, 128, 64, 10),
             (128, 128, 64, 4), (256, 256, 64, 8), (256, 384, 64, 8)}
    seen, split = set(), False
    for k, n in ((4096, 6144), (4096, 4096), (4096, 24576), (12288, 4096)):
        for m in range(1, 4097):
            plan = bi.bi_gemm_plan(m, n, k)
            seen |= {p[:4] for p in plan[:1]}
    for m in range(1, 257):
        plan = bi.bi_gemm_plan(m, 151936, 4096)
        split |= len(plan) == 2 and plan[0][:2] == (256, 384) and plan[1][:2] == (256, 256)
    assert seen == table and split, (seen, split)
