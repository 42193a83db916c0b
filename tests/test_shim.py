"""The torch op-override mode: routing decisions (CPU) and routed results (GPU).

GPU cases check that, inside ``batch_invariant_mode``, torch's own mm /
addmm / linear / log_softmax / mean / rms_norm calls return exactly the
bytes the C-ABI kernels return for the same operands and meet the fp64
oracle's tolerances, that a small bf16 model run through unchanged torch
code matches the oracle's composition of the same ops, and that it gives
each row the same bytes at every batch size.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
import synthetic as S
from helpers import ELEM_TOL, assert_close, bits, f32, same_bits

DEV = "cuda"


# ---------------------------------------------------------------- CPU: routing logic
def close_bf16(got, ref, what):
    """A bf16 result is one rounding of its exact value: rel-Frobenius
    <= 2^-8 and the elementwise bound against the unrounded oracle."""
    g = f32(got.float()).astype(np.float64).reshape(ref.shape)
    fro, el = O.relative_frobenius(g, ref), O.elementwise_ratio(g, ref)
    assert fro <= 2.0 ** -8 and el <= ELEM_TOL, f"{what}: rel-Frobenius {fro:.3e}, elementwise {el:.3e}"


def test_gemm_operands_layouts():
    from invariant_bi_mm_amd.shim import gemm_operands
    a = torch.zeros(4, 64, dtype=torch.bfloat16)
    w_kn = torch.zeros(64, 32, dtype=torch.bfloat16)
    w_nk = torch.zeros(32, 64, dtype=torch.bfloat16)
    a2, b2, nk = gemm_operands(a, w_kn)
    assert nk is False and b2 is w_kn
    a2, b2, nk = gemm_operands(a, w_nk.t())  # nn.Linear: x @ W.t()
    assert nk is True and b2.data_ptr() == w_nk.data_ptr() and b2.shape == (32, 64)
    assert isinstance(gemm_operands(a.float(), w_kn.float()), str)  # dtype
    assert isinstance(gemm_operands(torch.zeros(4, 12, dtype=torch.bfloat16),
                                    torch.zeros(12, 32, dtype=torch.bfloat16)), str)  # K % 8
    assert isinstance(gemm_operands(a, torch.zeros(64, 64, dtype=torch.bfloat16)[:, ::2]), str)  # strided b
    assert isinstance(gemm_operands(a.t().contiguous().t(), w_kn), str)  # a column-major


def test_mode_leaves_cpu_tensors_to_torch():
    from invariant_bi_mm_amd.shim import batch_invariant_mode
    g = torch.Generator().manual_seed(0)
    x = torch.randn(3, 16, generator=g).to(torch.bfloat16)
    w = torch.randn(8, 16, generator=g).to(torch.bfloat16)
    ref = (F.linear(x, w), F.log_softmax(x.float(), -1), x.mean(-1),
           F.rms_norm(x, (16,), weight=torch.ones(16, dtype=torch.bfloat16), eps=1e-6))
    with batch_invariant_mode() as mode:
        got = (F.linear(x, w), F.log_softmax(x.float(), -1), x.mean(-1),
               F.rms_norm(x, (16,), weight=torch.ones(16, dtype=torch.bfloat16), eps=1e-6))
    assert not mode.routed and not mode.passthrough
    for r, o in zip(ref, got):
        assert torch.equal(r, o)
    assert F.rms_norm is not mode._rms_norm  # restored on exit


# ---------------------------------------------------------------- GPU: routed results
@pytest.mark.gpu
def test_mm_linear_route_to_kernels(lib):
    from invariant_bi_mm_amd.shim import batch_invariant_mode
    x = S.normal_bf16((2, 37, 512), 1.0, seed=11, device=DEV)
    w = S.normal_bf16((768, 512), 1.0 / 512, seed=12, device=DEV)  # nn.Linear weight [N, K]
    b = S.normal_bf16((768,), 0.1, seed=13, device=DEV)
    w_kn = S.normal_bf16((512, 256), 1.0 / 512, seed=14, device=DEV)
    with batch_invariant_mode() as mode:
        y_lin = F.linear(x, w)
        y_lin_b = F.linear(x[0], w, b)
        y_mm = x[1] @ w_kn
        y_mm32 = torch.mm(x[1], w_kn, out_dtype=torch.float32) if hasattr(torch.ops.aten.mm, "dtype") else None
    assert mode.routed["mm"] >= 2 and mode.routed["addmm"] == 1
    assert y_lin.dtype == torch.bfloat16 and y_lin.shape == (2, 37, 768)
    assert same_bits(y_lin.reshape(-1, 768), lib.bi_mm(x.reshape(-1, 512), w, b_is_nk=True, out_dtype=torch.bfloat16))
    assert same_bits(y_lin_b, lib.bi_addmm(b, x[0], w, b_is_nk=True, out_dtype=torch.bfloat16))
    assert same_bits(y_mm, lib.bi_mm(x[1], w_kn, out_dtype=torch.bfloat16))
    if y_mm32 is not None:
        assert same_bits(y_mm32, lib.bi_mm(x[1], w_kn))
        assert_close(f32(y_mm32), O.mm(bits(x[1]), bits(w_kn)), "routed mm fp32 vs oracle")
    # the routed results against the fp64 oracle
    close_bf16(y_lin.reshape(-1, 768), O.mm(bits(x.reshape(-1, 512)), bits(w), b_is_nk=True), "routed linear")
    close_bf16(y_lin_b, O.addmm(bits(b), bits(x[0]), bits(w), b_is_nk=True), "routed linear + bias")
    close_bf16(y_mm, O.mm(bits(x[1]), bits(w_kn)), "routed x @ w")


@pytest.mark.gpu
def test_reductions_route_to_kernels(lib):
    from invariant_bi_mm_amd.shim import batch_invariant_mode
    logits = S.normal_f32((5, 2048), 4.0, seed=21, device=DEV)
    h = S.normal_bf16((3, 7, 4096), 1.0, seed=22, device=DEV)
    w = S.uniform_bf16((4096,), 0.5, 1.5, seed=23, device=DEV)
    with batch_invariant_mode() as mode:
        ls = F.log_softmax(logits, dim=-1)
        mu = h.mean(dim=-1)
        mu_k = h.float().mean(dim=-1, keepdim=True)
        rn = F.rms_norm(h, (4096,), weight=w, eps=1e-6)
    assert dict(mode.routed) == {"log_softmax": 1, "mean": 2, "rms_norm": 1}
    assert same_bits(ls, lib.bi_log_softmax(logits, want_argmax=False)[0])
    assert mu.dtype == torch.bfloat16 and mu.shape == (3, 7)
    assert same_bits(mu.reshape(-1), lib.bi_mean(h.reshape(-1, 4096)).to(torch.bfloat16))
    assert mu_k.shape == (3, 7, 1) and same_bits(mu_k.reshape(-1), lib.bi_mean(h.float().reshape(-1, 4096)))
    assert same_bits(rn.reshape(-1, 4096), lib.bi_rmsnorm(h.reshape(-1, 4096), w, 1e-6))
    # the routed results against the fp64 oracle
    assert_close(f32(ls), O.log_softmax(f32(logits)), "routed log_softmax")
    hb = bits(h.reshape(-1, 4096))
    close_bf16(mu.reshape(-1), O.mean(hb), "routed mean (bf16)")
    assert_close(f32(mu_k.reshape(-1)), O.mean(f32(h.float().reshape(-1, 4096))), "routed mean (fp32)")
    close_bf16(rn.reshape(-1, 4096), O.rmsnorm(hb, bits(w), 1e-6), "routed rms_norm")


@pytest.mark.gpu
def test_strict_refuses_and_lenient_passes_through(lib):
    from invariant_bi_mm_amd.shim import BiUnsupported, batch_invariant_mode
    a = S.normal_f32((4, 64), 1.0, seed=31, device=DEV)
    b = S.normal_f32((64, 32), 1.0, seed=32, device=DEV)
    with batch_invariant_mode():
        with pytest.raises(BiUnsupported):
            torch.mm(a, b)  # fp32 GEMM: not a covered dtype
        with pytest.raises(BiUnsupported):
            a.mean(dim=0)  # not the last dim
    with batch_invariant_mode(strict=False) as mode:
        c = torch.mm(a, b)
    torch.testing.assert_close(c, a @ b)
    assert mode.passthrough["mm"] == 1 and not mode.routed


class TinyLM(torch.nn.Module):
    """RMSNorm -> linear -> SiLU -> linear (+residual) -> RMSNorm -> LM head -> log_softmax, bf16."""

    def __init__(self, d=512, f=1536, v=4096, seed=40):
        super().__init__()
        g = lambda shape, var, s: torch.nn.Parameter(S.normal_bf16(shape, var, seed=seed + s, device=DEV),  # noqa: E731
                                                     requires_grad=False)
        self.w_up, self.w_down, self.w_head = g((f, d), 1 / d, 1), g((d, f), 1 / f, 2), g((v, d), 1 / d, 3)
        self.b_head = g((v,), 0.01, 4)
        self.n1 = torch.nn.Parameter(S.uniform_bf16((d,), 0.5, 1.5, seed=seed + 5, device=DEV), requires_grad=False)
        self.n2 = torch.nn.Parameter(S.uniform_bf16((d,), 0.5, 1.5, seed=seed + 6, device=DEV), requires_grad=False)

    def forward(self, x, keep=None):
        """keep: optional dict that receives each stored bf16 activation."""
        keep = {} if keep is None else keep
        keep["h1"] = h = F.rms_norm(x, (x.shape[-1],), weight=self.n1, eps=1e-6)
        keep["up"] = u = F.linear(h, self.w_up)
        keep["silu"] = a = F.silu(u)
        keep["down"] = d = F.linear(a, self.w_down)
        keep["res"] = r = x + d
        keep["h2"] = h = F.rms_norm(r, (r.shape[-1],), weight=self.n2, eps=1e-6)
        keep["logits"] = z = F.linear(h, self.w_head, self.b_head)
        return F.log_softmax(z.float(), dim=-1)


def oracle_tinylm(model, x_bits, tie):
    """TinyLM's forward composed from the oracle's ops in fp64, each bf16
    activation rounded where the model stores it. tie: the model's stored
    bf16 values, used only at near-ties (the near-tie rule of
    oracle.decode_step.round_at). Returns (values before rounding, fp64
    log-probabilities)."""
    from oracle.decode_step import round_at
    p = {k: bits(v.detach()) for k, v in model.named_parameters()}
    vals = {}

    def keep(name, u):
        vals[name] = u
        return O.bf16_bits_of(round_at(u, tie[name])[0])

    h = keep("h1", O.rmsnorm(x_bits, p["n1"], 1e-6))
    u = keep("up", O.mm(h, p["w_up"], b_is_nk=True))
    # silu alone: the gated form with an up part of ones
    a = keep("silu", O.silu_mul(np.concatenate([u, np.full_like(u, 0x3F80)], axis=1)))
    d = keep("down", O.mm(a, p["w_down"], b_is_nk=True))
    r = keep("res", O.bf16_bits_to_f64(x_bits) + O.bf16_bits_to_f64(d))
    h2 = keep("h2", O.rmsnorm(r, p["n2"], 1e-6))
    z = keep("logits", O.addmm(p["b_head"], h2, p["w_head"], b_is_nk=True))
    return vals, O.log_softmax(O.bf16_bits_to_f64(z).astype(np.float32))


@pytest.mark.gpu
def test_unchanged_model_code_matches_oracle(lib):
    """The TinyLM's routed forward against the oracle's composition of the
    same ops: every stored bf16 activation at the bf16 tolerance and the fp32
    log-probabilities at 1e-3 / 4e-3."""
    from invariant_bi_mm_amd.shim import batch_invariant_mode
    model = TinyLM()
    x = S.normal_bf16((64, 512), 1.0, seed=70, device=DEV)
    acts = {}
    with batch_invariant_mode():
        logp = model(x, keep=acts)
    tie = {k: bits(v) for k, v in acts.items()}
    vals, ref = oracle_tinylm(model, bits(x), tie)
    for name, u in vals.items():
        close_bf16(acts[name], u, f"TinyLM {name}")
    assert_close(f32(logp), ref, "TinyLM log-probabilities")


@pytest.mark.gpu
def test_unchanged_model_code_is_batch_invariant(lib):
    from invariant_bi_mm_amd.shim import batch_invariant_mode
    model = TinyLM()
    row = S.normal_bf16((1, 512), 1.0, seed=50, device=DEV)
    with batch_invariant_mode() as mode:
        alone = model(row)[0].clone()
        for m in (2, 7, 64, 129, 300):
            x = S.normal_bf16((m, 512), 1.0, seed=60 + m, device=DEV)
            for pos in (0, m // 2, m - 1):
                x[pos] = row[0]
                got = model(x)[pos]
                assert same_bits(got, alone), f"row changed at M={m}, position {pos}"
    assert mode.routed["mm"] > 0 and mode.routed["addmm"] > 0 and mode.routed["rms_norm"] > 0
    assert mode.routed["log_softmax"] > 0 and not mode.passthrough
