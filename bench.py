#!/usr/bin/env python3
"""Benchmark of the batch-invariant hot path on one MI355X.

One step runs every kernel of the path once, on synthetic Qwen3-8B-shaped
inputs already resident in HBM:
  gemm_qkv     bi_mm  A[4096,4096] @ W[4096,6144]     -> fp32
  gemm_o       bi_mm  A[4096,4096] @ W[4096,4096]     -> fp32
  gemm_gateup  bi_mm  A[4096,4096] @ W[4096,24576]    -> fp32
  gemm_down    bi_mm  A[4096,12288] @ W[12288,4096]   -> fp32
  lm_head      bi_addmm X[256,4096] @ W[4096,151936] + bias -> fp32 logits
  lm_logsm     bi_log_softmax + argmax over those logits [256,151936]
  rmsnorm      bi_rmsnorm x[2048,4096] bf16 -> bf16
  mean         bi_mean x[2048,4096] bf16 -> fp32
  logsm        bi_log_softmax + argmax x[2048,151936] fp32
  decode_attn  bi_decode_attention, B=256, lengths log-uniform in [1,32768]
Each kernel has a roofline time t_min = max(flops / 2.5 PFLOP/s, bytes /
8 TB/s) from its algorithmic flops and bytes. ``value`` is the whole step's
roofline fraction: sum of t_min over the step / measured step time, in %.

Reported beside it (not part of ``value``): ``e2e_decode_step``, greedy
decode steps of a Qwen3-8B-shaped model (36 layers, random weights, 64
sequences with lengths log-uniform in [1, 32768]) chained through the
library, with its own HBM bound; and ``prefill_attention``, causal prefill of
4 prompts of 2048 tokens with the decode split structure, against its
matrix-core plus vector-ALU bound.

Prints ONE JSON line on stdout; a human-readable table goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15   # MI355X dense bf16 MFMA, FLOP/s (published)
PEAK_HBM = 8.0e12    # MI355X HBM3E, B/s (published)
METRIC = "invariant bf16 GEMM TFLOP/s & reduction GB/s (% roofline), M=1..4096, 1 GPU"

GEMMS = [("gemm_qkv", 4096, 6144), ("gemm_o", 4096, 4096), ("gemm_gateup", 4096, 24576), ("gemm_down", 12288, 4096)]
M_GEMM = 4096
M_LM = 256
M_ROWS = 2048
HIDDEN = 4096
VOCAB = 151936
B_DECODE = 256


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_work(m, n, k, out_bytes=4, bias=False):
    flops = 2.0 * m * n * k
    byts = 2.0 * (m * k + k * n) + out_bytes * m * n + (2.0 * n if bias else 0.0)
    return flops, byts


def t_min(flops, byts):
    return max(flops / PEAK_BF16, byts / PEAK_HBM)


class Workload:
    """All inputs and outputs of one step, generated on the GPU from seeds."""

    def __init__(self, torch, S, bi, dev):
        self.torch, self.bi = torch, bi
        t0 = time.time()
        self.gemm = []
        for i, (name, k, n) in enumerate(GEMMS):
            a = S.normal_bf16((M_GEMM, k), 1.0, seed=3000 + i, device=dev)
            w = S.normal_bf16((k, n), 0.02, seed=3100 + i, device=dev)
            c = torch.empty((M_GEMM, n), dtype=torch.float32, device=dev)
            self.gemm.append((name, a, w, c, k, n))
        self.lm_x = S.normal_bf16((M_LM, HIDDEN), 1.0, seed=4000, device=dev)
        self.lm_w = S.normal_bf16((HIDDEN, VOCAB), 0.02, seed=4001, device=dev)
        self.lm_b = S.normal_bf16((VOCAB,), 0.1, seed=4002, device=dev)
        self.lm_logits = torch.empty((M_LM, VOCAB), dtype=torch.float32, device=dev)
        self.lm_lp = torch.empty_like(self.lm_logits)
        self.lm_am = torch.empty((M_LM,), dtype=torch.int64, device=dev)
        self.rx = S.normal_bf16((M_ROWS, HIDDEN), 1.0, seed=1000, device=dev)
        self.rw = S.uniform_bf16((HIDDEN,), 0.5, 1.5, seed=1001, device=dev)
        self.ry = torch.empty_like(self.rx)
        self.rmean = torch.empty((M_ROWS,), dtype=torch.float32, device=dev)
        self.lx = S.normal_f32((M_ROWS, VOCAB), 4.0, seed=1002, device=dev)
        self.ly = torch.empty_like(self.lx)
        self.lam = torch.empty((M_ROWS,), dtype=torch.int64, device=dev)
        self.lens = S.context_lens(B_DECODE, seed=5000)
        table, npages = S.paged_kv_layout(self.lens, 16, seed=5001)
        self.q = S.normal_bf16((B_DECODE, 32, 128), 1.0, seed=5002, device=dev)
        self.kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=5003, device=dev)
        self.vp = S.normal_bf16((npages, 8, 128, 16), 1.0, seed=5004, device=dev)  # d-major V
        self.table = table.to(dev)
        self.table_host = table
        self.lens_dev = self.lens.to(dev)
        offs, self.total_splits = bi.bi_decode_plan(self.lens)
        self.offs = offs.to(dev)
        self.ws = torch.empty(bi.bi_decode_workspace_bytes(self.total_splits, 32, 128), dtype=torch.uint8, device=dev)
        self.attn_out = torch.empty((B_DECODE, 32, 128), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        log(f"inputs generated in {time.time() - t0:.1f}s; decode tokens={int(self.lens.sum())} "
            f"splits={self.total_splits}")

    def ops(self):
        """(name, callable, flops, bytes) for every kernel launch group of a step."""
        bi = self.bi
        out = []
        for name, a, w, c, k, n in self.gemm:
            f, b = gemm_work(M_GEMM, n, k)
            out.append((name, (lambda a=a, w=w, c=c: bi.bi_mm(a, w, out=c)), f, b))
        f, b = gemm_work(M_LM, VOCAB, HIDDEN, bias=True)
        out.append(("lm_head", lambda: bi.bi_addmm(self.lm_b, self.lm_x, self.lm_w, out=self.lm_logits), f, b))
        out.append(("lm_logsm", lambda: bi.bi_log_softmax(self.lm_logits, out=self.lm_lp, argmax=self.lm_am),
                    5.0 * M_LM * VOCAB, 8.0 * M_LM * VOCAB + 8 * M_LM))
        out.append(("rmsnorm", lambda: bi.bi_rmsnorm(self.rx, self.rw, 1e-6, out=self.ry),
                    4.0 * M_ROWS * HIDDEN, 4.0 * M_ROWS * HIDDEN + 2 * HIDDEN))
        out.append(("mean", lambda: bi.bi_mean(self.rx, out=self.rmean),
                    1.0 * M_ROWS * HIDDEN, 2.0 * M_ROWS * HIDDEN + 4 * M_ROWS))
        out.append(("logsm", lambda: bi.bi_log_softmax(self.lx, out=self.ly, argmax=self.lam),
                    5.0 * M_ROWS * VOCAB, 8.0 * M_ROWS * VOCAB + 8 * M_ROWS))
        tokens = int(self.lens.sum())
        pages = int(((self.lens + 15) // 16).sum())
        attn_bytes = 4096.0 * tokens + B_DECODE * 32 * 128 * (2 + 4) + 4.0 * pages
        attn_flops = 4.0 * 32 * 128 * tokens
        out.append(("decode_attn", lambda: bi.bi_decode_attention(
            self.q, self.kp, self.vp, self.table, self.lens_dev, self.offs, self.total_splits,
            workspace=self.ws, out=self.attn_out), attn_flops, attn_bytes))
        return out

    def torch_ops(self):
        """The same work through torch's own (non-invariant) kernels."""
        torch = self.torch
        F = torch.nn.functional
        out = []
        for name, a, w, c, k, n in self.gemm:
            out.append((name, (lambda a=a, w=w: torch.mm(a, w, out_dtype=torch.float32))))
        out.append(("lm_head", lambda: torch.addmm(self.lm_b, self.lm_x, self.lm_w, out_dtype=torch.float32)))
        out.append(("lm_logsm", lambda: (torch.log_softmax(self.lm_logits, -1), torch.argmax(self.lm_logits, -1))))
        out.append(("rmsnorm", lambda: F.rms_norm(self.rx, (HIDDEN,), self.rw, 1e-6)))
        out.append(("mean", lambda: torch.mean(self.rx, dim=1, dtype=torch.float32)))
        out.append(("logsm", lambda: (torch.log_softmax(self.lx, -1), torch.argmax(self.lx, -1))))
        return out


# The HIP source that defines each step's kernel (with the shared headers,
# the input of a per-kernel digest: measured traffic stays valid until that
# kernel's own source changes).
_GEMM_SRC = ("gemm.hip", "gemm_plan.cpp")
KERNEL_SOURCE = {"gemm_qkv": _GEMM_SRC, "gemm_o": _GEMM_SRC, "gemm_gateup": _GEMM_SRC, "gemm_down": _GEMM_SRC,
                 "lm_head": _GEMM_SRC, "lm_logsm": ("rowreduce.hip",), "rmsnorm": ("rowreduce.hip",),
                 "mean": ("rowreduce.hip",), "logsm": ("rowreduce.hip",), "decode_attn": ("decode_attention.hip",)}


def source_digest(kernel: str) -> str:
    """sha256 over the sources defining `kernel` (its HIP file and, for the
    GEMM, the tile table) and the shared headers."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "invariant_bi_mm_amd", "csrc")
    for name in (*KERNEL_SOURCE[kernel], "bi_internal.h", "device_common.h"):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


COUNTER_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- python3 bench.py --steps 2 --warmup 1 "
    "--no-cpu --no-torch --no-e2e",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- python3 bench.py --steps 2 --warmup 1 "
    "--no-cpu --no-torch --no-e2e",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/cal_fetch -o run -- python3 bench.py --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/cal_write -o run -- python3 bench.py --copy-calibration",
    "python3 bench.py --summarize-counters <dir>",
]
COPY_BYTES = 256 << 20  # the --copy-calibration copy


def step_algorithmic_bytes(S):
    """Algorithmic bytes per launch group of a step (the Workload's figures,
    without a GPU: the decode lengths come from the same seeded draw)."""
    out = {name: gemm_work(M_GEMM, n, k)[1] for name, k, n in GEMMS}
    out["lm_head"] = gemm_work(M_LM, VOCAB, HIDDEN, bias=True)[1]
    out["lm_logsm"] = 8.0 * M_LM * VOCAB + 8 * M_LM
    out["rmsnorm"] = 4.0 * M_ROWS * HIDDEN + 2 * HIDDEN
    out["mean"] = 2.0 * M_ROWS * HIDDEN + 4 * M_ROWS
    out["logsm"] = 8.0 * M_ROWS * VOCAB + 8 * M_ROWS
    lens = S.context_lens(B_DECODE, seed=5000)
    out["decode_attn"] = (4096.0 * float(lens.sum()) + B_DECODE * 32 * 128 * (2 + 4)
                          + 4.0 * float(((lens + 15) // 16).sum()))
    return out


def summarize_counters(root: str, out_json: str) -> None:
    """HBM traffic per launch group from the rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs under `root` (subfolders fetch, write, cal_fetch,
    cal_write, as in COUNTER_COMMANDS): every complete step the runs
    dispatched (the step's kernels in their order, found by name) is averaged
    per op, scaled by what the same counter reads for a plain copy of
    COPY_BYTES, and written to `out_json` with each op's source digest; the
    markdown table goes to stdout."""
    import csv
    import glob
    import statistics
    import invariant_bi_mm_amd as bi
    import synthetic as S

    def rows(sub):
        files = glob.glob(os.path.join(root, sub, "**", "*counter_collection.csv"), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {os.path.join(root, sub)}, found {files}")
        with open(files[0], newline="") as fh:
            got = [(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(fh)]
        return sorted(got)

    def kib_of_copy(sub):
        vals = [v for _, name, v in rows(sub) if "copyBuffer" in name]
        if not vals:
            raise SystemExit(f"no copy kernel in {sub}")
        return statistics.median(vals)

    cal = {"copy_kernel": "__amd_rocclr_copyBuffer", "copy_bytes": COPY_BYTES,
           "copy_FETCH_SIZE_KiB": kib_of_copy("cal_fetch"), "copy_WRITE_SIZE_KiB": kib_of_copy("cal_write")}
    cal["fetch_scale"] = COPY_BYTES / (cal["copy_FETCH_SIZE_KiB"] * 1024.0)
    cal["write_scale"] = COPY_BYTES / (cal["copy_WRITE_SIZE_KiB"] * 1024.0)

    # the step's dispatches in order: (op, kernel name fragment)
    seq = []
    for name, k, n in GEMMS:
        seq += [(name, f"gemm_kernel<{p[0]}, {p[1]},") for p in bi.bi_gemm_plan(M_GEMM, n, k)]
    seq += [("lm_head", f"gemm_kernel<{p[0]}, {p[1]},") for p in bi.bi_gemm_plan(M_LM, VOCAB, HIDDEN)]
    seq += [("lm_logsm", "log_softmax_kernel"), ("rmsnorm", "rmsnorm_kernel"), ("mean", "mean_kernel"),
            ("logsm", "log_softmax_kernel"), ("decode_attn", "decode_split_kernel"),
            ("decode_attn", "decode_combine_kernel")]

    def per_op(sub):
        ours = [(name, v) for _, name, v in rows(sub) if "bi::" in name]
        sums, steps, i = {}, 0, 0
        while i + len(seq) <= len(ours):
            if all(frag in ours[i + j][0] for j, (_, frag) in enumerate(seq)):
                for j, (op, _) in enumerate(seq):
                    sums[op] = sums.get(op, 0.0) + ours[i + j][1]
                steps += 1
                i += len(seq)
            else:
                i += 1
        if steps == 0:
            raise SystemExit(f"no complete step found in {sub}")
        return {op: v / steps for op, v in sums.items()}, steps

    fetch, nf = per_op("fetch")
    write, nw = per_op("write")
    alg = step_algorithmic_bytes(S)
    kernels = {}
    print("| op | kernels | fetch MB | write MB | total MB | algorithmic MB | ratio |")
    print("|---|---|---|---|---|---|---|")
    for op in dict.fromkeys(o for o, _ in seq):
        fb = fetch[op] * 1024.0 * cal["fetch_scale"]
        wb = write[op] * 1024.0 * cal["write_scale"]
        frags = list(dict.fromkeys(f for o, f in seq if o == op))
        kernels[op] = {"hbm_fetch_bytes_per_launch": int(round(fb)), "hbm_write_bytes_per_launch": int(round(wb)),
                       "kernels": frags, "hbm_bytes_per_launch": int(round(fb + wb)),
                       "source_sha256": source_digest(op), "source": list(KERNEL_SOURCE[op])}
        print(f"| {op} | {', '.join('`' + f + '`' for f in frags)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
              f"{(fb + wb) / 1e6:.1f} | {alg[op] / 1e6:.1f} | {(fb + wb) / alg[op]:.2f} |")
    with open(out_json, "w") as fh:
        json.dump({"commands": COUNTER_COMMANDS, "calibration": cal, "steps_averaged": {"fetch": nf, "write": nw},
                   "kernels": kernels}, fh, indent=1)
        fh.write("\n")
    log(f"wrote {out_json}: {nf} / {nw} steps averaged; fetch scale {cal['fetch_scale']:.4f}, "
        f"write scale {cal['write_scale']:.4f}")


def time_step(torch, ops, steps, warmup):
    """Run `warmup` untimed steps, then `steps` timed steps bracketed by
    synchronize; every launch group is also bracketed by HIP events on the
    stream the kernels run on. Returns (ms per step, {name: avg ms})."""
    for _ in range(warmup):
        for _, fn, *_ in ops:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for (name, fn, *_), (e0, e1) in zip(ops, evs[s]):
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    per, dist = {}, {}
    for i, (name, *_) in enumerate(ops):
        xs = sorted(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(steps))
        per[name] = sum(xs) / steps
        dist[name] = {"median": round(xs[len(xs) // 2], 4), "min": round(xs[0], 4),
                      "p90": round(xs[min(len(xs) - 1, int(0.9 * len(xs)))], 4)}
    time_step.last_dist = dist
    return wall, per


def time_step_graph(torch, ops, steps, warmup, check=()):
    """The same step captured once as a HIP graph and replayed: `warmup`
    untimed replays, then `steps` timed ones bracketed by synchronize.
    `check` lists output tensors whose contents after a replay must equal
    those of an eager step (the replay runs the same kernels on the same
    buffers). Returns ms per step."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, fn, *_ in ops:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in check]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _, fn, *_ in ops:
            fn()
    for t in check:
        t.zero_()
    g.replay()
    torch.cuda.synchronize()
    for t, e in zip(check, eager):
        if not torch.equal(t.view(torch.uint8), e.view(torch.uint8)):
            raise RuntimeError("graph replay of the step differs from the eager step")
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    for t, e in zip(check, eager):  # and still equal after the timed replays
        if not torch.equal(t.view(torch.uint8), e.view(torch.uint8)):
            raise RuntimeError("graph replay of the step differs from the eager step")
    return e0.elapsed_time(e1) / steps


def negative_control(torch, S, dev):
    """The invariance harness on torch's own kernels: a fixed row at
    position 0 inside batches of M random rows, compared bit for bit with
    the same row alone; counts the Ms at which the row changed. Reported,
    not asserted: it shows the check can see a batch-dependent kernel."""
    k, n = 4096, 4096
    w = S.normal_bf16((k, n), 0.02, seed=7, device=dev)
    row = S.normal_bf16((1, k), 1.0, seed=11, device=dev)[0]
    ref = torch.mm(row[None], w, out_dtype=torch.float32)[0].clone()
    ms = (2, 8, 64, 512, 4096)
    mm_changed = []
    for m in ms:
        x = S.normal_bf16((m, k), 1.0, seed=m, device=dev)
        x[0] = row
        if not torch.equal(torch.mm(x, w, out_dtype=torch.float32)[0].view(torch.int32), ref.view(torch.int32)):
            mm_changed.append(m)
    lg = S.normal_f32((1, VOCAB), 4.0, seed=3, device=dev)
    ref_l = torch.log_softmax(lg, dim=-1)[0].clone()
    ls_ms = (2, 64, 513)
    ls_changed = []
    for m in ls_ms:
        x = S.normal_f32((m, VOCAB), 4.0, seed=m, device=dev)
        x[0] = lg[0]
        if not torch.equal(torch.log_softmax(x, dim=-1)[0].view(torch.int32), ref_l.view(torch.int32)):
            ls_changed.append(m)
    return {"torch_mm_K4096_N4096": {"M_tried": list(ms), "row_changed_at_M": mm_changed},
            "torch_log_softmax_N151936": {"M_tried": list(ls_ms), "row_changed_at_M": ls_changed}}


def gpu_clocks():
    """Shader and memory clocks as rocm-smi reports them (None where it is not available)."""
    import shutil
    import subprocess
    smi = shutil.which("rocm-smi")
    if smi is None:
        return None
    try:
        # rocm-smi is a Python script: run it with this interpreter rather than through its
        # "#!/usr/bin/env python3" line, so no process replaces itself with another
        r = subprocess.run([sys.executable, os.path.realpath(smi), "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        d = json.loads(r.stdout)
    except Exception:
        return None
    out = {}
    for card, v in d.items():
        if isinstance(v, dict):
            out[card] = {k: v[k] for k in v if "sclk" in k.lower() or "mclk" in k.lower()}
    return out or None


def cpu_baseline(wl, S):
    """The fp64 oracle on a bounded sample of the same step, extrapolated by
    the work ratio of each kernel."""
    import numpy as np
    import oracle as O
    ncores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(ncores)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    bits = S.bf16_bits_numpy
    total = 0.0
    parts = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # GEMMs: 128 rows x 2048 columns of each projection, scaled by flops
    for name, a, w, c, k, n in wl.gemm:
        ab, wb = bits(a[:128]), bits(w[:, :2048])
        t = timed(lambda: O.mm(ab, wb)) * (M_GEMM * n) / (128 * 2048)
        parts[name] = t
    xb, wb, bb = bits(wl.lm_x[:32]), bits(wl.lm_w[:, :4096]), bits(wl.lm_b[:4096])
    parts["lm_head"] = timed(lambda: O.addmm(bb, xb, wb)) * (M_LM * VOCAB) / (32 * 4096)
    lg = S.f32_numpy(wl.lm_logits[:16])
    parts["lm_logsm"] = timed(lambda: (O.log_softmax(lg), O.argmax(lg))) * M_LM / 16
    rx, rw = bits(wl.rx[:256]), bits(wl.rw)
    parts["rmsnorm"] = timed(lambda: O.rmsnorm(rx, rw, 1e-6)) * M_ROWS / 256
    parts["mean"] = timed(lambda: O.mean(rx)) * M_ROWS / 256
    lx = S.f32_numpy(wl.lx[:32])
    parts["logsm"] = timed(lambda: (O.log_softmax(lx), O.argmax(lx))) * M_ROWS / 32
    # decode attention: 3 sequences (their pages only), scaled by tokens
    lens = wl.lens.numpy()
    seqs = [int(np.argsort(lens)[len(lens) // 2]), 0, 1]
    kp = bits(wl.kp)
    vp = bits(wl.vp)
    q = bits(wl.q)
    tb = wl.table_host.numpy()
    ta = timed(lambda: O.decode_attention(q, kp, vp, tb, lens, 128 ** -0.5, seqs=seqs))
    parts["decode_attn"] = ta * float(lens.sum()) / float(lens[seqs].sum())
    total = sum(parts.values())
    sample = ("oracle (numpy fp64) on: 128 rows x 2048 cols per projection GEMM, 32 rows x 4096 cols of the "
              "LM head, 16 rows of LM-head log_softmax, 256 rows of RMSNorm/mean, 32 rows of the 2048-row "
              "log_softmax, 3 decode sequences; each extrapolated to the full step by its work ratio")
    cpu_baseline.cores = {"os_cpu_count": os.cpu_count(), "affinity_cores": ncores, "blas_threads": threads}
    return total, parts, threads, sample


def sweep(torch, S, bi):
    """Per-config sweep (the workloads' M values), each line beside torch's
    non-invariant kernel on the same tensors. Prints a markdown table."""
    def timed(f, it=None):
        """Mean device time per call. The calls are captured once into a
        HIP graph and the graph is replayed, so short kernels are timed
        without the Python/ctypes launch overhead between them."""
        n = it or 20
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            f()  # warm the side stream (allocations made by torch ops)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=side):
                for _ in range(n):
                    f()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3

    rows = ["| op | shape | M | bi us | bi rate | bi % roofline | torch us | tax (bi/torch) | fixed-tile us |",
            "|---|---|---|---|---|---|---|---|---|"]

    def line(op, shape, m, t, f, b, tt, tf=None):
        tm = t_min(f, b)
        bound_mfma = f / PEAK_BF16 >= b / PEAK_HBM
        rate = f"{f / t / 1e12:.1f} TFLOP/s" if bound_mfma else f"{b / t / 1e12:.2f} TB/s"
        rows.append(f"| {op} | {shape} | {m} | {t * 1e6:.1f} | {rate} | {100 * tm / t:.1f} | "
                    f"{'' if tt is None else f'{tt * 1e6:.1f}'} | {'' if tt is None else f'{t / tt:.2f}'} | "
                    f"{'' if tf is None else f'{tf * 1e6:.1f}'} |")
        log(rows[-1])

    dev = "cuda:0"
    for (k, n), ms in [((512, 512), (1, 2, 3, 8, 16)), ((4096, 6144), (1, 8, 64, 512, 4096)),
                       ((4096, 4096), (1, 8, 64, 512, 4096)), ((4096, 24576), (1, 8, 64, 512, 4096)),
                       ((12288, 4096), (1, 8, 64, 512, 4096))]:
        w = S.normal_bf16((k, n), 0.02, seed=7, device=dev)
        for m in ms:
            a = S.normal_bf16((m, k), 1.0, seed=m, device=dev)
            c = torch.empty((m, n), device=dev)
            t = timed(lambda: bi.bi_mm(a, w, out=c))
            tt = timed(lambda: torch.mm(a, w, out_dtype=torch.float32))
            tf = timed(lambda: bi.bi_gemm(a, w, out=c, fixed_tile=True))
            line("bi_mm", f"K={k} N={n}", m, t, *gemm_work(m, n, k), tt, tf)
    k, n = HIDDEN, VOCAB
    w = S.normal_bf16((k, n), 0.02, seed=8, device=dev)
    bias = S.normal_bf16((n,), 0.1, seed=9, device=dev)
    for m in (1, 32, 256):
        x = S.normal_bf16((m, k), 1.0, seed=m, device=dev)
        c = torch.empty((m, n), device=dev)
        t = timed(lambda: bi.bi_addmm(bias, x, w, out=c), 10)
        tt = timed(lambda: torch.addmm(bias, x, w, out_dtype=torch.float32), 10)
        tf = timed(lambda: bi.bi_gemm(x, w, bias, out=c, fixed_tile=True), 10)
        line("bi_addmm (LM head)", f"K={k} N={n}", m, t, *gemm_work(m, n, k, bias=True), tt, tf)
        lp = torch.empty_like(c)
        am = torch.empty((m,), dtype=torch.int64, device=dev)
        t = timed(lambda: bi.bi_log_softmax(c, out=lp, argmax=am))
        tt = timed(lambda: (torch.log_softmax(c, -1), torch.argmax(c, -1)))
        line("bi_log_softmax+argmax (LM head)", f"N={n}", m, t, 5.0 * m * n, 8.0 * m * n + 8 * m, tt)
    F = torch.nn.functional
    wr = S.uniform_bf16((HIDDEN,), 0.5, 1.5, seed=10, device=dev)
    for m in (1, 7, 64, 513, 2048):
        x = S.normal_bf16((m, HIDDEN), 1.0, seed=m, device=dev)
        y = torch.empty_like(x)
        t = timed(lambda: bi.bi_rmsnorm(x, wr, 1e-6, out=y))
        tt = timed(lambda: F.rms_norm(x, (HIDDEN,), wr, 1e-6))
        line("bi_rmsnorm", f"N={HIDDEN}", m, t, 4.0 * m * HIDDEN, 4.0 * m * HIDDEN + 2 * HIDDEN, tt)
        ym = torch.empty((m,), device=dev)
        t = timed(lambda: bi.bi_mean(x, out=ym))
        tt = timed(lambda: torch.mean(x, dim=1, dtype=torch.float32))
        line("bi_mean", f"N={HIDDEN}", m, t, 1.0 * m * HIDDEN, 2.0 * m * HIDDEN + 4 * m, tt)
        lx = S.normal_f32((m, VOCAB), 4.0, seed=m, device=dev)
        ly = torch.empty_like(lx)
        am = torch.empty((m,), dtype=torch.int64, device=dev)
        t = timed(lambda: bi.bi_log_softmax(lx, out=ly, argmax=am))
        tt = timed(lambda: (torch.log_softmax(lx, -1), torch.argmax(lx, -1)))
        line("bi_log_softmax+argmax", f"N={VOCAB}", m, t, 5.0 * m * VOCAB, 8.0 * m * VOCAB + 8 * m, tt)
    for bsz in (1, 8, 64, 256):
        lens = S.context_lens(bsz, seed=6000 + bsz)
        table, npages = S.paged_kv_layout(lens, 16, seed=6001)
        q = S.normal_bf16((bsz, 32, 128), 1.0, seed=6002, device=dev)
        kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=6003, device=dev)
        vp = S.normal_bf16((npages, 8, 128, 16), 1.0, seed=6004, device=dev)
        offs, total = bi.bi_decode_plan(lens)
        ws = torch.empty(bi.bi_decode_workspace_bytes(total, 32, 128), dtype=torch.uint8, device=dev)
        out = torch.empty((bsz, 32, 128), device=dev)
        tb, ld, of = table.to(dev), lens.to(dev), offs.to(dev)
        t = timed(lambda: bi.bi_decode_attention(q, kp, vp, tb, ld, of, total, workspace=ws, out=out), 10)
        tok = int(lens.sum())
        byts = 4096.0 * tok + bsz * 32 * 128 * 6 + 4.0 * int(((lens + 15) // 16).sum())
        line("bi_decode_attention", f"B={bsz}, {tok} tokens", bsz, t, 4.0 * 32 * 128 * tok, byts, None)
    print("\n".join(rows))


E2E_BATCH = 64
E2E_STEPS = 3


def e2e_decode(torch, S, bi, dev, steps=E2E_STEPS, warmup=1, batch_size=E2E_BATCH):
    """Greedy decode steps of a Qwen3-8B-shaped model (all 36 layers, random
    weights) for batch_size sequences whose cached lengths are log-uniform
    in [1, 32768], every step through the library's kernels. Reported next
    to the per-kernel metric, not folded into it. Its roofline: the bytes a
    step must move at least (every weight once, the whole KV cache once,
    activations and logits) over 8 TB/s."""
    from invariant_bi_mm_amd.decode import QWEN3_8B, Batch, Decoder
    s = QWEN3_8B
    t0 = time.time()
    w = S.qwen3_weights(s.hidden, s.num_q_heads, s.num_kv_heads, s.head_dim, s.intermediate, s.vocab, s.layers,
                        seed=20000, device=dev)
    lens = S.context_lens(batch_size, seed=21000)
    room = steps + warmup
    table, num_pages = S.paged_kv_layout(lens + room, s.page_size, seed=21001)
    dec = Decoder(s, w, num_pages=num_pages, device=dev)
    for l in range(s.layers):  # the cached context: random keys and values
        dec.k_pages[l].normal_()
        dec.v_pages[l].normal_()
    batch = Batch(block_table=table.to(dev), lens=lens.clone())
    tok = torch.randint(0, s.vocab, (batch_size,), generator=S.generator(21002)).to(dev)
    torch.cuda.synchronize()
    log(f"e2e decode: weights + {num_pages} cache pages x {s.layers} layers ready in {time.time() - t0:.1f}s")
    for _ in range(warmup):
        _, _, tok = dec.step(tok, batch)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        _, _, tok = dec.step(tok, batch)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / steps
    # the same steps replayed from one captured graph (no host launch cost between kernels)
    gs = dec.graph(batch, steps + 1)
    gs.run(tok)
    torch.cuda.synchronize()
    ctx0 = int(batch.lens.sum())
    t_host = time.perf_counter()
    e0.record()
    for _ in range(steps):
        gs.run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ms_wall = (time.perf_counter() - t_host) * 1e3 / steps
    h, i_, v = s.hidden, s.intermediate, s.vocab
    qkv_n = (s.num_q_heads + 2 * s.num_kv_heads) * s.head_dim
    w_bytes = 2 * s.layers * (h * qkv_n + h * h + h * 2 * i_ + i_ * h) + 2 * h * v + 2 * v
    ctx_mid = ctx0 + batch_size * (steps + 1) / 2  # cached tokens read, averaged over the timed graph steps
    kv_bytes = 2 * 2 * s.num_kv_heads * s.head_dim * s.layers * ctx_mid
    act_bytes = batch_size * (2 * h + 4 * v * 3 + 8)  # embed row, logits + log-probs written, logits read, token
    t_min_ms = (w_bytes + kv_bytes + act_bytes) / PEAK_HBM * 1e3
    res = {"model": "Qwen3-8B-shaped (36 layers, hidden 4096, 32/8 heads, intermediate 12288, vocab 151936), "
                    "random weights", "batch": batch_size, "context_tokens_at_start": ctx0,
           "steps": steps, "ms_per_step": round(ms, 3), "tokens_per_s": round(batch_size / (ms / 1e3), 1),
           "mode": "one captured HIP graph replayed per step (host refreshes lengths/offsets between replays)",
           "ms_per_step_wall": round(ms_wall, 3), "ms_per_step_eager_launches": round(ms_eager, 3),
           "hbm_bytes_min_per_step": w_bytes + kv_bytes + act_bytes, "roofline_frac": round(t_min_ms / ms, 4)}
    log(f"e2e decode: {ms:.2f} ms/step at batch {batch_size} ({res['tokens_per_s']:.0f} tokens/s), "
        f"{100 * t_min_ms / ms:.1f}% of the HBM bound ({t_min_ms:.2f} ms); eager launches {ms_eager:.2f} ms/step")
    del dec, w, gs
    torch.cuda.empty_cache()
    return res


PREFILL_SEQS, PREFILL_TOKENS = 4, 2048


def cold_read(torch, S, bi, dev, reps=9):
    """Cold reads with clean or dirty caches. A 1 GiB buffer is either read
    (the caches then hold clean lines) or written (the Infinity Cache then
    holds dirty lines, each evicted by a later miss with a write-back) before
    every timed launch. Timed: a plain read of the 201 MB gate+up weight
    (bi_mean over its 24576 rows), and bi_mm on the decode step's projections at
    M = 1 and 64 with the weights stored [N,K]. Median of the timed launches;
    rates in bytes of weights per second."""
    fl = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.zeros((), device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, dirty):
        ts = []
        for rep in range(reps + 1):
            if dirty:
                fl.fill_(float(rep))
            else:
                sink.copy_(fl.sum())
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts = sorted(ts[1:])
        return ts[len(ts) // 2]

    res = {}
    w_gu = S.normal_bf16((24576, 4096), 0.02, seed=2, device=dev)
    means = torch.empty(24576, device=dev)
    for dirty in (False, True):
        key = "after_write" if dirty else "after_read"
        t = timed(lambda: bi.bi_mean(w_gu, out=means), dirty)
        res[f"read_201MB_{key}"] = {"us": round(t, 1), "TB/s": round(w_gu.numel() * 2 / t / 1e6, 2)}
    for name, k, n in (("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 24576), ("down", 12288, 4096)):
        w = S.normal_bf16((n, k), 0.02, seed=3, device=dev)
        for m in (1, 64):
            a = S.normal_bf16((m, k), 1.0, seed=4, device=dev)
            c = torch.empty((m, n), device=dev)
            for dirty in (False, True):
                t = timed(lambda: bi.bi_mm(a, w, b_is_nk=True, out=c), dirty)
                res[f"bi_mm_{name}_M{m}_{'after_write' if dirty else 'after_read'}"] = {
                    "us": round(t, 1), "TB/s": round(2.0 * n * k / t / 1e6, 2)}
        del w
    return res


def prefill_measure(torch, S, bi, dev, reps=5):
    """Causal prefill attention of PREFILL_SEQS prompts of PREFILL_TOKENS
    tokens (Qwen3-8B heads: 32 q / 8 kv, head_dim 128, one layer), with the
    decode split structure so every token's output equals its decode-step
    bits. q.k and p.v both run on the bf16 matrix cores (p.v with p as two
    bf16 parts, which doubles its MFMA work; the bound counts the algorithmic
    flops only): each product is 2 * D * Hq * sum over tokens of
    (position + 1) flops, so the bound is t_min = flops / 2.5 PFLOP/s."""
    n, T = PREFILL_SEQS, PREFILL_TOKENS
    lens = torch.full((n,), T, dtype=torch.int32)
    table, npages = S.paged_kv_layout(lens, 16, seed=22000)
    kp = S.normal_bf16((npages, 8, 16, 128), 1.0, seed=22001, device=dev)
    vp = S.normal_bf16((npages, 8, 128, 16), 1.0, seed=22002, device=dev)
    q = S.normal_bf16((n * T, 32, 128), 1.0, seed=22003, device=dev)
    q_pos, q_offs, work, sizes = bi.bi_prefill_plan(lens, torch.zeros(n, dtype=torch.int32))
    qp, qo, wk, tb = q_pos.to(dev), q_offs.to(dev), work.to(dev), table.to(dev)
    ws = torch.empty(bi.bi_decode_workspace_bytes(sizes[1], 32, 128), dtype=torch.uint8, device=dev)
    out = torch.empty((n * T, 32, 128), dtype=torch.float32, device=dev)
    f = lambda: bi.bi_prefill_attention(q, kp, vp, tb, qp, qo, wk, sizes, workspace=ws, out=out)  # noqa: E731
    f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    half = 2.0 * 128 * 32 * n * (T * (T + 1) / 2)  # q.k and p.v each
    t_min_ms = (2 * half / PEAK_BF16) * 1e3
    res = {"sequences": n, "tokens_per_sequence": T, "ms": round(ms, 3), "TFLOP/s": round(2 * half / ms / 1e9, 1),
           "bound": "mfma: q.k and p.v on bf16 matrix cores", "t_min_ms": round(t_min_ms, 3),
           "frac": round(t_min_ms / ms, 4), "tokens_per_s": round(n * T / (ms / 1e3))}
    log(f"prefill attention: {n} x {T} tokens in {ms:.3f} ms, {res['TFLOP/s']} TFLOP/s, "
        f"{100 * res['frac']:.1f}% of its bound ({t_min_ms:.3f} ms)")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--no-torch", action="store_true", help="skip the non-invariant torch baseline")
    ap.add_argument("--no-e2e", action="store_true",
                    help="skip the end-to-end decode-step and prefill measurements")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"),
                    help="measured HBM traffic per kernel (written from rocprofv3 FETCH_SIZE/WRITE_SIZE runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="per-config sweep over the workloads' M values (markdown table), then exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only measure the prefill attention workload (4 x 2048 tokens) and print its JSON")
    ap.add_argument("--cold-read", action="store_true",
                    help="only time cold reads after a read-only or a write flush (a 201 MB weight and the "
                         "decode step's small-M GEMMs) and print their JSON")
    ap.add_argument("--e2e-only", action="store_true",
                    help="only measure the end-to-end decode step (36 layers, batch 64) and print its JSON")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only run each projection GEMM at M = 64, 512 and 4096 and the LM head at M = 256, "
                         "3 launches each ([K,N] weights, fp32 out), for rocprofv3 counter and trace runs; "
                         "prints which launch is which and exits")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for scaling the HBM counters) and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="no GPU: turn the rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR (fetch/, write/, "
                         "cal_fetch/, cal_write/) into the --traffic JSON and print the per-op table")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.traffic)
        return
    if args.copy_calibration:
        import torch
        nbytes = 256 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}))
        return
    if args.gemm_probe:
        import torch
        import invariant_bi_mm_amd as bi
        import synthetic as S
        dev = "cuda:0"
        cases = [(m, k, n) for (_, k, n) in GEMMS for m in (64, 512, 4096)] + [(M_LM, HIDDEN, VOCAB)]
        for m, k, n in cases:
            a = S.normal_bf16((m, k), 1.0, seed=m, device=dev)
            w = S.normal_bf16((k, n), 0.02, seed=7, device=dev)
            c = torch.empty((m, n), device=dev)
            torch.cuda.synchronize()
            for _ in range(3):
                bi.bi_mm(a, w, out=c)
            torch.cuda.synchronize()
            print(json.dumps({"M": m, "K": k, "N": n, "launches": bi.bi_gemm_plan(m, n, k), "reps": 3}), flush=True)
            del a, w, c
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (each GPU would run it "
              "on its own shard of rows, columns or sequences). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_bi_mm_amd as bi
    import synthetic as S
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(torch, S, bi)
        return
    if args.prefill_only:
        print(json.dumps(prefill_measure(torch, S, bi, dev)), flush=True)
        return
    if args.cold_read:
        print(json.dumps(cold_read(torch, S, bi, dev)), flush=True)
        return
    if args.e2e_only:
        print(json.dumps(e2e_decode(torch, S, bi, dev)), flush=True)
        return
    wl = Workload(torch, S, bi, dev)
    ops = wl.ops()
    clocks_before = gpu_clocks()
    ms_eager, per = time_step(torch, ops, args.steps, args.warmup)
    dist = time_step.last_dist
    # the timed step: the same launches replayed as one HIP graph (no host
    # launch gaps); the per-kernel times above come from the eager run
    ms_step = time_step_graph(torch, ops, args.steps, args.warmup,
                              check=(wl.attn_out, wl.lm_logits, wl.ly, wl.ry))
    clocks_after = gpu_clocks()
    tmin = {name: t_min(f, b) for name, _, f, b in ops}
    work = {name: (f, b) for name, _, f, b in ops}
    sum_tmin_ms = sum(tmin.values()) * 1e3
    value = 100.0 * sum_tmin_ms / ms_step

    log(f"{'kernel':12s} {'ms':>9s} {'t_min ms':>9s} {'frac':>6s} {'TFLOP/s':>9s} {'GB/s':>9s}")
    for name, *_ in ops:
        f, b = work[name]
        log(f"{name:12s} {per[name]:9.4f} {tmin[name] * 1e3:9.4f} {tmin[name] * 1e3 / per[name]:6.3f} "
            f"{f / per[name] / 1e9:9.1f} {b / per[name] / 1e6:9.1f}")
    log(f"step: {ms_step:.3f} ms as a replayed graph ({ms_eager:.3f} ms eager; sum of kernel events "
        f"{sum(per.values()):.3f} ms), sum t_min {sum_tmin_ms:.3f} ms -> {value:.1f}% of roofline")

    gemm_names = [g[0] for g in GEMMS] + ["lm_head"]
    red_names = ["rmsnorm", "mean", "logsm", "lm_logsm"]

    def group(names, use_flops):
        t = sum(per[n] for n in names) / 1e3
        amount = sum(work[n][0 if use_flops else 1] for n in names)
        frac = sum(tmin[n] for n in names) / t
        return amount / t, frac

    g_tf, g_frac = group(gemm_names, True)
    r_bw, r_frac = group(red_names, False)
    a_bw, a_frac = group(["decode_attn"], False)

    dom = max(per, key=lambda n: per[n])
    f, b = work[dom]
    is_mfma = f / PEAK_BF16 >= b / PEAK_HBM
    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        with open(args.traffic) as fh:
            rec = json.load(fh)
        # counters are only valid for the kernel source they were taken on
        kr = rec.get("kernels", {}).get(dom, {})
        if kr.get("source_sha256") == source_digest(dom):
            traffic = kr.get("hbm_bytes_per_launch")
    if is_mfma:
        roof = {"bound": "mfma", "achieved": f / (per[dom] / 1e3) / 1e12, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": b / (per[dom] / 1e3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = {"flops": f, "bytes": b}
    roof["avg_launch_ms"] = per[dom]

    e2e = None if args.no_e2e else e2e_decode(torch, S, bi, dev)
    pre = None if args.no_e2e else prefill_measure(torch, S, bi, dev)

    torch_base = None
    if not args.no_torch:
        tops = [(n, fn, *work[n]) for n, fn in wl.torch_ops()]
        t_ms, t_per = time_step(torch, tops, max(5, args.steps // 2), 2)
        bi_same = sum(per[n] for n in t_per)
        torch_base = {"ms_per_step_without_decode": t_ms, "per_kernel_ms": {k: round(v, 4) for k, v in t_per.items()},
                      "invariance_tax": bi_same / sum(t_per.values()),
                      "note": "torch.mm/addmm with out_dtype=float32 (hipBLASLt/rocBLAS as dispatched), F.rms_norm, torch.mean, "
                              "torch.log_softmax+argmax on the same tensors; decode attention has no torch "
                              "counterpart here"}
        torch_base["negative_control"] = negative_control(torch, S, dev)
        log(f"torch baseline: {t_ms:.3f} ms/step (no decode); tax bi/torch on the same kernels "
            f"{torch_base['invariance_tax']:.3f}x; negative control {torch_base['negative_control']}")

    cpu = None
    if not args.no_cpu:
        t_cpu, parts, threads, sample = cpu_baseline(wl, S)
        cpu = {"value": 100.0 * sum_tmin_ms / (t_cpu * 1e3), "unit": "% of MI355X roofline (same step)",
               "cores": threads, "core_counts": cpu_baseline.cores, "kind": "oracle", "sample": sample,
               "step_seconds_extrapolated": t_cpu,
               "per_kernel_seconds": {k: round(v, 3) for k, v in parts.items()}}
        log(f"cpu oracle: {t_cpu:.1f} s per step (extrapolated), threads={threads}")

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "% roofline (sum of per-kernel roofline times / measured step time)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "step_timing": "one HIP graph of the step's launches, replayed (bits checked equal to an eager step); "
                       "per-kernel times from an eager run with HIP events around each launch",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen3-8B-shaped invariant step: 4 projection GEMMs at M=4096 (fp32 out), "
                               "LM-head addmm M=256 + log_softmax/argmax, RMSNorm+mean 2048x4096, "
                               "log_softmax+argmax 2048x151936, decode attention B=256 (split 256)",
                   "gemm_m": M_GEMM, "lm_head_m": M_LM, "row_m": M_ROWS, "decode_batch": B_DECODE,
                   "decode_tokens": int(wl.lens.sum()), "accumulate": "fp32"},
        "components": {
            "gemm": {"TFLOP/s": round(g_tf / 1e12, 2), "frac": round(g_frac, 4)},
            "reductions": {"GB/s": round(r_bw / 1e9, 1), "frac": round(r_frac, 4)},
            "decode_attention": {"GB/s": round(a_bw / 1e9, 1), "frac": round(a_frac, 4)},
        },
        "per_kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "per_kernel_ms_dist": dist,
        "clocks": {"before": clocks_before, "after": clocks_after},
        "roofline": roof,
        "e2e_decode_step": e2e,
        "prefill_attention": pre,
        "torch_baseline": torch_base,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
