#!/usr/bin/env python3
"""Benchmark of the Flux single-stream DiT block forward on one MI355X.

A step is one denoising step of a 57-block stack of Flux-shaped
single-stream blocks (S=4608, dim 3072, 24 heads x 128, MLP 12288, bf16,
independent random weights), replayed as one captured hipGraph per step.
The headline value is milliseconds per block forward (step time / 57,
HIP events on the replay stream around exactly K steps).  Beside it:
per-kernel times inside the replayed graph (device wall-clock stamp kernels
around every kernel of every block in a second replay of the same steps:
GEMM TFLOP/s, attention TFLOP/s), the fused LayerNorm+modulate and
gated-residual HBM GB/s (graph-timed, with buffer rotation so the 256 MB
last-level cache cannot hold the working set) against the same-size copy
probe, the roofline fraction of the dominant kernel with its byte counters,
kernels per block and launch gaps from a committed rocprofv3 trace, the
copy and MFMA ceilings, the other configurations and legs, and the CPU
oracle's time on the host cores.

Prints ONE JSON line on stdout.  Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--blocks 57] [--no-cpu-baseline]
  python bench.py --kernels-only linear1_gelu,copy --kernel-iters 3   (profiler runs)
  python bench.py --trace-summary <rocprofv3 output dir>               (kernels per block, gaps)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per DiT block forward (S=4608,d=3072 bf16) + fused-norm HBM GB/s"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
S, D, H, DH, MLP = 4608, 3072, 24, 128, 12288
N1, N2 = 3 * D + MLP, D + MLP
GEMM1_FLOP = 2.0 * S * D * N1
GEMM2_FLOP = 2.0 * S * N2 * D
ATTN_FLOP = 4.0 * H * S * S * DH
BLOCK_FLOP = GEMM1_FLOP + GEMM2_FLOP + ATTN_FLOP + 2.0 * 3 * D * D
NORM_BYTES = 2 * S * D * 2                   # read x, write u (bf16)
GRES_BYTES = 3 * S * D * 2                   # read x and h, write y
QKNORM_BYTES = 4 * S * D * 2                 # read and write q and k
MOD_BYTES = 3 * D * D * 2                    # the modulation weight


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the GEMM sources with comments and blank lines removed: the
    stored traffic counters stay valid across comment-only edits and are
    dropped on any change of the code."""
    import re
    h = hashlib.sha256()
    for name in ("gemm.hip", "dit_common.hpp"):
        with open(os.path.join(ROOT, "diffusion_transformer_dit_amd", "csrc", name)) as f:
            src = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = [ln.split("//", 1)[0].rstrip() for ln in src.splitlines()]
        h.update("\n".join(ln for ln in lines if ln.strip()).encode())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    PMC summary, or None when it is absent or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "gemm_linear1_flux_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def load_launch_gaps():
    """Kernels per block and the gaps between kernels inside the replayed
    steps, from the committed summary of a rocprofv3 kernel trace of this
    bench (written by --trace-summary), or None when it is absent."""
    path = os.path.join(ROOT, "profiles", "flux_stack_launch_gaps.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    keep = ("kernels_per_block", "kernels_per_step", "gap_us_per_step_mean", "mean_gap_us", "max_gap_us",
            "gap_frac", "steps")
    out = {k: t.get(k) for k in keep}
    out["source"] = "profiles/flux_stack_launch_gaps.json (rocprofv3 kernel trace)"
    return out


def time_launches(fn, iters, warm=2):
    import torch
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        fn(i)
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def time_graph(fn, iters, replays=3):
    """Mean ms per launch of `iters` launches fn(0..iters-1) captured into one
    graph and replayed: launch gaps are the graph's, not the Python loop's
    (short kernels would otherwise be timed at the host's launch rate)."""
    import torch
    fn(0)
    fn(1 % iters)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(iters):
                fn(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / (replays * iters)
    del g
    return ms


KERNEL_NAMES = ("modulation", "block_modulate_norm", "modulate_norm", "linear1_gelu", "qk_rmsnorm_rope",
                "attention", "linear2_gated_residual", "gated_residual", "copy", "block_forward", "other_blocks",
                "config_blocks", "ceilings")


def block_sequence_times(B, blocks, x_in, temb, rc, rs, iters, only=None):
    """Per-kernel durations measured as the kernels run in the block: `iters`
    eager block forwards (the same six launches, in the same order, as one
    block of the replayed stack), each launch bracketed by HIP events on the
    stream it is launched on.  Returns {name: mean ms per launch}."""
    import torch
    want = lambda n: only is None or n in only
    dev = x_in.device
    nb = len(blocks)
    u = torch.empty(S, D, dtype=torch.bfloat16, device=dev)
    qkv = torch.empty(S, 3 * D, dtype=torch.bfloat16, device=dev)
    cat = torch.empty(S, N2, dtype=torch.bfloat16, device=dev)
    y = torch.empty(S, D, dtype=torch.bfloat16, device=dev)
    mod = torch.empty(3 * D, dtype=torch.float32, device=dev)
    seq = [
        ("modulation", lambda w: B.modulation(temb[0], w.tensors[0], w.tensors[1], out=mod)),
        ("block_modulate_norm", lambda w: B.modulate_norm(x_in, mod[:D], mod[D:2 * D], 1e-6, out=u)),
        ("linear1_gelu", lambda w: B.linear1_gelu(u, w.tensors[2], w.tensors[3], qkv, cat, MLP)),
        ("qk_rmsnorm_rope", lambda w: B.qk_rmsnorm_rope(qkv, w.tensors[6], w.tensors[7], rc, rs, H, DH)),
        ("attention", lambda w: B.attention(qkv, cat, H, DH)),
        ("linear2_gated_residual", lambda w: B.linear2_gated_residual(cat, w.tensors[4], w.tensors[5], x_in,
                                                                      mod[2 * D:], y)),
    ]
    ev = {n: [] for n, _ in seq}
    for i in range(iters + 1):
        w = blocks[i % nb]
        for name, fn in seq:
            if i > 0 and want(name):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn(w)
                b.record()
                ev[name].append((a, b))
            else:
                fn(w)
    torch.cuda.synchronize()
    return {n: sum(a.elapsed_time(b) for a, b in v) / len(v) for n, v in ev.items() if v}


def hbm_kernel_times(B, g, dev, it, only=None):
    """HBM rates of the memory-bound kernels at the chain shape: each launch
    works on one of 12 buffer sets (12 x 56.6 MB > the 256 MB last-level
    cache), so the data comes from HBM; the launches are captured in a graph
    and replayed.  Returns ({name: ms}, cache-warm ms of modulate_norm)."""
    import torch
    want = lambda n: only is None or n in only
    randn = lambda shape: torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    k, warm = {}, None
    if want("copy"):
        # calibration for byte counters: a plain copy of a known size (256 MiB read + 256 MiB written)
        src = torch.empty(128 * 1024 * 1024, dtype=torch.bfloat16, device=dev).normal_(generator=g)
        dst = torch.empty_like(src)
        k["copy"] = time_launches(lambda i: dst.copy_(src), min(it, 5))
        del src, dst
    if want("modulate_norm") or want("gated_residual"):
        nrot = 12
        xs = [randn((S, D)) for _ in range(nrot)]
        hs = [randn((S, D)) for _ in range(nrot)]
        us = [torch.empty(S, D, dtype=torch.bfloat16, device=dev) for _ in range(nrot)]
        shift = torch.randn(D, generator=g, device=dev) * 0.1
        scale = torch.randn(D, generator=g, device=dev) * 0.1
        gvec = torch.randn(D, generator=g, device=dev) * 0.1
        n = max(it, 4 * nrot)
        if want("modulate_norm"):
            k["modulate_norm"] = time_graph(
                lambda i: B.modulate_norm(xs[i % nrot], shift, scale, 1e-6, out=us[i % nrot]), n)
            warm = time_graph(lambda i: B.modulate_norm(xs[0], shift, scale, 1e-6, out=us[0]), n)
        if want("gated_residual"):
            k["gated_residual"] = time_graph(
                lambda i: B.gated_residual(xs[i % nrot], hs[i % nrot], gvec, out=us[i % nrot]), n)
    if want("qk_rmsnorm_rope"):
        # the standalone entry point (the block fuses it into linear1 at this
        # shape): 4 rotating qkv buffers of 85 MB, more than the 256 MB cache
        nq = 4
        qkvs = [randn((S, 3 * D)) for _ in range(nq)]
        pos = torch.arange(S, device=dev, dtype=torch.float32)[:, None]
        ang = pos * torch.exp2(-torch.arange(DH // 2, device=dev, dtype=torch.float32) / 8.0)[None, :]
        rc, rs = torch.cos(ang).contiguous(), torch.sin(ang).contiguous()
        qw = torch.ones(DH, device=dev)
        k["qk_rmsnorm_rope_standalone"] = time_graph(
            lambda i: B.qk_rmsnorm_rope(qkvs[i % nq], qw, qw, rc, rs, H, DH), max(it, 8 * nq))
        del qkvs
    torch.cuda.synchronize()
    return k, warm


def chunked_attention_times(B, g, dev, reps=3):
    """The one-GPU math of the pages' ring attention at the Flux shape: 8 key
    chunks of 576 tokens (dit_attention_partial) merged by log-sum-exp
    (dit_attention_merge), against the single-pass kernel; and the share of
    one rank under an 8-way head split (3 heads x 4608 tokens)."""
    import torch
    C = 8
    qkv = (torch.randn(S, 3 * D, generator=g, device=dev, dtype=torch.float32)).to(torch.bfloat16)
    o_parts = torch.empty(C, S, D, dtype=torch.float32, device=dev)
    lses = torch.empty(C, H, S, dtype=torch.float32, device=dev)
    out = torch.empty(S, D, dtype=torch.bfloat16, device=dev)
    ck = S // C

    def partials(i):
        for c in range(C):
            B.attention_partial(qkv, H, DH, c * ck, (c + 1) * ck, o_part=o_parts[c], lse=lses[c])

    res = {"chunks": C, "chunk_tokens": ck}
    res["partials_ms"] = time_graph(partials, 1, reps)
    res["merge_ms"] = time_graph(lambda i: B.attention_merge(o_parts, lses, out, H, DH), 4, reps)
    res["single_pass_ms"] = time_graph(lambda i: B.attention(qkv, out, H, DH), 4, reps)
    hq = 3
    qkv3 = (torch.randn(S, 3 * hq * DH, generator=g, device=dev, dtype=torch.float32)).to(torch.bfloat16)
    out3 = torch.empty(S, hq * DH, dtype=torch.bfloat16, device=dev)
    res["ulysses_share_3heads_ms"] = time_graph(lambda i: B.attention(qkv3, out3, hq, DH), 8, reps)
    # the same share with the keys split over more workgroups (one launch of
    # chunk partials + the merge): 108 workgroups x n chunks
    op3 = torch.empty(8, S, hq * DH, dtype=torch.float32, device=dev)
    ls3 = torch.empty(8, hq, S, dtype=torch.float32, device=dev)
    res["ulysses_share_3heads_split_ms"] = {
        n: time_graph(lambda i, n=n: B.attention_split(qkv3, out3, hq, DH, n, o_parts=op3, lses=ls3), 8, reps)
        for n in (2, 4, 6, 8)}
    del o_parts, lses, qkv, qkv3, op3, ls3
    torch.cuda.synchronize()
    return res


def other_block_times(B, g, dev, reps=3):
    """One block forward of the other block kinds, captured in a graph and
    replayed: the two-stream (MMDiT) block at the Flux shape (512 text + 4096
    image tokens, each stream with its own weights) and the sequential block
    at the video shape (S=16384, d=1536, 12x128, MLP 8960, 3D RoPE)."""
    import torch
    import dit_inputs as DI

    def rnd(shape, sigma=0.02):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * sigma).to(torch.bfloat16)

    def stream(d, mlp, dh):
        one = torch.ones(dh, device=dev)
        return B.StreamWeights(rnd((6 * d, d)), rnd((6 * d,)), rnd((3 * d, d)), rnd((3 * d,)), one, one,
                               rnd((d, d)), rnd((d,)), rnd((mlp, d)), rnd((mlp,)), rnd((d, mlp)), rnd((d,)))

    res = {}
    for name, sh, n_txt in (("mmdit_double_block", DI.FLUX_DOUBLE, 512), ("sequential_video_block", DI.VIDEO, 0)):
        d, mlp, dh = sh.dim, sh.mlp_hidden, sh.head_dim
        cfg = B.make_config(sh.seq_len, d, sh.num_heads, dh, mlp)
        ws = B.alloc_workspace(B.mmdit_block_workspace_bytes(cfg))
        pos = torch.from_numpy(DI.positions(sh)).to(dev)
        rc, rs = B.rope_table(pos, list(sh.rope_axes_dims), dh)
        x = rnd((sh.seq_len, d), 1.0)
        temb = rnd((d,), 1.0)
        y = torch.empty_like(x)
        wi = stream(d, mlp, dh)
        wt = stream(d, mlp, dh) if n_txt else None
        ms = time_graph(lambda i: B.mmdit_block_forward(cfg, n_txt, wt, wi, x, temb, rc, rs, y=y, workspace=ws),
                        4, reps)
        S = sh.seq_len
        flop = 2.0 * S * d * (4 * d + 2 * mlp) + 4.0 * sh.num_heads * S * S * dh + 2 * 6.0 * d * d * (2 if n_txt else 1)
        res[name] = dict(S=S, text_tokens=n_txt, dim=d, heads=sh.num_heads, mlp_hidden=mlp, ms=round(ms, 4),
                         gflop=round(flop / 1e9, 1), tflops=round(flop / (ms * 1e-3) / 1e12, 1))
        del ws, x, y, wi, wt
    torch.cuda.synchronize()
    return res


def block_flop(S_, d, H_, dh, mlp):
    """Algorithmic flops of one single-stream block forward: linear1, linear2,
    attention (QK^T and PV) and the modulation GEMV."""
    return 2.0 * S_ * d * (3 * d + mlp) + 2.0 * S_ * (d + mlp) * d + 4.0 * H_ * S_ * S_ * dh + 2.0 * 3 * d * d


def config_block_times(B, g, dev, reps=3):
    """One single-stream block forward at the other configurations of the
    workload list, captured in a graph and replayed: the tiny block (S=256,
    d=256, 4x64, MLP 1024, 2D RoPE on 16x16) and the long-sequence video
    block (S=16384, d=1536, 12x128, MLP 8960, 3D RoPE on 16x32x32)."""
    import torch
    import dit_inputs as DI
    res = {}
    for name, sh in (("tiny_block", DI.TINY), ("video_block", DI.VIDEO)):
        d, mlp, dh, H_, S_ = sh.dim, sh.mlp_hidden, sh.head_dim, sh.num_heads, sh.seq_len
        rnd = lambda shape, sigma=0.02: (torch.randn(shape, generator=g, device=dev) * sigma).to(torch.bfloat16)
        w = B.BlockWeights(rnd((3 * d, d)), rnd((3 * d,)), rnd((3 * d + mlp, d)), rnd((3 * d + mlp,)),
                           rnd((d, d + mlp)), rnd((d,)), torch.ones(dh, device=dev), torch.ones(dh, device=dev))
        cfg = B.make_config(S_, d, H_, dh, mlp)
        ws = B.alloc_workspace(B.block_workspace_bytes(cfg))
        pos = torch.from_numpy(DI.positions(sh)).to(dev)
        rc, rs = B.rope_table(pos, list(sh.rope_axes_dims), dh)
        x = rnd((S_, d), 1.0)
        temb = rnd((d,), 1.0)
        y = torch.empty_like(x)
        n = 64 if S_ <= 1024 else 4
        ms = time_graph(lambda i: B.block_forward(cfg, w, x, temb, rc, rs, y=y, workspace=ws), n, reps)
        flop = block_flop(S_, d, H_, dh, mlp)
        tfl = flop / (ms * 1e-3) / 1e12
        res[name] = dict(S=S_, dim=d, heads=H_, head_dim=dh, mlp_hidden=mlp, ms=round(ms, 4),
                         gflop=round(flop / 1e9, 2), tflops=round(tfl, 1), frac=round(tfl / BF16_PEAK_TFLOPS, 4))
        del w, ws, x, y
    torch.cuda.synchronize()
    return res


def ceiling_times(B, g, dev, reps=3):
    """What the chip delivers: the streaming copy at the chain's sizes (12
    rotating buffer sets, more than the 256 MB last-level cache) and at 1
    and 4 GiB, and bf16 MFMA throughput with fixed and with changing
    operands.  Copy GB/s count bytes read plus bytes written."""
    import torch
    res = {"copy": {}, "mfma": {}}
    for label, nbytes, nrot in (("56.6MB_moved", S * D * 2, 12), ("84.9MB_moved", S * D * 3, 12),
                                ("1GiB_moved", 1 << 29, 1), ("4GiB_moved", 1 << 31, 1)):
        srcs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nrot)]
        dsts = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nrot)]
        for t in srcs:
            t.random_(0, 255, generator=g)
        n = max(4 * nrot, 8)
        ms = time_graph(lambda i: B.probe_copy(srcs[i % nrot], dsts[i % nrot]), n, reps)
        res["copy"][label] = dict(bytes_moved=2 * nbytes, us=round(ms * 1e3, 2),
                                  gbs=round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                                  frac_of_8TBs=round(2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
        del srcs, dsts
        torch.cuda.synchronize()
    nwg, iters = 2 * 256, 40000
    out = torch.empty(nwg * 256, dtype=torch.float32, device=dev)
    flop = nwg * 4.0 * iters * 4 * 32768
    for label, vary in (("fixed_operands", 0), ("changing_operands", 1)):
        ms = time_graph(lambda i: B.probe_mfma(out, nwg, iters, vary), 2, reps)
        tfl = flop / (ms * 1e-3) / 1e12
        res["mfma"][label] = dict(tflops=round(tfl, 1), frac=round(tfl / BF16_PEAK_TFLOPS, 4),
                                  ms=round(ms, 3))
    res["mfma"]["shape"] = (f"{nwg} workgroups x 4 waves x {iters} x 4 v_mfma_f32_32x32x16_bf16, "
                            "4 independent accumulators per wave (2 waves per SIMD)")
    return res


def library_gemm_times(g, dev, reps=3):
    """The vendor library on the same GEMM shapes, for comparison only:
    torch.matmul (hipBLASLt) of u [S, d] by W1^T and of the concat buffer
    [S, N2] by W2^T, bf16 in and out, no epilogue, captured in a graph and
    replayed.  "tn": the weight stored [out, in] as the block's kernels take
    it (both operands K-contiguous; the right operand is a transposed view of
    a 2-D weight, a plain matrix product); "nn": the weight made contiguous
    as [in, out] first, a different problem for the library."""
    import torch
    res = {}
    for name, (m, k, n, flop) in (("linear1", (S, D, N1, GEMM1_FLOP)), ("linear2", (S, N2, D, GEMM2_FLOP))):
        a = (torch.randn(m, k, generator=g, device=dev)).to(torch.bfloat16)
        w = (torch.randn(n, k, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        for layout, rhs in (("tn", w.t()), ("nn", w.t().contiguous())):
            ms = time_graph(lambda i: torch.matmul(a, rhs, out=out), 4, reps)
            tfl = flop / (ms * 1e-3) / 1e12
            res[f"{name}_{layout}"] = dict(us=round(ms * 1e3, 1), tflops=round(tfl, 1),
                                           frac=round(tfl / BF16_PEAK_TFLOPS, 4))
            del rhs
        del a, w, out
    torch.cuda.synchronize()
    return res


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return model, avail


def trace_summary(path, n_blocks=57):
    """Kernels per step and per block and the gaps between consecutive
    kernels inside each replayed step of the 57-block stack, from a
    rocprofv3 kernel trace (CSV).  A step starts at each launch of the
    batched modulation kernel and holds the launches up to the next one that
    is not a block kernel (copies, probes, other legs)."""
    import csv
    import glob
    if os.path.isdir(path):
        cands = sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
        if not cands:
            raise SystemExit(f"no *kernel_trace.csv under {path}")
        path = cands[0]
    with open(path) as f:
        rows = list(csv.DictReader(f))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    block_kernels = ("gemm_bf16_tn_kernel", "gemm4w_kernel", "attention_fwd_kernel", "attention_mod_kernel", "ln_modulate_kernel",
                     "qk_rmsnorm_rope_kernel", "mod_gemv")
    is_block = lambda name: any(k in name for k in block_kernels)
    steps = []
    i = 0
    while i < len(rows):
        if "mod_gemv_multi_kernel" in rows[i]["Kernel_Name"]:
            j = i + 1
            while j < len(rows) and is_block(rows[j]["Kernel_Name"]) and \
                    "mod_gemv_multi_kernel" not in rows[j]["Kernel_Name"]:
                j += 1
            steps.append(rows[i:j])
            i = j
        else:
            i += 1
    # only the plain (unprobed) single-stream replays: a probed step
    # interleaves stamp kernels, a mixed stack has two block kinds
    want = [st for st in steps if (len(st) - 1) % n_blocks == 0 and 1 <= (len(st) - 1) // n_blocks <= 8
            and all("EpiGated" not in r["Kernel_Name"] for r in st)]
    if not want:
        raise SystemExit("no replayed step of the stack found in the trace")
    out = []
    for st in want:
        t0, t1 = int(st[0]["Start_Timestamp"]), int(st[-1]["End_Timestamp"])
        gaps = [int(b["Start_Timestamp"]) - int(a["End_Timestamp"]) for a, b in zip(st, st[1:])]
        busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in st)
        out.append(dict(kernels=len(st), kernels_per_block=(len(st) - 1) / n_blocks, span_us=(t1 - t0) / 1e3,
                        busy_us=busy / 1e3, gap_us=sum(gaps) / 1e3, max_gap_us=max(gaps) / 1e3,
                        mean_gap_us=sum(gaps) / len(gaps) / 1e3, negative_gaps=sum(1 for x in gaps if x < 0)))
    # mean duration of each kernel inside the replayed steps (block kernels
    # by name; the batched modulation once per step)
    per_kernel = {}
    for st in want:
        for r in st:
            nm = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("dit::", "")
            per_kernel.setdefault(nm, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    kernel_means = {k: dict(calls=len(v), mean_us=round(sum(v) / len(v) / 1e3, 2)) for k, v in per_kernel.items()}
    agg = dict(source=os.path.relpath(path), steps=len(out), kernels_per_step=out[0]["kernels"],
               kernels_per_block=out[0]["kernels_per_block"],
               span_us_mean=round(sum(o["span_us"] for o in out) / len(out), 1),
               gap_us_per_step_mean=round(sum(o["gap_us"] for o in out) / len(out), 1),
               mean_gap_us=round(sum(o["mean_gap_us"] for o in out) / len(out), 3),
               max_gap_us=round(max(o["max_gap_us"] for o in out), 3),
               gap_frac=round(sum(o["gap_us"] for o in out) / sum(o["span_us"] for o in out), 5),
               kernel_means=kernel_means,
               per_step=[{k: (round(v, 3) if isinstance(v, float) else v) for k, v in o.items()} for o in out])
    return agg


def cpu_oracle_per_config():
    """The oracle's time per workload on the host cores: the tiny block and
    the chain ops in full, the video block on two sampled query-row counts
    (every key and value computed) extrapolated linearly to all rows, and
    the 57 x 50 stack extrapolated from the Flux block (labelled)."""
    import numpy as np
    import dit_inputs as DI
    from oracle import dit_oracle as O
    res = {}

    def timed(fn, reps=1):
        best = None
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        return best

    sh = DI.TINY
    w = DI.block_weights(sh)
    x, temb = DI.block_activations(sh)
    pos = DI.positions(sh)
    res["tiny_block_ms"] = round(1e3 * timed(lambda: O.block_forward(sh, w, x, temb, pos), 3), 2)
    ch = DI.chain_inputs()
    res["chain_modulate_norm_ms"] = round(1e3 * timed(
        lambda: O.layer_norm_modulate(ch["x"], ch["shift"], ch["scale"], 1e-6), 2), 1)
    res["chain_gated_residual_ms"] = round(1e3 * timed(lambda: O.gated_residual(ch["x"], ch["gate"], ch["h"]), 2), 1)
    sh = DI.VIDEO
    w = DI.block_weights(sh)
    x, temb = DI.block_activations(sh)
    pos = DI.positions(sh)
    pts = {}
    for r in (256, 1024):
        rows = np.arange(0, sh.seq_len, sh.seq_len // r)[:r]
        pts[r] = timed(lambda: O.block_forward(sh, w, x, temb, pos, rows=rows))
    slope = (pts[1024] - pts[256]) / (1024 - 256)
    res["video_block"] = dict(ms_256_rows=round(pts[256] * 1e3, 1), ms_1024_rows=round(pts[1024] * 1e3, 1),
                              ms_all_rows_extrapolated=round((pts[1024] + slope * (sh.seq_len - 1024)) * 1e3, 1),
                              note="linear in the number of query rows; K and V always cover all 16384 tokens")
    return res


def kernel_phase(B, g, dev, blocks, x_in, temb, rc, rs, it, only=None):
    """Block-sequence times of the six block kernels plus the HBM-rate loops."""
    seq_names = ("modulation", "block_modulate_norm", "linear1_gelu", "qk_rmsnorm_rope", "attention",
                 "linear2_gated_residual")
    k = {}
    if only is None or any(n in only for n in seq_names):
        k = block_sequence_times(B, blocks, x_in, temb, rc, rs, it, only)
    k2, warm = hbm_kernel_times(B, g, dev, it, only)
    k.update(k2)
    if only is not None and "block_forward" in only:
        # whole eager block forwards: the kernels as the stack launches them
        # (at this shape linear1 carries the q/k RMSNorm + RoPE epilogue)
        import torch
        cfg = B.make_config(S, D, H, DH, MLP)
        ws = B.alloc_workspace(B.block_workspace_bytes(cfg))
        y = torch.empty_like(x_in)
        k["block_forward"] = time_launches(
            lambda i: B.block_forward(cfg, blocks[i % len(blocks)], x_in, temb[0], rc, rs, y=y, workspace=ws), it)
    for name, ms in k.items():
        log(f"kernel {name}: {ms * 1000:.1f} us")
    return k, warm


def cpu_baseline():
    """The oracle (numpy float64) on one full Flux-shape block on the host cores."""
    import numpy as np
    import dit_inputs as DI
    from oracle import dit_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    model, avail = host_cpu()
    shape = DI.FLUX
    w = DI.block_weights(shape)
    x, temb = DI.block_activations(shape)
    pos = DI.positions(shape)
    t0 = time.perf_counter()
    y = O.block_forward(shape, w, x, temb, pos)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(y))
    return dict(value=round(dt * 1000.0, 1), unit="ms per block", cores=int(threads), kind="oracle",
                sample="one full Flux-shape block forward (S=4608, d=3072, 24x128, MLP 12288) "
                       "in numpy float64, BLAS threads = cores; 1 of the 57 blocks of a step",
                cpu_model=model, cpus_available=avail,
                stack_57x50_extrapolated_s=round(dt * 57 * 50, 1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--blocks", type=int, default=57)
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-summary", default=None,
                    help="summarise a rocprofv3 kernel trace (CSV file or output folder) of a bench run: kernels "
                         "per block and launch gaps inside the replayed steps; prints JSON and exits")
    ap.add_argument("--kernels-only", default=None,
                    help="comma list of kernels (%s): time only these, no stack replay (for profiler runs)"
                         % ",".join(KERNEL_NAMES))
    args = ap.parse_args()
    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary, args.blocks)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the block's multi-GPU sharding is a design, not built)", file=sys.stderr)
        return 2

    import torch
    from diffusion_transformer_dit_amd import binding as B
    import dit_inputs as DI

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3000)

    def randn(shape, sigma):
        return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * sigma).to(torch.bfloat16)

    if args.kernels_only:
        only = set(args.kernels_only.split(","))
        bad = only - set(KERNEL_NAMES)
        if bad:
            print(f"unknown kernels: {sorted(bad)}", file=sys.stderr)
            return 2
        nb = 2
        blocks = [B.BlockWeights(randn((3 * D, D), 0.02), randn((3 * D,), 0.02), randn((N1, D), 0.02),
                                 randn((N1,), 0.02), randn((D, N2), 0.02), randn((D,), 0.02),
                                 torch.ones(DH, device=dev), torch.ones(DH, device=dev)) for _ in range(nb)]
        x_in = randn((S, D), 1.0)
        temb = randn((1, D), 1.0)
        pos = torch.from_numpy(DI.positions(DI.FLUX)).to(dev)
        rc, rs = B.rope_table(pos, list(DI.FLUX.rope_axes_dims), DH)
        k, _ = kernel_phase(B, g, dev, blocks, x_in, temb, rc, rs, args.kernel_iters, only)
        out = {"kernels_us": {n: round(v * 1e3, 2) for n, v in k.items()}}
        if "other_blocks" in only:
            out["other_blocks"] = other_block_times(B, g, dev)
        if "config_blocks" in only:
            out["config_blocks"] = config_block_times(B, g, dev)
        if "ceilings" in only:
            out["ceilings"] = ceiling_times(B, g, dev)
            out["ceilings"]["library_gemm"] = library_gemm_times(g, dev)
        print(json.dumps(out), flush=True)
        return 0

    nb = args.blocks
    log(f"allocating {nb} Flux blocks ({nb * (3 * D * D + N1 * D + D * N2) * 2 / 1e9:.1f} GB of weights)")
    blocks = []
    for b in range(nb):
        blocks.append(B.BlockWeights(randn((3 * D, D), 0.02), randn((3 * D,), 0.02), randn((N1, D), 0.02),
                                     randn((N1,), 0.02), randn((D, N2), 0.02), randn((D,), 0.02),
                                     torch.ones(DH, device=dev), torch.ones(DH, device=dev)))
    x_in = randn((S, D), 1.0)
    n_total = args.warmup + args.steps
    temb = randn((max(n_total, 1), D), 1.0)
    pos = torch.from_numpy(DI.positions(DI.FLUX)).to(dev)
    rc, rs = B.rope_table(pos, list(DI.FLUX.rope_axes_dims), DH)
    cfg = B.make_config(S, D, H, DH, MLP)
    ws = B.alloc_workspace(B.stack_workspace_bytes(cfg, nb))
    out = torch.empty(max(n_total, 1), S, D, dtype=torch.bfloat16, device=dev)
    st = B.Stack()
    torch.cuda.synchronize()

    # ---- warmup (the first replay captures the graph)
    if args.warmup:
        st.replay(cfg, blocks, x_in, temb[:args.warmup], rc, rs, out[:args.warmup], ws)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # ---- timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    st.replay(cfg, blocks, x_in, temb[args.warmup:n_total], rc, rs, out[args.warmup:n_total], ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / max(args.steps, 1)
    ms_block = ms_step / nb
    assert torch.isfinite(out[args.warmup:n_total].float()).all(), "non-finite output"
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step, {ms_block:.4f} ms/block (wall {wall:.3f} s)")

    # ---- the same timed steps on a second stack whose graph brackets every
    # kernel of every block with wall-clock stamps: per-kernel durations inside
    # the replay, as the kernels run there
    stp = B.Stack()
    stp.set_probe(B.Stack.KERNELS)
    wsp = B.alloc_workspace(B.stack_workspace_bytes(cfg, nb))
    stp.replay(cfg, blocks, x_in, temb[:max(args.warmup, 1)], rc, rs, out[:max(args.warmup, 1)], wsp)
    stp.probe_ms(nb)  # discards the warmup steps
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    stp.replay(cfg, blocks, x_in, temb[args.warmup:n_total], rc, rs, out[args.warmup:n_total], wsp)
    p1.record()
    torch.cuda.synchronize()
    ms_step_probed = p0.elapsed_time(p1) / max(args.steps, 1)
    pm = stp.probe_ms(nb)
    stp.close()
    names = {"modulation": "modulation", "modulate_norm": "block_modulate_norm", "linear1": "linear1_gelu",
             "qk_rmsnorm_rope": "qk_rmsnorm_rope", "attention": "attention", "linear2": "linear2_gated_residual"}
    k = {names[n]: sum(v) / len(v) for n, v in pm.items()}
    # the step's modulation launch is bracketed by block 0's first probe; it
    # covers block 0 only (blocks 1-56 get theirs from the previous block's
    # attention launch, in the CUs its last round leaves idle)
    k["modulation"] = pm["modulation"][0]
    log(f"probed replay: {ms_step_probed:.3f} ms/step; in-graph kernel means over {nb} blocks x {args.steps} steps: "
        + ", ".join(f"{n} {v * 1e3:.1f} us" for n, v in k.items()))
    k2, k_warm_norm = hbm_kernel_times(B, g, dev, args.kernel_iters)
    k.update(k2)
    tf = lambda flop, ms: flop / (ms * 1e-3) / 1e12
    gbs = lambda byt, ms: byt / (ms * 1e-3) / 1e9
    kernels = {
        "linear1_gelu": dict(us=k["linear1_gelu"] * 1e3, tflops=tf(GEMM1_FLOP, k["linear1_gelu"]),
                             frac=tf(GEMM1_FLOP, k["linear1_gelu"]) / BF16_PEAK_TFLOPS),
        "linear2_gated_residual": dict(us=k["linear2_gated_residual"] * 1e3,
                                       tflops=tf(GEMM2_FLOP, k["linear2_gated_residual"]),
                                       frac=tf(GEMM2_FLOP, k["linear2_gated_residual"]) / BF16_PEAK_TFLOPS),
        "attention": dict(us=k["attention"] * 1e3, tflops=tf(ATTN_FLOP, k["attention"]),
                          frac=tf(ATTN_FLOP, k["attention"]) / BF16_PEAK_TFLOPS),
        "modulate_norm": dict(us=k["modulate_norm"] * 1e3, gbs=gbs(NORM_BYTES, k["modulate_norm"]),
                              frac=gbs(NORM_BYTES, k["modulate_norm"]) / HBM_PEAK_GBS,
                              cache_warm_gbs=gbs(NORM_BYTES, k_warm_norm)),
        "gated_residual": dict(us=k["gated_residual"] * 1e3, gbs=gbs(GRES_BYTES, k["gated_residual"]),
                               frac=gbs(GRES_BYTES, k["gated_residual"]) / HBM_PEAK_GBS),
        "qk_rmsnorm_rope": dict(us=k["qk_rmsnorm_rope_standalone"] * 1e3,
                                gbs=gbs(QKNORM_BYTES, k["qk_rmsnorm_rope_standalone"]),
                                frac=gbs(QKNORM_BYTES, k["qk_rmsnorm_rope_standalone"]) / HBM_PEAK_GBS,
                                in_graph_us=k["qk_rmsnorm_rope"] * 1e3),
        "modulation": dict(us=k["modulation"] * 1e3, gbs=gbs(MOD_BYTES, k["modulation"]),
                           frac=gbs(MOD_BYTES, k["modulation"]) / HBM_PEAK_GBS,
                           blocks_in_attention_launches=nb - 1),
        "block_modulate_norm": dict(us=k["block_modulate_norm"] * 1e3,
                                    gbs=gbs(NORM_BYTES, k["block_modulate_norm"])),
    }
    for v in kernels.values():
        for kk in list(v):
            v[kk] = round(v[kk], 4 if kk == "frac" else 2)

    g1 = tf(GEMM1_FLOP, k["linear1_gelu"])
    traffic = load_traffic()
    result = {
        "metric": METRIC,
        "value": round(ms_block, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, x and temb ~ N(0,1); no trained weights)",
        "config": {"workload": "flux_single_stream_block_stack", "seq_len": S, "dim": D, "num_heads": H,
                   "head_dim": DH, "mlp_hidden": MLP, "blocks": nb, "rope": "2d (64 row | 64 col dims)",
                   "replay": "one hipGraph of the whole stack per denoising step"},
        "block_tflops": round(BLOCK_FLOP / (ms_block * 1e-3) / 1e12, 1),
        "fused_norm_gbs": kernels["modulate_norm"]["gbs"],
        "fused_norm_frac": kernels["modulate_norm"]["frac"],
        "roofline": {"bound": "mfma", "kernel": ("linear1_gelu (GEMM1 + bias + GELU epilogue; q/k RMSNorm + RoPE "
                                                 "fused into the epilogue)"),
                     "achieved": round(g1, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g1 / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "flop_per_launch": GEMM1_FLOP},
        "kernels": kernels,
        "launch_gaps": load_launch_gaps(),
        "ms_per_step_probed": round(ms_step_probed, 3),
        "timing_note": ("per-kernel times: device wall-clock stamps captured around every kernel of every "
                        "block in a second replay of the same timed steps (ms_per_step_probed), stamp overhead "
                        "subtracted, mean over 57 blocks x steps; modulation: block 0's GEMV, launched at the "
                        "start of the step (blocks 1-56 compute theirs inside the previous block's attention "
                        "launch, whose time includes it); modulate_norm and gated_residual HBM rates: "
                        "12 rotating buffer sets at the chain shape"),
        "context": {"pages_h20_ms_per_57_block_forward_eager": 762.7,
                    "pages_h20_ms_per_57_block_forward_compiled": 637.8,
                    "this_ms_per_57_block_step": round(ms_block * 57, 2),
                    "note": "H20 figures cover 19 double- and 38 single-stream Flux blocks; context only"},
    }
    ca = chunked_attention_times(B, g, dev)
    merge_bytes = ca["chunks"] * (S * D * 4 + H * S * 4) + S * D * 2
    result["chunked_attention"] = {
        "workload": "Flux attention (S=4608, 24x128) as 8 key chunks of 576 merged by log-sum-exp",
        "partials_us": round(ca["partials_ms"] * 1e3, 1),
        "partials_tflops": round(tf(ATTN_FLOP, ca["partials_ms"]), 1),
        "merge_us": round(ca["merge_ms"] * 1e3, 1),
        "merge_gbs": round(gbs(merge_bytes, ca["merge_ms"]), 1),
        "single_pass_us": round(ca["single_pass_ms"] * 1e3, 1),
        "ulysses_share_3_heads_us": round(ca["ulysses_share_3heads_ms"] * 1e3, 1),
        "ulysses_share_3_heads_split_us": {f"{n}_chunks": round(v * 1e3, 1)
                                           for n, v in ca["ulysses_share_3heads_split_ms"].items()},
        "note": "outside the graph of the stack; partials write fp32 outputs that the merge reads back",
    }
    log(f"chunked attention: 8 partials {ca['partials_ms'] * 1e3:.1f} us + merge {ca['merge_ms'] * 1e3:.1f} us, "
        f"single pass {ca['single_pass_ms'] * 1e3:.1f} us, 3-head share {ca['ulysses_share_3heads_ms'] * 1e3:.1f} us, "
        "split " + ", ".join(f"{n}: {v * 1e3:.1f} us" for n, v in ca["ulysses_share_3heads_split_ms"].items()))
    # ---- step-level skip (MeanCache-style control): 50 denoising steps with
    # steps 0, 1 and every even step after computed (26 forwards), the others
    # predicted from the last two computed outputs, against all 50 computed
    n50 = 50
    fresh = [1 if (s_ < 2 or s_ % 2 == 0) else 0 for s_ in range(n50)]
    temb50 = randn((n50, D), 1.0)
    out50 = torch.empty(n50, S, D, dtype=torch.bfloat16, device=dev)
    tsteps = [1.0 - s_ / n50 for s_ in range(n50)]
    c0, c1, c2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    c0.record()
    st.replay(cfg, blocks, x_in, temb50, rc, rs, out50, ws)
    c1.record()
    st.replay_cached(cfg, blocks, x_in, temb50, rc, rs, out50, ws, fresh, tsteps)
    c2.record()
    torch.cuda.synchronize()
    ms_all, ms_cached = c0.elapsed_time(c1), c1.elapsed_time(c2)
    result["step_skip"] = {
        "workload": "57-block Flux stack, 50 denoising steps",
        "schedule": "steps 0, 1 and every even step computed (26 of 50); skipped steps predicted by the "
                    "first-order finite difference in t through the last two computed outputs",
        "forwards": sum(fresh), "ms_50_steps_all_computed": round(ms_all, 2),
        "ms_50_steps_cached": round(ms_cached, 2), "speedup": round(ms_all / ms_cached, 3),
    }
    log(f"step skip: 50 steps {ms_all:.1f} ms all computed, {ms_cached:.1f} ms with {sum(fresh)} computed")
    del out50
    # ---- the Flux composition: 19 two-stream blocks then 38 single-stream
    # blocks in one captured graph (the 57 blocks of the pages' forward)
    import dit_inputs as DI
    nd_, ns_ = 19, 38
    one = torch.ones(DH, device=dev)
    sw = lambda: B.StreamWeights(randn((6 * D, D), 0.02), randn((6 * D,), 0.02), randn((3 * D, D), 0.02),
                                 randn((3 * D,), 0.02), one, one, randn((D, D), 0.02), randn((D,), 0.02),
                                 randn((MLP, D), 0.02), randn((MLP,), 0.02), randn((D, MLP), 0.02), randn((D,), 0.02))
    fdoubles = [(sw(), sw()) for _ in range(nd_)]
    fsingles = blocks[:ns_]
    wsf = B.alloc_workspace(B.stack_mixed_workspace_bytes(cfg, DI.FLUX.text_tokens, nd_, ns_))
    outf = torch.empty(4, S, D, dtype=torch.bfloat16, device=dev)
    stf = B.Stack()
    stf.replay_mixed(cfg, DI.FLUX.text_tokens, fdoubles, fsingles, x_in, temb[:1], rc, rs, outf[:1], wsf)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    stf.replay_mixed(cfg, DI.FLUX.text_tokens, fdoubles, fsingles, x_in, temb50[:3], rc, rs, outf[1:4], wsf)
    f1.record()
    torch.cuda.synchronize()
    ms_flux = f0.elapsed_time(f1) / 3
    stf.close()
    result["flux_forward"] = {
        "workload": "Flux transformer blocks: 19 two-stream (512 text + 4096 image tokens) + 38 single-stream, "
                    "S=4608, d=3072, one captured graph per denoising step",
        "ms_per_step": round(ms_flux, 2),
        "pages_h20_ms_per_forward_eager": 762.7, "pages_h20_ms_per_forward_compiled": 637.8,
        "note": "context only: the pages' figures are another machine's whole transformer forward",
    }
    log(f"flux forward (19 two-stream + 38 single-stream blocks): {ms_flux:.2f} ms per step")
    del fdoubles, wsf, outf, temb50
    ob = other_block_times(B, g, dev)
    for v in ob.values():
        v["note"] = "one block forward captured in a graph and replayed (same weights each replay)"
    result["other_blocks"] = ob
    log("other blocks: " + ", ".join(f"{n} {v['ms']:.3f} ms ({v['tflops']} TFLOP/s)" for n, v in ob.items()))
    cb = config_block_times(B, g, dev)
    cb["note"] = "single-stream block forward captured in a graph and replayed; frac of 2.5 PFLOP/s"
    result["config_blocks"] = cb
    log("config blocks: " + ", ".join(f"{n} {v['ms']:.4f} ms ({v['tflops']} TFLOP/s)"
                                      for n, v in cb.items() if isinstance(v, dict)))
    ce = ceiling_times(B, g, dev)
    lg = library_gemm_times(g, dev)
    ce["library_gemm"] = lg
    ce["library_gemm"]["note"] = ("torch.matmul (hipBLASLt) on the same shapes without epilogues, graph-timed "
                                  "outside the stack; comparison only")
    result["ceilings"] = ce
    cpy_n, cpy_g = ce["copy"]["56.6MB_moved"]["gbs"], ce["copy"]["84.9MB_moved"]["gbs"]
    kernels["modulate_norm"]["frac_of_copy_same_size"] = round(kernels["modulate_norm"]["gbs"] / cpy_n, 4)
    kernels["gated_residual"]["frac_of_copy_same_size"] = round(kernels["gated_residual"]["gbs"] / cpy_g, 4)
    kernels["modulate_norm"]["frac_of_copy_4GiB"] = round(kernels["modulate_norm"]["gbs"] /
                                                          ce["copy"]["4GiB_moved"]["gbs"], 4)
    kernels["gated_residual"]["frac_of_copy_4GiB"] = round(kernels["gated_residual"]["gbs"] /
                                                           ce["copy"]["4GiB_moved"]["gbs"], 4)
    log("ceilings: copy " + ", ".join(f"{n} {v['gbs']} GB/s" for n, v in ce["copy"].items()) + "; mfma "
        + ", ".join(f"{n} {v['tflops']} TFLOP/s" for n, v in ce["mfma"].items() if isinstance(v, dict))
        + "; library gemm " + ", ".join(f"{n} {v['us']} us" for n, v in lg.items() if isinstance(v, dict)))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one Flux block ...")
        result["cpu_baseline"] = cpu_baseline()
        log(f"cpu oracle: {result['cpu_baseline']['value']} ms/block on {result['cpu_baseline']['cores']} threads")
        log("timing the CPU oracle on the other workloads ...")
        result["cpu_oracle_per_config"] = cpu_oracle_per_config()
        log(f"cpu oracle per config: {result['cpu_oracle_per_config']}")
    st.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
