"""Throughput of the tiled ViT tower on one MI355X.

A step is one forward pass of the whole path -- patchify + patch embed, the
32 blocks (LayerNorm, QKV, tiled RoPE attention, O, LayerNorm, MLP), the
raster-order tower output, the 2x2 merge and the projector -- over one batch
of synthetic input that is already resident in device memory.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload tower_448]
    python bench.py --kernel {fc1,resid_gemm,attention,attention_bwd,block_bwd,copy} [--workload ...]   # one case

Prints one JSON line.  Beside the headline workload it times, with HIP events
on the stream the kernels run on (the kernel rooflines: a loop of launches
captured into one HIP graph and replayed, so that no host time between
launches enters a kernel's average duration):
  roofline           the dominant kernel of the headline workload at 1,024
                     tokens: the split-K partial GEMM of the O and FC2
                     residual Linears (vt_linear with the partials epilogue,
                     the kernel the blocks launch), and the same Linears with
                     their fused split-K reduce + LayerNorm
                     (vt_linear_residual_ln);
  fc1_roofline       the FC1 GEMM (bias + GELU epilogue);
  attention_roofline the attention kernels as the tower runs them
                     (vt_attention_packed), beside one whole
                     vt_attention_varlen call;
one vt_attention_backward and one vt_block_backward call, the 2016x2016
single image as a secondary workload, and further workloads (224x224 one
block, clips, 16 x 448x448 with its own attention and GEMM rooflines, mixed
grids, 4096x4096).  "traffic" (HBM-side bytes per launch) comes from the
FETCH_SIZE / WRITE_SIZE counter summaries under profiles/, and is null when
those were taken on other kernel sources.  The CPU oracle is timed on a
bounded sample (one 448x448 image through the full tower) on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA, 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
CUS, BF16_FLOP_PER_CLK_CU = 256, 4096


def gemm_flops_per_token(d=1280, mlp=5120, P=6144):
    """Algorithmic GEMM FLOPs per token for one block and for the projector."""
    block = 2 * (3 * d * d + d * d + 2 * d * mlp)
    proj = 2 * (d * P + P * P) + 2 * (4 * P * P + P * P) / 4
    return block, proj


def workload_flops(wl):
    N = wl.tokens
    block, proj = gemm_flops_per_token()
    gemm = N * (2 * 1176 * 1280 + wl.layers * block + (proj if wl.projector else 0))
    attn = wl.layers * sum(4 * (t * h * w) ** 2 * 1280 for t, h, w in wl.grids)
    return gemm, attn


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="tower_448", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--secondary", default="tower_2016", help="second workload ('' to skip)")
    ap.add_argument("--more", default="block_224,tower_clip16,tower_448x16,tower_mixed8,tower_4096",
                    help="comma-separated further workloads, throughput only ('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass lines (forward-only kernel profiles)")
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--kernel", choices=["fc1", "resid_gemm", "attention", "attention_bwd", "block_bwd", "copy"],
                    default=None,
                    help="run only this kernel case (counter runs) and exit")
    return ap.parse_args()


class Runner:
    def __init__(self, vt, torch, tw, wl):
        self.vt, self.torch, self.tw, self.wl = vt, torch, tw, wl
        self.grids = list(wl.grids)
        self.cfg = vt.config(layers=wl.layers)
        N = wl.tokens
        self.px = torch.from_numpy(synth.make_batch_pixels(wl).view(np.int16)).cuda()
        self.ws = vt.workspace(vt.vt_tower_workspace_size(self.cfg, self.grids))
        self.tower = torch.empty((N, 1280), dtype=torch.int16, device="cuda")
        self.out = (torch.empty((N // 4, 6144), dtype=torch.int16, device="cuda")
                    if wl.projector else None)

    def step(self):
        self.vt.vt_tower_forward(self.cfg, self.px, self.grids, self.tw, self.tower, None,
                                 self.out, self.ws)

    def time(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record()
        for _ in range(steps):
            self.step()
        e.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return s.elapsed_time(e) / 1e3, wall


def time_kernel(torch, fn, iters):
    """Average duration of one launch sequence of ``fn`` with HIP events
    recorded on the current stream, the stream the library launches on.
    Three untimed launches are queued just before the start event, so the
    GPU is already busy when it is recorded and the host's time to issue
    the first timed launches is not counted as kernel time."""
    fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        fn()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / iters


def time_graph(torch, fn, iters):
    """Average duration of one launch sequence of ``fn``: ``iters`` calls
    captured into one HIP graph (the library only enqueues kernels on the
    caller's stream, so its calls capture), the graph replayed once untimed
    and once between HIP events on the current stream.  Unlike the eager
    loop of time_kernel, no host time between launches can leave the GPU
    idle, which matters for kernels of ~10 us against ~8 us of host time per
    call from Python."""
    fn()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(iters):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) / 1e3 / iters


def clock_under(vt, torch, fn, iters, t_each):
    """Core clock (GHz) while ``fn`` runs: the loop of ``iters`` launches
    again, with vt_clock_probe on a second (default-priority) stream, started
    once a few launches are queued and timing ~80% of the rest."""
    side = torch.cuda.Stream()
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    pre = max(1, min(5, iters // 10))
    wait_us = max(100, int(0.8 * (iters - pre) * t_each * 1e6))
    torch.cuda.synchronize()
    for _ in range(pre):
        fn()
    hz = vt.vt_clock_probe(wait_us, out, stream=side.cuda_stream)
    for _ in range(iters - pre):
        fn()
    torch.cuda.synchronize()
    c0, c1, r0, r1 = out.cpu().tolist()
    return (c1 - c0) / (r1 - r0) * hz / 1e9


def at_clock(achieved_tflops, ghz):
    """The bf16 dense peak at the measured clock, and the fraction of it."""
    peak = CUS * BF16_FLOP_PER_CLK_CU * ghz * 1e9 / 1e12
    return {"clock_ghz": ghz, "peak_at_clock": peak, "frac_at_clock": achieved_tflops / peak}


COLD_BYTES = 320 << 20   # more than the 256 MB memory-side cache


def weight_copies(torch, w):
    """Distinct copies of a weight tensor totalling more than the memory-side
    cache, so that a loop that cycles through them reads every weight from
    HBM, as the tower does (each layer's weights are used once per step); the
    activations stay shared and cache-hot, as in the tower."""
    n = max(2, -(-COLD_BYTES // (w.numel() * w.element_size())))
    return [w.clone() for _ in range(n)]


def cycled(fns):
    """One call of the next function of the list per call (round robin)."""
    state = [0]

    def call():
        fns[state[0] % len(fns)]()
        state[0] += 1
    return call


def fc1_case(vt, torch, M):
    """The FC1 GEMM of one block (M x 5120 x 1280, bias + GELU epilogue) as a
    vt_linear call on seeded bf16 operands, cycling through cold weight copies."""
    N, K = 5120, 1280
    g = np.random.Generator(np.random.PCG64(0))
    x = torch.from_numpy(synth.bf16_bits(g.standard_normal((M, K), dtype=np.float32)).view(np.int16)).cuda()
    w = torch.from_numpy(synth.bf16_bits(g.standard_normal((N, K), dtype=np.float32) * 0.02).view(np.int16)).cuda()
    b = torch.zeros(N, dtype=torch.int16, device="cuda")
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = vt.workspace(vt.vt_linear_workspace_size(M, N, K))
    fns = [lambda wc=wc: vt.vt_linear(x, M, K, wc, N, b, vt.VT_EPI_GELU_TANH_BF16, out, ws)
           for wc in weight_copies(torch, w)]
    return cycled(fns), 2.0 * M * N * K


def residual_cases(vt, torch, M):
    """The O (M x 1280 x 1280) and FC2 (M x 1280 x 5120) residual Linears of a
    block on seeded bf16 operands, each call on the next of its cold weight
    copies (weight_copies): per shape, (the GEMM kernel alone -- the
    split-K partial products when the shape splits K, else the GEMM with its
    residual epilogue --, the whole residual step with its reduce +
    LayerNorm, FLOPs, splits)."""
    g = np.random.Generator(np.random.PCG64(4))
    bits = lambda shape, sc=1.0: torch.from_numpy(
        synth.bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(sc)).view(np.int16)).cuda()
    N = 1280
    R = torch.from_numpy(g.standard_normal((M, N), dtype=np.float32)).cuda()
    gam = torch.from_numpy(synth.bf16_bits(np.ones(N, np.float32)).view(np.int16)).cuda()
    bet = torch.zeros(N, dtype=torch.int16, device="cuda")
    ln = torch.empty((M, N), dtype=torch.int16, device="cuda")
    out = []
    for K in (1280, 5120):
        x, w, b = bits((M, K)), bits((N, K), 0.02), torch.zeros(N, dtype=torch.int16, device="cuda")
        ws_copies = weight_copies(torch, w)
        nws = vt.vt_linear_workspace_size(M, N, K)
        ws = vt.workspace(nws)
        splits = nws // (M * N * 4) if nws else 1
        if splits > 1:
            part = torch.empty(nws // 4, dtype=torch.float32, device="cuda")
            gemm = cycled([lambda x=x, w=wc, K=K, part=part:
                           vt.vt_linear(x, M, K, w, N, None, vt.VT_EPI_SPLITK_PARTIALS_F32, part)
                           for wc in ws_copies])
        else:
            gemm = cycled([lambda x=x, w=wc, K=K, b=b, ws=ws: vt.vt_linear(x, M, K, w, N, b, vt.VT_EPI_RESID_F32, R, ws)
                           for wc in ws_copies])
        step = cycled([lambda x=x, w=wc, K=K, b=b, ws=ws:
                       vt.vt_linear_residual_ln(x, M, K, w, N, b, R, gam, bet, 1e-6, ln, ws)
                       for wc in ws_copies])
        out.append((gemm, step, 2.0 * M * N * K, splits))
    return out


def attention_case(vt, torch, grids):
    """vt_attention_varlen on the workload's token layout (random bf16 q, k, v)."""
    N = sum(t * h * w for t, h, w in grids)
    g = np.random.Generator(np.random.PCG64(1))
    qkv = torch.from_numpy(synth.bf16_bits(g.standard_normal((N, 3840), dtype=np.float32) * 0.7).view(np.int16)).cuda()
    cfg = vt.config()
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    max_seq = max(t * h * w for t, h, w in grids)
    ws = vt.workspace(vt.vt_block_workspace_size(cfg, N, len(grids), max_seq))
    out = torch.empty((N, 1280), dtype=torch.int16, device="cuda")
    flops = float(sum(4 * (t * h * w) ** 2 * 1280 for t, h, w in grids))
    return (lambda: vt.vt_attention_varlen(cfg, qkv, cu, pos, len(grids), N, max_seq, out, vt.VT_BF16, ws)), flops


def attention_packed_case(vt, torch, grids):
    """The attention kernels alone, as the tower runs them after its QKV
    Linear: vt_attention_pack once, then vt_attention_packed (timed) on what it
    left in the workspace."""
    N = sum(t * h * w for t, h, w in grids)
    g = np.random.Generator(np.random.PCG64(1))
    qkv = torch.from_numpy(synth.bf16_bits(g.standard_normal((N, 3840), dtype=np.float32) * 0.7).view(np.int16)).cuda()
    cfg = vt.config()
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    max_seq = max(t * h * w for t, h, w in grids)
    ws = vt.workspace(vt.vt_block_workspace_size(cfg, N, len(grids), max_seq))
    out = torch.empty((N, 1280), dtype=torch.int16, device="cuda")
    vt.vt_attention_pack(cfg, qkv, cu, pos, len(grids), N, max_seq, ws)
    lens = [t * h * w for t, h, w in grids]  # known to the caller, as to the tower
    return lambda: vt.vt_attention_packed(cfg, len(grids), N, max_seq, out, vt.VT_BF16, ws, host_seqlens=lens)


def attention_backward_case(vt, torch, grids):
    """vt_attention_backward on the workload's token layout (random bf16 q, k,
    v and dO).  FLOPs counted: the gradient's four n^2 products (dP = dO V^T,
    dV = P^T dO, dQ = dS K, dK = dS^T Q) per head; the call also recomputes
    the forward (S and P V) and S once more in each backward kernel."""
    N = sum(t * h * w for t, h, w in grids)
    g = np.random.Generator(np.random.PCG64(2))
    qkv = torch.from_numpy(synth.bf16_bits(g.standard_normal((N, 3840), dtype=np.float32) * 0.7).view(np.int16)).cuda()
    dout = torch.from_numpy(synth.bf16_bits(g.standard_normal((N, 1280), dtype=np.float32)).view(np.int16)).cuda()
    cfg = vt.config()
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    max_seq = max(t * h * w for t, h, w in grids)
    ws = vt.workspace(vt.vt_attention_backward_workspace_size(cfg, N, len(grids), max_seq))
    dqkv = torch.empty((N, 3840), dtype=torch.int16, device="cuda")
    flops = float(sum(8 * (t * h * w) ** 2 * 1280 for t, h, w in grids))
    return (lambda: vt.vt_attention_backward(cfg, qkv, cu, pos, len(grids), N, max_seq, dout, dqkv,
                                             vt.VT_BF16, ws)), flops


def block_backward_case(vt, torch, grids):
    """vt_block_backward of one block (random-init bf16 weights, a random fp32
    residual stream and dL/d(output), all gradients formed).  FLOPs counted:
    the block's forward (which the call recomputes) plus its backward -- three
    times the linear layers' products and 12 n^2 d for attention (forward
    S and P V, backward dP, dV, dQ, dK)."""
    N = sum(t * h * w for t, h, w in grids)
    W = synth.make_weights(1, projector=False)
    dev = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in W.items()}
    bw = vt.block_weights(dev, "l0.")
    g = np.random.Generator(np.random.PCG64(3))
    R = torch.from_numpy(g.standard_normal((N, 1280), dtype=np.float32)).cuda()
    dR0 = torch.from_numpy(g.standard_normal((N, 1280), dtype=np.float32)).cuda()
    dR = dR0.clone()
    grads = {k[3:]: torch.empty(v.shape, dtype=torch.float32, device="cuda")
             for k, v in W.items() if k.startswith("l0.")}
    gs = vt.block_grads(grads)
    cfg = vt.config(layers=1)
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    max_seq = max(t * h * w for t, h, w in grids)
    ws = vt.workspace(vt.vt_block_backward_workspace_size(cfg, N, len(grids), max_seq))
    block, _ = gemm_flops_per_token()
    flops = 3.0 * N * block + float(sum(12 * (t * h * w) ** 2 * 1280 for t, h, w in grids))
    # dR is overwritten with dL/d(input) each call; the work does not depend on its values
    return (lambda: vt.vt_block_backward(cfg, R, bw, cu, pos, len(grids), N, max_seq, dR, gs, ws)), flops


def tower_backward_case(vt, torch, wl, tw, W):
    """vt_tower_backward of the 32-layer tower on the workload's items, with
    dL/d(tower output) = 1/n per token (the mean-pool probe).  FLOPs counted:
    the tower's forward (patch embed + blocks) plus its backward (2x the block
    products, dW of the patch embed, 8 n^2 d attention per layer); the call
    also recomputes each block's forward."""
    N = wl.tokens
    px = torch.from_numpy(synth.make_batch_pixels(wl).view(np.int16)).cuda()
    grids = list(wl.grids)
    dT = torch.cat([torch.full((t * h * w, 1280), 1.0 / (t * h * w), device="cuda") for t, h, w in grids])
    grads = {k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in W.items()
             if not k.startswith("p_")}
    tg = vt.TowerGrads(grads, 32)
    cfg = vt.config()
    ws = vt.workspace(vt.vt_tower_backward_workspace_size(cfg, grids))
    block, _ = gemm_flops_per_token()
    flops = N * (2 * 2 * 1176 * 1280 + 32 * 3 * block) + 32 * float(
        sum(12 * (t * h * w) ** 2 * 1280 for t, h, w in grids))
    return (lambda: vt.vt_tower_backward(cfg, px, grids, tw, dT, tg, ws)), flops


def copy_case(torch, nbytes=256 << 20):
    """A plain device-to-device copy of nbytes (the HBM-counter calibration)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    return (lambda: dst.copy_(src)), 0.0


def profile_traffic(name, source):
    """HBM bytes per launch of a kernel from the counter summary in
    profiles/<name>.txt: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the
    kernel and of a plain copy of known size, each scaled by the copy's
    known bytes / its counter reading.  None if the summary is missing or
    was taken on other kernel sources (sha1 recorded in the summary)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "`")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha1(open(os.path.join(ROOT, source), "rb").read()).hexdigest()
    if kv.get("source_sha1") != sha:
        return None
    try:
        fr = float(kv["copy_known_read_bytes"]) / (float(kv["copy_fetch_kib"]) * 1024)
        fw = float(kv["copy_known_write_bytes"]) / (float(kv["copy_write_kib"]) * 1024)
        return float(kv["kernel_fetch_kib"]) * 1024 * fr + float(kv["kernel_write_kib"]) * 1024 * fw
    except (KeyError, ValueError):
        return None


def residual_gemm_roofline(vt, torch, M, iters):
    """The split-K partial GEMM of the O and FC2 residual Linears at M tokens
    (the kernel of the blocks with the largest share of the 448x448 step):
    achieved = (2 M N K of O + of FC2) / (the average launch time at the O
    shape + at the FC2 shape).  with_reduce_ln: the same FLOPs over the time
    of the whole residual step as the blocks run it, partials + the fused
    split-K reduce, residual update and LayerNorm."""
    cases = residual_cases(vt, torch, M)
    flops = sum(c[2] for c in cases)
    t_gemm = [time_graph(torch, c[0], iters) for c in cases]
    t_step = [time_graph(torch, c[1], iters) for c in cases]
    both = lambda: (cases[0][0](), cases[1][0]())
    ghz = clock_under(vt, torch, both, iters, sum(t_gemm))
    ach = flops / sum(t_gemm) / 1e12
    splits = [c[3] for c in cases]
    name = ("gemm_dl_kernel<128, 128, 4, 2, 3, 3, true, 64, 0> (split-K partial products of the O %dx1280x1280 "
            "and FC2 %dx1280x5120 residual Linears, %d and %d splits)" % (M, M, splits[0], splits[1])
            if min(splits) > 1 else "gemm_dl_kernel (O and FC2 residual Linears at %d tokens, unsplit)" % M)
    return {"kernel": name, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS,
            "traffic": profile_traffic("gemm_residual_%d_traffic" % M,
                                       "vision_transformer_encoder_tiled_amd/csrc/gemm.hip"),
            **at_clock(ach, ghz), "flops_per_launch": flops / 2, "flops_O_FC2": [c[2] for c in cases],
            "avg_launch_us": sum(t_gemm) / 2 * 1e6, "launch_us_O_FC2": [t * 1e6 for t in t_gemm],
            "with_reduce_ln": {"kernels": "partials + resid_ln_row_kernel (split-K sum, bias, residual, LayerNorm)",
                               "achieved": flops / sum(t_step) / 1e12,
                               "frac": flops / sum(t_step) / 1e12 / PEAK_BF16_TFLOPS,
                               "step_us_O_FC2": [t * 1e6 for t in t_step]},
            "note": "traffic is per launch, averaged over one O and one FC2 launch"}


def gemm_roofline(vt, torch, M, iters):
    fn, flops = fc1_case(vt, torch, M)
    t = time_graph(torch, fn, iters)
    ghz = clock_under(vt, torch, fn, iters, t)
    return {"kernel": "gemm_dl_kernel (FC1: %d x 5120 x 1280, bias+GELU epilogue)" % M,
            "bound": "mfma", "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS,
            "traffic": profile_traffic("gemm_fc1_%d_traffic" % M, "vision_transformer_encoder_tiled_amd/csrc/gemm.hip"),
            **at_clock(flops / t / 1e12, ghz),
            "flops_per_launch": flops, "avg_launch_us": t * 1e6}


def attention_roofline(vt, torch, grids, iters, traffic_profile=None):
    """The attention kernels as the tower runs them (vt_attention_packed: the
    attention kernel and, when the last round is split, its merge), and the
    whole vt_attention_varlen call beside them (with the RoPE/pack kernel and
    the per-call schedule and RoPE-table kernels, which the tower's blocks do
    in the QKV Linear's epilogue and once per call)."""
    fn = attention_packed_case(vt, torch, grids)
    call, flops = attention_case(vt, torch, grids)
    t = time_graph(torch, fn, iters)
    ghz = clock_under(vt, torch, fn, iters, t)
    tc = time_graph(torch, call, iters)
    N = sum(t_ * h * w for t_, h, w in grids)
    traffic = (profile_traffic(traffic_profile, "vision_transformer_encoder_tiled_amd/csrc/attention.hip")
               if traffic_profile else None)
    return {"kernel": "attention kernels (%d tokens, %d images)" % (N, len(grids)), "bound": "mfma",
            "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS, "traffic": traffic,
            "traffic_note": "attention kernel only (not the pack kernel)" if traffic else None,
            **at_clock(flops / t / 1e12, ghz),
            "flops_per_launch": flops,
            "avg_launch_us": t * 1e6,
            "varlen_call_us": tc * 1e6,
            "varlen_call_frac": flops / tc / 1e12 / PEAK_BF16_TFLOPS,
            "note": "avg_launch_us: one vt_attention_packed call (the attention kernel, plus the tail "
                    "merge when the last round is split), as in the tower; varlen_call_us: one whole "
                    "vt_attention_varlen call (schedule, RoPE table, RoPE/pack kernel, attention)"}


def layernorm_roofline(vt, torch, rows, iters):
    """vt_layer_norm (a3/a7) on rows x 1280: 7,680 algorithmic bytes per row
    (the fp32 row read, the bf16 row written) per launch time, against HBM."""
    g = np.random.Generator(np.random.PCG64(3))
    x = torch.from_numpy(g.standard_normal((rows, 1280), dtype=np.float32)).cuda()
    gam = torch.from_numpy(synth.bf16_bits(np.ones(1280, np.float32)).view(np.int16)).cuda()
    bet = torch.zeros(1280, dtype=torch.int16, device="cuda")
    out = torch.empty((rows, 1280), dtype=torch.int16, device="cuda")
    fn = lambda: vt.vt_layer_norm(x, rows, 1280, gam, bet, 1e-6, out)
    t = time_graph(torch, fn, iters)
    gbs = rows * 7680 / t / 1e9
    return {"kernel": "layer_norm_kernel (%d x 1280, fp32 in, bf16 out)" % rows, "bound": "hbm",
            "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "bytes_per_launch": rows * 7680, "avg_launch_us": t * 1e6}


def attention_backward_line(vt, torch, grids, iters):
    fn, flops = attention_backward_case(vt, torch, grids)
    t = time_kernel(torch, fn, iters)
    N = sum(t_ * h * w for t_, h, w in grids)
    return {"call": "vt_attention_backward (%d tokens, %d images, bf16 dqkv)" % (N, len(grids)),
            "bound": "mfma", "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS, "flops_per_call": flops,
            "avg_call_us": t * 1e6,
            "note": "whole call: schedule, forward recompute with log-sum-exp, both packs, the dQ "
                    "and the dK/dV kernels; FLOPs are the four gradient products only"}


def block_backward_line(vt, torch, grids, iters):
    fn, flops = block_backward_case(vt, torch, grids)
    t = time_kernel(torch, fn, iters)
    N = sum(t_ * h * w for t_, h, w in grids)
    return {"call": "vt_block_backward (%d tokens, %d images, all gradients)" % (N, len(grids)),
            "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / t / 1e12 / PEAK_BF16_TFLOPS, "flops_per_call": flops,
            "avg_call_us": t * 1e6, "tokens_per_s": N / t,
            "note": "one block's recomputed forward and backward; FLOPs = forward + backward "
                    "(3x the linear products, 12 n^2 d attention)"}


def tower_backward_line(vt, torch, wl, tw, weights, iters):
    fn, fl = tower_backward_case(vt, torch, wl, tw, weights)
    tt = time_kernel(torch, fn, max(2, iters // 5))
    return {"call": "vt_tower_backward (%s: 32 layers + patch embed, all gradients)" % wl.name,
            "achieved": fl / tt / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": fl / tt / 1e12 / PEAK_BF16_TFLOPS, "flops_per_call": fl, "ms_per_call": tt * 1e3,
            "patches_per_s": wl.tokens / tt,
            "note": "forward with every block input kept, then the backward of each block (which "
                    "recomputes that block's forward) and of the patch embed"}


def kernel_only(a):
    """--kernel: run one kernel case a fixed number of times (for counter runs)."""
    import torch
    import vision_transformer_encoder_tiled_amd as vt
    wl = synth.WORKLOADS[a.workload]
    if a.kernel == "fc1":
        fn, _ = fc1_case(vt, torch, wl.tokens)
    elif a.kernel == "resid_gemm":  # one O and one FC2 partial GEMM per call
        cases = residual_cases(vt, torch, wl.tokens)
        fn = lambda: (cases[0][0](), cases[1][0]())
    elif a.kernel == "attention":
        fn, _ = attention_case(vt, torch, list(wl.grids))
    elif a.kernel == "attention_bwd":
        fn, _ = attention_backward_case(vt, torch, list(wl.grids))
    elif a.kernel == "block_bwd":
        fn, _ = block_backward_case(vt, torch, list(wl.grids))
    else:
        fn, _ = copy_case(torch)
    fn()
    torch.cuda.synchronize()
    t = time_kernel(torch, fn, a.kernel_iters)
    print(json.dumps({"kernel": a.kernel, "workload": wl.name, "launches": a.kernel_iters + 5,
                      "avg_us": t * 1e6}), flush=True)


def cpu_baseline(weights):
    """The oracle, untuned, on the 448x448 image through the full tower,
    repeated until about 10 s of host work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    wl = synth.WORKLOADS["tower_448"]
    px = synth.make_batch_pixels(wl)
    # Whole passes over the 448x448 image until at least 10 s of host work.
    passes, t0 = 0, time.perf_counter()
    while passes < 8 and (passes == 0 or time.perf_counter() - t0 < 10.0):
        oracle.tower_forward(px, list(wl.grids), weights)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": passes * wl.tokens / dt, "unit": "patches/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d passes of one 448x448 image (1024 patches) through the 32-layer tower, merge "
                      "and projector, numpy fp32 on the host, %.1f s in all" % (passes, dt),
            "host_cpus": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; --gpus %d is not supported "
                                   "(how the path would shard is described, not implemented)" % a.gpus}))
        sys.exit(2)
    if a.kernel:
        return kernel_only(a)
    import torch
    import vision_transformer_encoder_tiled_amd as vt
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    wl = synth.WORKLOADS[a.workload]
    weights = synth.make_weights(32, projector=True)
    dev = {k: torch.from_numpy(v.view(np.int16)).cuda() for k, v in weights.items()}
    tw = vt.TowerWeights(dev, 32)

    run = Runner(vt, torch, tw, wl)
    secs, wall = run.time(a.steps, a.warmup)
    ms = secs / a.steps * 1e3
    gemm_f, attn_f = workload_flops(wl)
    value = wl.tokens * a.steps / secs

    res = {
        "metric": "ViT-tower patches/s (MiniMax-M3 tower: 32 layers + 2x2 merge + projector)",
        "value": value, "unit": "patches/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded U[0,1) pixels, random-init N(0,0.02) bf16 weights)",
        "config": {"workload": wl.name, "images": wl.n_img, "patches": wl.tokens,
                   "grid_hw": [list(g[1:]) for g in wl.grids][:16], "layers": wl.layers,
                   "projector": wl.projector, "attention_operands": "fp16", "gemm_operands": "bf16",
                   "accumulate": "fp32", "residual": "fp32"},
        "images_per_s": wl.n_img * a.steps / secs,
        "wall_s_timed_region": wall,
        "tflops_total": (gemm_f + attn_f) / (secs / a.steps) / 1e12,
    }
    M = wl.tokens
    res["roofline"] = residual_gemm_roofline(vt, torch, M, a.kernel_iters)
    res["fc1_roofline"] = gemm_roofline(vt, torch, M, a.kernel_iters)
    res["attention_roofline"] = attention_roofline(vt, torch, list(wl.grids), a.kernel_iters)
    if not a.no_backward:
        res["attention_backward"] = attention_backward_line(vt, torch, list(wl.grids), a.kernel_iters)
        res["block_backward"] = block_backward_line(vt, torch, list(wl.grids), a.kernel_iters)
        res["tower_backward"] = tower_backward_line(vt, torch, wl, tw, weights, a.kernel_iters)

    if a.secondary:
        wl2 = synth.WORKLOADS[a.secondary]
        del run
        run2 = Runner(vt, torch, tw, wl2)
        k2 = max(3, a.steps // 4)
        s2, _ = run2.time(k2, 1)
        g2, at2 = workload_flops(wl2)
        res["secondary"] = {
            "workload": wl2.name, "patches": wl2.tokens, "images": wl2.n_img,
            "patches_per_s": wl2.tokens * k2 / s2, "images_per_s": wl2.n_img * k2 / s2,
            "ms_per_step": s2 / k2 * 1e3, "steps": k2,
            "tflops_total": (g2 + at2) / (s2 / k2) / 1e12,
            "attention_roofline": attention_roofline(
                vt, torch, list(wl2.grids), max(3, a.kernel_iters // 4),
                "attention_2016_traffic" if wl2.name == "tower_2016" else None),
            "gemm_roofline": gemm_roofline(vt, torch, wl2.tokens, max(3, a.kernel_iters // 4)),
            "layernorm_roofline": layernorm_roofline(vt, torch, wl2.tokens, a.kernel_iters),
        }
        if not a.no_backward:
            res["secondary"]["attention_backward"] = attention_backward_line(
                vt, torch, list(wl2.grids), max(3, a.kernel_iters // 4))
            res["secondary"]["block_backward"] = block_backward_line(vt, torch, list(wl2.grids),
                                                                     max(3, a.kernel_iters // 4))
        del run2

    more = []
    for name in [m for m in a.more.split(",") if m]:
        wl3 = synth.WORKLOADS[name]
        run3 = Runner(vt, torch, tw, wl3)
        k3 = max(3, a.steps // 4)
        s3, _ = run3.time(k3, 1)
        g3, at3 = workload_flops(wl3)
        line = {"workload": wl3.name, "patches": wl3.tokens, "items": wl3.n_img,
                "grids": [list(g) for g in wl3.grids][:16], "layers": wl3.layers, "projector": wl3.projector,
                "patches_per_s": wl3.tokens * k3 / s3, "items_per_s": wl3.n_img * k3 / s3,
                "ms_per_step": s3 / k3 * 1e3, "steps": k3,
                "tflops_total": (g3 + at3) / (s3 / k3) / 1e12}
        del run3
        if name in ("tower_448x16", "tower_mixed8"):  # workloads that fill the chip: their own rooflines
            it3 = max(3, a.kernel_iters // 2)
            line["attention_roofline"] = attention_roofline(vt, torch, list(wl3.grids), it3)
            line["gemm_roofline"] = gemm_roofline(vt, torch, wl3.tokens, it3)
        more.append(line)
    if more:
        res["more_workloads"] = more

    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(weights)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
