#!/usr/bin/env python3
"""Benchmark of the MTLA hot path on one MI355X.

Headline (the JSON line's `value`): decode tokens/s of one MTLA layer on the
LLM-scale step (B=128, d=4096, H=32, d_h=128, r=512, d_hR=64, s=2, 32768
frames of context = 16384 compressed slots per sequence, bf16 cache, fp32
accumulation), the largest decode workload.  One step is one full
mtla_decode_step: latent and absorbed query projection, hyper-network gate
with the in-place merge into slot floor(t/s), split-K attention over the
compressed cache, combine and the absorbed output projection.  tokens/s = B /
step time.

The timed region is `--steps` consecutive decode steps enqueued while the GPU
is held by a spin kernel, so that they then execute back to back: host launch
latency stays out of the GPU timeline, as it would under graph replay.  A
second pass of the same steps launches the attention kernel with a pair of HIP
events that the runtime stamps with that kernel's own start and end
(hipExtLaunchKernel through the library's timed entry point); its step time
is reported beside the first pass's.  Caches smaller than 1 GiB are
replicated and each step reads a different replica, so the cache is streamed
from HBM and not from the 256 MB Infinity Cache (the LLM-scale cache is
2.4 GB and needs none).

`roofline` is that of the split-K attention kernel: algorithmic bytes (the
compressed cache rows the step must read, sum_b (floor(t_b/s)+1) *
(r + d_hR) * 2 B) over its average duration, from the HIP event pairs of the
second pass; `traffic` is the HBM bytes per launch from the committed counter
summary under profiles/ while the kernel's sources are unchanged.

Also reported (same line): the speech-decoder and ragged decode workloads
(each with its roofline), the strided prefill (TFLOP/s of the attention kernel
on visible pairs only, and of the whole forward, in the absorbed form and in
the per-head form), the backward of the per-head form (also both at the
LLM-scale head widths d_h = 128, d_hR = 64, r = 512), the chunked
merge-append (frames/s), the library's decoupled-RoPE inputs, the speech
decode at s = 1 (the MLA reduction: twice the slots, for the speed and memory
ratio), and the CPU oracle timed on the host cores beside each decode workload
and the prefill, on bounded samples (`cpu_baseline` for the headline,
`cpu_baseline` entries inside the other records).

All inputs are seeded synthetic tensors (no datasets or trained weights).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "kv_cache_compressed_amd", "csrc")
# Sources that define each timed kernel (its device code and launch plan):
# a counter summary under profiles/ applies only while these files are
# unchanged.
KERNEL_SOURCES = {
    "decode_ws_kernel": ("decode.hip", "common.h"),
    "prefill_ws_kernel": ("attention.hip", "common.h"),
    "heads_attn_kernel": ("heads.hip", "common.h"),
}
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "decode tokens/s + achieved HBM GB/s (compressed cache); prefill TFLOP/s, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Timing events of the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence: recording them adds no system-scope release
    (no L2 write-back), so a pair recorded around one kernel brackets that
    kernel alone."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so.7")   # already loaded by torch: same runtime
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the counter summary
    profiles/<workload>_traffic.md (rocprofv3 FETCH_SIZE and WRITE_SIZE,
    scaled by the factor a plain copy of known size gave in the same runs),
    or None when there is no summary or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic_record: "):
                rec = json.loads(line[len("traffic_record: "):])
    if not rec or rec.get("kernel") != kernel or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec


def calib_copy(mib: int):
    """A plain elementwise pass of known size for counter calibration: reads
    `mib` MiB and writes `mib` MiB (bf16 negation into a second buffer, both
    larger than the 256 MB Infinity Cache)."""
    import torch
    n = (mib << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def _decode_setup(cfg: int, seed_pos=None, stride=None):
    import torch
    import synth
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16
    name, dims, ex = synth.config(cfg)
    if stride is not None:
        dims = synth.Dims(**{**dims.asdict(), "s": stride})
        name = f"{name}_s{stride}"
    B = ex["B"]
    if "ctx" in ex:
        pos = np.full(B, ex["ctx"] - 1, dtype=np.int32)
    else:
        rng = np.random.default_rng(synth.seed_for(cfg))
        pos = (rng.integers(ex["ctx_lo"], ex["ctx_hi"] + 1, size=B) - 1).astype(np.int32)
    max_pos = int(pos.max())
    ms = max_pos // dims.s + 1
    w = synth.make_weights(dims, synth.seed_for(cfg), "bf16", pe_rows=ms)
    layer = MTLALayer.from_arrays(dims, w, MTLA_BF16)
    row = dims.r + dims.d_hR
    one = B * ms * row * 2
    n_rep = max(1, math.ceil((1 << 30) / one)) if one < (1 << 30) else 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.seed_for(cfg))
    caches = []
    for _ in range(n_rep):
        c = torch.empty(B, ms, row, dtype=torch.bfloat16, device="cuda")
        c[..., :dims.r].normal_(0.0, 0.7, generator=gen)
        c[..., dims.r:].normal_(0.0, 1.0, generator=gen)
        caches.append(c)
    step = synth.make_step(dims, w, pos, seed=synth.seed_for(cfg) + 2)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    inputs = (dev(step["x"]), dev(step["QR"]), dev(step["KR"]), torch.from_numpy(pos).cuda())
    Y = torch.empty(B, dims.d, dtype=torch.bfloat16, device="cuda")
    cache_bytes = int(np.sum(pos // dims.s + 1)) * row * 2
    return dict(name=name, dims=dims, B=B, pos=pos, max_pos=max_pos, layer=layer, caches=caches,
                inputs=inputs, Y=Y, cache_bytes=cache_bytes, weights=w, ms=ms)


def _host_ahead(fn, n, sleep_cycles):
    """Enqueue n calls of fn(i) while the GPU is held busy by a spin kernel,
    so the GPU then runs them back to back: host launch latency stays out of
    the GPU timeline and events recorded between kernels bracket exactly the
    kernel between them.  Returns (total_ms, ok) where ok says the spin
    outlasted the host's enqueueing."""
    import torch
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin_done = torch.cuda.Event()
    torch.cuda.synchronize()
    torch.cuda._sleep(sleep_cycles)
    spin_done.record()
    t0.record()
    for i in range(n):
        fn(i)
    t1.record()
    ok = not spin_done.query()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), ok


def _timed_loop(fn, n):
    """_host_ahead with a spin long enough to cover the enqueueing."""
    cycles = 20_000_000
    for _ in range(6):
        total, ok = _host_ahead(fn, n, cycles)
        if ok:
            return total
        cycles *= 4
    raise RuntimeError("could not keep the GPU busy while enqueueing the timed steps")


def run_decode(cfg: int, steps: int, warmup: int, stride=None) -> dict:
    """Time `steps` decode steps; returns step and attention-kernel times.
    `stride` overrides the workload's s (s = 1 is the MLA reduction: one
    slot per frame)."""
    import torch
    S = _decode_setup(cfg, stride=stride)
    layer, caches, (x, qr, kr, pos), Y = S["layer"], S["caches"], S["inputs"], S["Y"]
    n_rep, max_pos = len(caches), S["max_pos"]
    hip = HipEvents()
    ev = [(hip.create(), hip.create()) for _ in range(steps)]

    def one(i, events=None):
        layer.decode_step(caches[i % n_rep], x, qr, kr, pos, max_pos, Y, events=events)

    for i in range(max(warmup, 1)):
        one(i)
    torch.cuda.synchronize()
    # Throughput: `steps` plain decode steps.  Then the same steps again with
    # event pairs recorded around the attention kernel (the markers add gaps
    # between kernels, so they stay out of the throughput pass).
    total_ms = _timed_loop(lambda i: one(i), steps)
    total_ev_ms = _timed_loop(lambda i: one(i, ev[i]), steps)
    attn_ms = [hip.elapsed_ms(a, b) for a, b in ev]
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    step_ms = total_ms / steps
    attn_avg = float(np.mean(attn_ms))
    return dict(name=S["name"], B=S["B"], dims=S["dims"].asdict(), steps=steps,
                replicas=n_rep, step_ms=step_ms, step_ms_event_pass=total_ev_ms / steps,
                attn_ms=attn_avg,
                attn_ms_median=float(np.median(attn_ms)), cache_bytes=S["cache_bytes"],
                tokens_per_s=S["B"] / (step_ms * 1e-3),
                attn_gbs=S["cache_bytes"] / (attn_avg * 1e-3) / 1e9,
                ctx_min=int(S["pos"].min()) + 1, ctx_max=int(S["pos"].max()) + 1)


def prefill_flops(B, T, H, r, dR, s):
    """Algorithmic flops of the strided attention (visible pairs only) and of
    the projections of the parallel form."""
    pairs_per_bh = sum(m // s + 1 for m in range(T))
    attn = B * H * pairs_per_bh * (2 * (r + dR) + 2 * r)
    return attn, pairs_per_bh


def run_prefill(steps: int = 10, warmup: int = 3) -> dict:
    import torch
    import synth
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16
    name, dims, ex = synth.config(4)
    B, T = ex["B"], ex["T"]
    ms = -(-T // dims.s)
    w = synth.make_weights(dims, synth.seed_for(4), "bf16", pe_rows=ms)
    layer = MTLALayer.from_arrays(dims, w, MTLA_BF16)
    seq = synth.make_sequence(dims, w, B, T, synth.seed_for(4) + 1, "bf16")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    X, QR, KR = dev(seq["X"]), dev(seq["QR"]), dev(seq["KR"])
    del seq
    Y = torch.empty(B, T, dims.d, dtype=torch.bfloat16, device="cuda")
    cache = layer.new_cache(B, ms)
    hip = HipEvents()
    ev = [(hip.create(), hip.create()) for _ in range(steps)]
    for i in range(warmup):
        layer.prefill(X, QR, KR, Y, cache=cache)
    torch.cuda.synchronize()
    fwd_ms = _timed_loop(lambda i: layer.prefill(X, QR, KR, Y, cache=cache), steps) / steps
    _timed_loop(lambda i: layer.prefill(X, QR, KR, Y, cache=cache, events=ev[i]), steps)
    attn_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in ev]))
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    attn_flops, pairs = prefill_flops(B, T, dims.H, dims.r, dims.d_hR, dims.s)
    M = B * T
    proj_flops = (2 * M * dims.d * dims.r            # latent
                  + 2 * M * dims.r * dims.r          # gate content branch
                  + 2 * M * dims.d * dims.H * dims.r  # absorbed queries
                  + 2 * M * dims.H * dims.r * dims.d)  # absorbed output
    return dict(name=name, B=B, T=T, dims=dims.asdict(), steps=steps, forward_ms=fwd_ms,
                attn_ms=attn_ms, visible_pairs=B * dims.H * pairs, attn_flops=attn_flops,
                proj_flops=proj_flops, attn_tflops=attn_flops / (attn_ms * 1e-3) / 1e12,
                forward_tflops=(attn_flops + proj_flops) / (fwd_ms * 1e-3) / 1e12,
                tokens_per_s=M / (fwd_ms * 1e-3))


def run_append(steps: int = 20, warmup: int = 3) -> dict:
    """Chunked merge-append on the speech-decoder shapes: 32 sequences take
    512 new frames each, starting at seeded positions in 0..1535 (most inside
    a group), into caches of 1024 slots.  One step is one mtla_append_chunk
    call (latent and gate projection of the 16384 frames, then the chunk
    merge); every step writes a different cache replica."""
    import torch
    import synth
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16
    _, dims, _ = synth.config(2)
    B, Lc, ms = 32, 512, 1024
    rng = np.random.default_rng(synth.seed_for(2) + 10)
    pos0 = rng.integers(0, ms * dims.s - Lc + 1, size=B).astype(np.int32)
    w = synth.make_weights(dims, synth.seed_for(2), "bf16", pe_rows=ms)
    layer = MTLALayer.from_arrays(dims, w, MTLA_BF16)
    ch = synth.make_chunk(dims, w, pos0, Lc, synth.seed_for(2) + 11, "bf16")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    X, KR = dev(ch["X"]), dev(ch["KR"])
    p0 = torch.from_numpy(pos0).cuda()
    max_pos = int(pos0.max()) + Lc - 1
    row = dims.r + dims.d_hR
    n_rep = 4
    caches = [torch.zeros(B, ms, row, dtype=torch.bfloat16, device="cuda") for _ in range(n_rep)]
    one = lambda i: layer.append_chunk(caches[i % n_rep], X, KR, p0, max_pos)
    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    step_ms = _timed_loop(one, steps) / steps
    frames = B * Lc
    slots = int(np.sum((pos0 + Lc - 1) // dims.s - pos0 // dims.s + 1))
    # bytes the call cannot avoid: frames and rotary keys in, weights, the
    # partial slots read back, every touched slot written
    io_bytes = (frames * (dims.d + dims.d_hR) * 2 + 2 * dims.r * dims.d * 2
                + int(np.sum(pos0 % dims.s != 0)) * dims.r * 2 + slots * row * 2)
    proj_flops = 2 * frames * dims.d * 2 * dims.r
    return dict(name="append_chunk_b32_l512", B=B, L=Lc, dims=dims.asdict(), steps=steps,
                step_ms=step_ms, frames_per_s=frames / (step_ms * 1e-3), slots_written=slots,
                io_bytes=io_bytes, io_gbs=io_bytes / (step_ms * 1e-3) / 1e9,
                proj_flops=proj_flops, proj_tflops=proj_flops / (step_ms * 1e-3) / 1e12)


def _prefill_workload(wide: bool):
    """(name, dims, B, T) of the prefill workload, or with wide=True the same
    frames per sequence at the LLM-scale head widths (d_h = 128, d_hR = 64,
    r = 4 d_h = 512; d = 1024, 8 heads, 8 sequences)."""
    import synth
    name, dims, ex = synth.config(4)
    if not wide:
        return name, dims, ex["B"], ex["T"]
    from synth import Dims
    return "prefill_b8_t4096_dh128", Dims(d=1024, H=8, d_h=128, r=512, d_hR=64, s=2), 8, ex["T"]


def run_prefill_unabsorbed(steps: int = 10, warmup: int = 3, wide: bool = False) -> dict:
    """The same prefill workload in the per-head form (mtla_prefill_unabsorbed):
    attention at head width over explicit per-head keys and values."""
    import torch
    import synth
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16
    name, dims, B, T = _prefill_workload(wide)
    ms = -(-T // dims.s)
    w = synth.make_weights(dims, synth.seed_for(4), "bf16", pe_rows=ms)
    layer = MTLALayer.from_arrays(dims, {**w, **synth.head_maps(w)}, MTLA_BF16)
    seq = synth.make_sequence(dims, w, B, T, synth.seed_for(4) + 1, "bf16")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    X, QR, KR = dev(seq["X"]), dev(seq["QR"]), dev(seq["KR"])
    del seq
    Y = torch.empty(B, T, dims.d, dtype=torch.bfloat16, device="cuda")
    cache = layer.new_cache(B, ms)
    hip = HipEvents()
    ev = [(hip.create(), hip.create()) for _ in range(steps)]
    run = lambda i, e=None: layer.prefill_unabsorbed(X, QR, KR, Y, cache=cache, events=e)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    fwd_ms = _timed_loop(run, steps) / steps
    _timed_loop(lambda i: run(i, ev[i]), steps)
    attn_ms = float(np.mean([hip.elapsed_ms(a, b) for a, b in ev]))
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    _, pairs = prefill_flops(B, T, dims.H, dims.r, dims.d_hR, dims.s)
    dh, dR, H, M = dims.d_h, dims.d_hR, dims.H, B * T
    attn_flops = B * H * pairs * (2 * (dh + dR) + 2 * dh)
    proj_flops = (2 * M * dims.d * 2 * dims.r          # latent and gate
                  + 2 * M * dims.d * H * dh            # per-head queries
                  + 2 * M * dims.r * 2 * H * dh        # per-head keys and values
                  + 2 * M * H * dh * dims.d)           # output
    return dict(name=name + "_per_head", B=B, T=T, dims=dims.asdict(), steps=steps,
                forward_ms=fwd_ms, attn_ms=attn_ms, visible_pairs=B * H * pairs,
                attn_flops=attn_flops, proj_flops=proj_flops,
                attn_tflops=attn_flops / (attn_ms * 1e-3) / 1e12,
                forward_tflops=(attn_flops + proj_flops) / (fwd_ms * 1e-3) / 1e12,
                tokens_per_s=M / (fwd_ms * 1e-3))


def run_backward(steps: int = 5, warmup: int = 2, wide: bool = False) -> dict:
    """Backward of the per-head form on the prefill workload: one step is one
    mtla_prefill_unabsorbed_backward call (the forward recomputed inside,
    then every input and weight gradient) for a seeded loss gradient dY."""
    import torch
    import synth
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16
    name, dims, B, T = _prefill_workload(wide)
    ms = -(-T // dims.s)
    w = synth.make_weights(dims, synth.seed_for(4), "bf16", pe_rows=ms)
    layer = MTLALayer.from_arrays(dims, {**w, **synth.head_maps(w)}, MTLA_BF16)
    seq = synth.make_sequence(dims, w, B, T, synth.seed_for(4) + 1, "bf16")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    X, QR, KR = dev(seq["X"]), dev(seq["QR"]), dev(seq["KR"])
    del seq
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.seed_for(4) + 3)
    dY = torch.randn(B, T, dims.d, generator=gen, device="cuda").to(torch.bfloat16)
    run = lambda i: layer.backward_unabsorbed(X, QR, KR, dY)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    step_ms = _timed_loop(run, steps) / steps
    _, pairs = prefill_flops(B, T, dims.H, dims.r, dims.d_hR, dims.s)
    dh, dR, H, M = dims.d_h, dims.d_hR, dims.H, B * T
    # attention backward, each product once: S, dP, dV, dK, dK^R, dQ, dQ^R
    attn_flops = B * H * pairs * (2 * (dh + dR) + 2 * dh + 2 * dh + 2 * dh + 2 * dR + 2 * dh + 2 * dR)
    return dict(name=name + "_backward", B=B, T=T, dims=dims.asdict(), steps=steps,
                step_ms=step_ms, attn_bwd_flops=attn_flops,
                tokens_per_s=M / (step_ms * 1e-3))


def run_rope(steps: int = 20, warmup: int = 3) -> dict:
    """Decoupled-RoPE inputs of the prefill workload's 65,536 frames
    (mtla_rope_inputs: one product pass and the rotation)."""
    import torch
    import synth
    from kv_cache_compressed_amd import MTLA_BF16, make_dims, mtla_rope_inputs, workspace, OP_ROPE
    name, dims, ex = synth.config(4)
    B, T = ex["B"], ex["T"]
    w = synth.make_weights(dims, synth.seed_for(4), "bf16", pe_rows=8)
    d = make_dims(dims.d, dims.H, dims.d_h, dims.r, dims.d_hR, dims.s, MTLA_BF16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.seed_for(4) + 5)
    X = torch.randn(B, T, dims.d, generator=gen, device="cuda").to(torch.bfloat16)
    W_QR, W_KR = dev(w["W_QR"].reshape(-1, dims.d)), dev(w["W_KR"])
    pos = torch.arange(T, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    QR = torch.empty(B, T, dims.H, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    KR = torch.empty(B, T, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    ws = workspace(d, OP_ROPE, B * T, 1)
    run = lambda i: mtla_rope_inputs(d, W_QR, W_KR, X, pos, 10000.0, QR, KR, ws)
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    step_ms = _timed_loop(run, steps) / steps
    M = B * T
    N = (dims.H + 1) * dims.d_hR
    return dict(name=name + "_rope_inputs", B=B, T=T, step_ms=step_ms,
                frames_per_s=M / (step_ms * 1e-3),
                io_bytes=M * (dims.d + N) * 2 + M * 4, flops=2 * M * dims.d * N)


def _blas_info():
    from threadpoolctl import threadpool_info
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    return int(threads), (blas[0].get("internal_api") if blas else "none")


def _decode_positions(cfg: int, ex: dict, B: int) -> np.ndarray:
    """The positions _decode_setup uses for workload cfg (same seed)."""
    import synth
    if "ctx" in ex:
        return np.full(B, ex["ctx"] - 1, dtype=np.int32)
    rng = np.random.default_rng(synth.seed_for(cfg))
    return (rng.integers(ex["ctx_lo"], ex["ctx_hi"] + 1, size=B) - 1).astype(np.int32)


def cpu_baseline(cfg: int, seconds: float, max_seqs: int) -> dict:
    """The oracle (numpy, fp32, untuned) on a bounded sample of decode
    workload `cfg`: its first `max_seqs` sequences (at their own positions),
    each given a seeded cache of its length, stepped one after another with
    oracle.decode_step until `seconds` of wall time have passed.  tokens/s =
    sequence steps done / time (every sequence of a step costs the same at
    equal lengths; at ragged lengths the sample is the workload's first
    sequences)."""
    import synth
    import oracle.mtla as om
    name, dims, ex = synth.config(cfg)
    B = ex["B"]
    pos = _decode_positions(cfg, ex, B)[:max_seqs]
    n = len(pos)
    ms = int(pos.max()) // dims.s + 1
    w = synth.make_weights(dims, synth.seed_for(cfg), "bf16", pe_rows=ms)
    W = om.with_position_table(w, ms)
    W = {k: np.asarray(v, dtype=np.float32) for k, v in W.items()}
    rng = np.random.default_rng(synth.seed_for(cfg))
    lat = [rng.normal(0, 0.7, size=(int(t) // dims.s + 1, dims.r)).astype(np.float32) for t in pos]
    rk = [rng.normal(0, 1.0, size=(int(t) // dims.s + 1, dims.d_hR)).astype(np.float32) for t in pos]
    step = synth.make_step(dims, w, pos, seed=synth.seed_for(cfg) + 2)
    x, qr, kr = (np.asarray(step[k], dtype=np.float32) for k in ("x", "QR", "KR"))
    n_tok, rounds = 0, 0
    t0 = time.perf_counter()
    while True:
        for b in range(n):
            om.decode_step(lat[b], rk[b], int(pos[b]), x[b], qr[b], kr[b], W, dims.s,
                           np.float32(dims.scale))
            n_tok += 1
        rounds += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads, blas = _blas_info()
    return dict(value=round(n_tok / el, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{rounds} rounds of decode steps over {n} of the {B} sequences of {name} "
                       f"({int(pos.min()) // dims.s + 1}-{ms} slots each), numpy fp32, {el:.1f} s; "
                       f"host cores visible: {len(os.sched_getaffinity(0))}; BLAS: {blas}")


def cpu_prefill_baseline() -> dict:
    """The oracle (numpy, fp32) on the prefill workload: sequence 0 alone
    (1/16 of the batch: sequences are independent), one oracle.prefill call;
    the full-batch figure is that time x 16."""
    import synth
    import oracle.mtla as om
    name, dims, ex = synth.config(4)
    B, T = ex["B"], ex["T"]
    ms = -(-T // dims.s)
    w = synth.make_weights(dims, synth.seed_for(4), "bf16", pe_rows=ms)
    W = om.with_position_table(w, ms)
    W = {k: np.asarray(v, dtype=np.float32) for k, v in W.items()}
    seq = synth.make_sequence(dims, w, 1, T, synth.seed_for(4) + 1, "bf16")
    X, QR, KR = (np.asarray(seq[k][0], dtype=np.float32) for k in ("X", "QR", "KR"))
    t0 = time.perf_counter()
    om.prefill(X, QR, KR, W, dims.s, np.float32(dims.scale))
    el = time.perf_counter() - t0
    threads, blas = _blas_info()
    return dict(value=round(T / el, 2), unit="frames/s", cores=threads, kind="oracle",
                full_batch_s=round(el * B, 2),
                sample=f"sequence 0 of {name} ({T} frames), one oracle.prefill call, numpy fp32, "
                       f"{el:.1f} s (x{B} for the batch); host cores visible: "
                       f"{len(os.sched_getaffinity(0))}; BLAS: {blas}")


def roofline(rec: dict, workload: str) -> dict:
    """Roofline block of the attention kernel of a decode record."""
    tr = measured_traffic(workload, "decode_ws_kernel")
    traffic = round(tr["fetch_bytes_per_launch"] + tr["write_bytes_per_launch"]) if tr else None
    return {"bound": "hbm", "kernel": "decode_ws_kernel",
            "achieved": round(rec["attn_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(rec["attn_gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": rec["cache_bytes"],
            "avg_kernel_us": round(rec["attn_ms"] * 1e3, 3)}


def mfma_roofline(rec: dict, kernel: str, traffic_workload=None) -> dict:
    """Roofline block of a bf16 attention kernel (bound by the matrix cores):
    algorithmic flops on visible pairs per launch over the kernel's HIP-event
    time, against the dense bf16 peak; traffic from the kernel's counter
    summary when one is valid for its sources."""
    tr = measured_traffic(traffic_workload, kernel) if traffic_workload else None
    traffic = round(tr["fetch_bytes_per_launch"] + tr["write_bytes_per_launch"]) if tr else None
    return {"bound": "mfma", "kernel": kernel, "achieved": round(rec["attn_tflops"], 1),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(rec["attn_tflops"] / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "flops_per_launch": rec["attn_flops"], "avg_kernel_us": round(rec["attn_ms"] * 1e3, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only", choices=["decode_b32_ctx2048", "ragged_decode_b64_s4",
                                       "llm_decode_b128_ctx32768", "prefill_b16_t4096",
                                       "append_chunk_b32_l512", "prefill_b16_t4096_per_head",
                                       "prefill_b16_t4096_backward", "rope_inputs_b16_t4096",
                                       "prefill_b8_t4096_dh128_per_head",
                                       "prefill_b8_t4096_dh128_backward",
                                       "decode_b32_ctx2048_s1"],
                    help="time one workload alone and print its record (for profiling runs)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="first run a plain elementwise pass reading and writing MIB MiB each "
                         "(the reference for scaling memory counters in profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the MTLA hot path here has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

    if args.calib_copy:
        calib_copy(args.calib_copy)
    if args.only == "rope_inputs_b16_t4096":
        print(json.dumps(run_rope(args.steps, args.warmup)), flush=True)
        return
    if args.only == "decode_b32_ctx2048_s1":
        print(json.dumps(run_decode(2, args.steps, args.warmup, stride=1)), flush=True)
        return
    if args.only == "prefill_b16_t4096_backward":
        print(json.dumps(run_backward(args.steps, args.warmup)), flush=True)
        return
    if args.only in ("prefill_b16_t4096_per_head", "prefill_b8_t4096_dh128_per_head"):
        rec = run_prefill_unabsorbed(args.steps, args.warmup,
                                     wide=args.only == "prefill_b8_t4096_dh128_per_head")
        rec["roofline"] = mfma_roofline(rec, "heads_attn_kernel", args.only)
        print(json.dumps(rec), flush=True)
        return
    if args.only == "prefill_b8_t4096_dh128_backward":
        print(json.dumps(run_backward(args.steps, args.warmup, wide=True)), flush=True)
        return
    if args.only == "append_chunk_b32_l512":
        print(json.dumps(run_append(args.steps, args.warmup)), flush=True)
        return
    if args.only:
        cfg = {"decode_b32_ctx2048": 2, "ragged_decode_b64_s4": 3,
               "llm_decode_b128_ctx32768": 5, "prefill_b16_t4096": 4}[args.only]
        rec = run_prefill(args.steps, args.warmup) if cfg == 4 else \
            run_decode(cfg, args.steps, args.warmup)
        rec["roofline"] = roofline(rec, args.only) if cfg != 4 else \
            mfma_roofline(rec, "prefill_ws_kernel", "prefill_b16_t4096")
        print(json.dumps(rec), flush=True)
        return
    log("llm_decode_b128_ctx32768 ...")
    head = run_decode(5, args.steps, args.warmup)
    log(f"  step {head['step_ms']*1e3:.1f} us, attention {head['attn_ms']*1e3:.1f} us, "
        f"{head['attn_gbs']:.0f} GB/s, {head['tokens_per_s']:.0f} tok/s")
    extra = {}
    log("decode_b32_ctx2048 ...")
    c2 = extra["decode_b32_ctx2048"] = run_decode(2, 50, 10)
    log("ragged_decode_b64_s4 ...")
    c3 = extra["ragged_decode_b64_s4"] = run_decode(3, 50, 10)
    for k, rec in (("decode_b32_ctx2048", c2), ("ragged_decode_b64_s4", c3)):
        rec["roofline"] = roofline(rec, k)
        log(f"  {k}: step {rec['step_ms']*1e3:.2f} us, attention {rec['attn_ms']*1e3:.2f} us "
            f"{rec['attn_gbs']:.0f} GB/s ({rec['roofline']['frac']:.1%}), "
            f"{rec['tokens_per_s']:.0f} tok/s")
    torch.cuda.empty_cache()
    log("prefill_b16_t4096 ...")
    p = extra["prefill_b16_t4096"] = run_prefill()
    p["roofline"] = mfma_roofline(p, "prefill_ws_kernel", "prefill_b16_t4096")
    log(f"  prefill: attention {p['attn_ms']:.3f} ms {p['attn_tflops']:.0f} TFLOP/s "
        f"({p['roofline']['frac']:.1%}), forward {p['forward_ms']:.3f} ms")
    log("prefill_b16_t4096_per_head ...")
    u = extra["prefill_b16_t4096_per_head"] = run_prefill_unabsorbed()
    u["roofline"] = mfma_roofline(u, "heads_attn_kernel", "prefill_b16_t4096_per_head")
    log(f"  per-head prefill: attention {u['attn_ms']:.3f} ms {u['attn_tflops']:.0f} TFLOP/s "
        f"({u['roofline']['frac']:.1%}), forward {u['forward_ms']:.3f} ms")
    log("prefill_b16_t4096_backward ...")
    bw = extra["prefill_b16_t4096_backward"] = run_backward()
    log(f"  backward (per-head form, forward recomputed): {bw['step_ms']:.3f} ms")
    torch.cuda.empty_cache()
    log("prefill_b8_t4096_dh128 (per-head form and backward at d_h = 128) ...")
    uw = extra["prefill_b8_t4096_dh128_per_head"] = run_prefill_unabsorbed(wide=True)
    uw["roofline"] = mfma_roofline(uw, "heads_attn_kernel", "prefill_b8_t4096_dh128_per_head")
    bww = extra["prefill_b8_t4096_dh128_backward"] = run_backward(wide=True)
    log(f"  d_h=128 per-head: attention {uw['attn_ms']:.3f} ms {uw['attn_tflops']:.0f} TFLOP/s "
        f"({uw['roofline']['frac']:.1%}), forward {uw['forward_ms']:.3f} ms; backward {bww['step_ms']:.3f} ms")
    log("decode_b32_ctx2048_s1 (the MLA reduction, one slot per frame) ...")
    m1 = extra["decode_b32_ctx2048_s1"] = run_decode(2, 50, 10, stride=1)
    m1["cache_bytes_vs_s2"] = m1["cache_bytes"] / c2["cache_bytes"]
    m1["step_time_vs_s2"] = m1["step_ms"] / c2["step_ms"]
    log(f"  s=1: step {m1['step_ms']*1e3:.2f} us, cache {m1['cache_bytes']/1e6:.1f} MB "
        f"({m1['cache_bytes_vs_s2']:.2f}x s=2), step time {m1['step_time_vs_s2']:.2f}x s=2")
    log("rope_inputs_b16_t4096 ...")
    ro = extra["rope_inputs_b16_t4096"] = run_rope()
    log(f"  rotary inputs: {ro['step_ms']*1e3:.1f} us for {ro['B'] * ro['T']} frames")
    log("append_chunk_b32_l512 ...")
    a = extra["append_chunk_b32_l512"] = run_append()
    log(f"  append: {a['step_ms']*1e3:.1f} us per chunk, {a['frames_per_s']:.3g} frames/s")
    log("cpu baselines (the oracle on bounded samples) ...")
    cpu = cpu_baseline(5, args.cpu_seconds, 8)
    log(f"  llm decode: {cpu['value']:.1f} tok/s ({cpu['sample']})")
    c2["cpu_baseline"] = cpu_baseline(2, args.cpu_seconds / 2, 32)
    c3["cpu_baseline"] = cpu_baseline(3, args.cpu_seconds / 2, 16)
    p["cpu_baseline"] = cpu_prefill_baseline()
    log(f"  speech decode {c2['cpu_baseline']['value']:.0f} tok/s, ragged "
        f"{c3['cpu_baseline']['value']:.0f} tok/s, prefill {p['cpu_baseline']['value']:.0f} frames/s")
    _, dims5, ex5 = __import__("synth").config(5)
    out = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random inputs and random-init weights of the workload's shapes)",
        "config": {"workload": "llm_decode_b128_ctx32768", "B": ex5["B"], "d": dims5.d,
                   "H": dims5.H, "d_h": dims5.d_h, "r": dims5.r, "d_hR": dims5.d_hR,
                   "s": dims5.s, "context_frames": ex5["ctx"],
                   "slots": ex5["ctx"] // dims5.s, "cache_replicas": head["replicas"]},
        "roofline": roofline(head, "llm_decode_b128_ctx32768"),
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
