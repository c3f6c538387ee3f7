"""The decode step replayed from a captured HIP graph (as the benchmark times
it) gives the same bits as eager launches, replay after replay, with eager
work and synchronisations in between."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, layer, needs_gpu, say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    needs_gpu()
    name, dims, ex = synth.config(2)
    B = 8
    # t mod s == 0: the step reopens its slot, so replaying it is idempotent
    pos = np.full(B, 2046, dtype=np.int32)
    ms = 2046 // dims.s + 1
    w, W, L = layer(dims, 91, "bf16", pe_rows=ms)
    state = synth.make_decode_state(dims, pos, ms, seed=92)
    step = synth.make_step(dims, w, pos, seed=93)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
    x, qr, kr = dev(step["x"], "bf16"), dev(step["QR"], "bf16"), dev(step["KR"], "bf16")
    p = torch.from_numpy(pos).cuda()
    Y = torch.empty(B, dims.d, dtype=torch.bfloat16, device="cuda")
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev[0].record()
    ev[1].record()
    L.decode_step(cache, x, qr, kr, p, 2046, Y)
    torch.cuda.synchronize()
    ref_y, ref_c = Y.clone(), cache.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L.decode_step(cache, x, qr, kr, p, 2046, Y, events=ev)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        Y.zero_()
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("replay", i, "attention kernel ms", ev[0].elapsed_time(ev[1]))
        assert torch.equal(Y, ref_y), i
        assert torch.equal(cache.view(torch.int16), ref_c.view(torch.int16)), i
        del junk


def _replay_check(fn, outs, tol=None, n=3, reset=None):
    """Run fn eagerly, capture it, replay n times with eager work and
    synchronisations between the replays, and compare every output with the
    eager result (bit for bit, or within the relative tolerance `tol`).
    Before each replay the outputs are poisoned with NaN, or `reset()` puts
    them back in the state the eager call started from."""
    if reset is not None:
        reset()
    fn()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    for i in range(n):
        if reset is not None:
            reset()
        else:
            for o in outs:
                o.fill_(float("nan"))
        junk = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            if tol is None:
                assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                                   r.view(torch.int16) if r.dtype == torch.bfloat16 else r), (i, k)
            else:
                den = r.abs().max().clamp_min(1e-30)
                assert float((o - r).abs().max() / den) <= tol, (i, k)
        del junk


def test_graph_replay_prefill_and_backward():
    """The absorbed and per-head forwards and the per-head backward from
    captured graphs, bit for bit (the backward adds its partial sums in a
    fixed order)."""
    needs_gpu()
    from synth import Dims
    import oracle.mtla as om
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    B, T = 2, 300
    ms = om.n_slots(T, dims.s)
    w = synth.make_weights(dims, 9900, "bf16", pe_rows=ms)
    L = MTLALayer.from_arrays(dims, {**w, **synth.head_maps(w)}, MTLA_BF16)
    seq = synth.make_sequence(dims, w, B, T, 9901, "bf16")
    X, QR, KR = dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16")
    Y = torch.empty(B, T, dims.d, dtype=torch.bfloat16, device="cuda")
    cache = L.new_cache(B, ms)
    say("graph: per-head forward")
    _replay_check(lambda: L.prefill_unabsorbed(X, QR, KR, Y, cache=cache), [Y, cache])
    say("graph: absorbed forward")
    Cp = torch.empty(B, T, dims.r, dtype=torch.bfloat16, device="cuda")
    _replay_check(lambda: L.prefill(X, QR, KR, Y, cache=cache, Cprime=Cp), [Y, cache, Cp])
    dY = dev(np.random.default_rng(9902).normal(size=(B, T, dims.d)), "bf16")
    outs = {}

    def bwd():
        dX, dQR, dKR, grads = L.backward_unabsorbed(X, QR, KR, dY)
        outs.update(dX=dX, dQR=dQR, dKR=dKR, **grads)
    bwd()
    torch.cuda.synchronize()
    # the binding allocates its outputs; capture a call writing into fixed ones
    from kv_cache_compressed_amd import mtla_prefill_unabsorbed_backward, GRAD_NAMES, OP_BACKWARD
    fixed = {k: v.clone() for k, v in outs.items()}
    ws = L.workspace(OP_BACKWARD, B, T)
    fn = lambda: mtla_prefill_unabsorbed_backward(
        L.dims, L.wu, L.t["W_hc"], X, QR, KR, dY, {k: fixed[k] for k in GRAD_NAMES},
        fixed["dX"], fixed["dQR"], fixed["dKR"], ws)
    say("graph: backward")
    _replay_check(fn, [fixed["dX"], fixed["dQR"], fixed["dKR"]] + [fixed[k] for k in GRAD_NAMES])


def test_graph_replay_chunk_append_and_rope():
    """A chunked merge-append that starts on group boundaries (so replaying it
    reopens the same slots) and the RoPE inputs, from captured graphs."""
    needs_gpu()
    from synth import Dims
    from kv_cache_compressed_amd import mtla_rope_inputs
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    B, Lc = 4, 64
    pos0 = np.array([0, 10, 100, 1000], dtype=np.int32)
    ms = (int(pos0.max()) + Lc) // dims.s + 1
    w, W, L = layer(dims, 9910, "bf16", pe_rows=ms)
    ch = synth.make_chunk(dims, w, pos0, Lc, 9911, "bf16")
    cache = L.new_cache(B, ms)
    X, KR = dev(ch["X"], "bf16"), dev(ch["KR"], "bf16")
    p0 = torch.from_numpy(pos0).cuda()
    Cp = torch.empty(B, Lc, dims.r, dtype=torch.bfloat16, device="cuda")
    say("graph: chunk append")
    _replay_check(lambda: L.append_chunk(cache, X, KR, p0, int(pos0.max()) + Lc - 1, Cprime=Cp),
                  [cache, Cp], reset=lambda: (cache.zero_(), Cp.fill_(float("nan"))))
    W_QR = dev(w["W_QR"].reshape(-1, dims.d), "bf16")
    W_KRm = dev(w["W_KR"], "bf16")
    pos = (p0[:, None] + torch.arange(Lc, device="cuda", dtype=torch.int32)[None]).contiguous()
    QRo = torch.empty(B, Lc, dims.H, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    KRo = torch.empty(B, Lc, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    from kv_cache_compressed_amd import workspace, OP_ROPE
    ws = workspace(L.dims, OP_ROPE, B * Lc, 1)
    say("graph: rope inputs")
    _replay_check(lambda: mtla_rope_inputs(L.dims, W_QR, W_KRm, X, pos, 10000.0, QRo, KRo, ws),
                  [QRo, KRo])
