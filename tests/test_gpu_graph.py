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
