"""Decode launches replayed from a captured HIP graph, and the no-allocation
scratch across calls of different shapes.

The split partials of a decode call are merged by the last block of each
(batch, KV head) to arrive, found through an arrival counter in the
workspace that this block sets back to zero; a replayed launch (whose
arguments are frozen at capture) therefore finds the counters as the
previous launch left them.  Each replay gets new inputs, copied eagerly
into the captured buffers, and must reproduce an eager call on a separate
workspace bit for bit (same kernels, same split count, fixed summation
order); eager decode calls on the captured workspace run between the
replays too.  The no-allocation entry point is called with a batch, a
larger batch (more counter words than before) and the first batch again,
each checked against the workspace entry point."""
import numpy as np
import pytest
import torch

from calibration_free_kv_amd import kvq, synth
from tests.gpu_util import needs_gpu, to_np

pytestmark = [pytest.mark.gpu, needs_gpu]


def codes(seed, B, Hkv, T, bits):
    c = synth.random_codes(seed, (B, Hkv, T), bits)
    return (torch.from_numpy(c["codes"]).cuda(), torch.from_numpy(c["norms"]).cuda())


def fill(dst, seed, positive=False):
    x = synth.random_tensor(seed, tuple(dst.shape), dtype=np.float32)
    if positive:  # norms
        x = np.abs(x) + 1.0
    dst.copy_(torch.from_numpy(x).cuda())


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays_match_eager(noalloc):
    B, Hkv, Hq, T, bits = 1, 8, 32, 5000, 3
    ctx = kvq.Context(Hkv, bits, seed=3)
    kc, kn = codes(11, B, Hkv, T, bits)
    vc, vn = codes(12, B, Hkv, T, bits)
    q = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
    ws = ctx.decode_ws(B, Hq, T)
    ws_eager = ctx.decode_ws(B, Hq, T)

    def launch():
        if noalloc:
            ctx.attn_decode_noalloc(q, kc, kn, vc, vn, out=out)
        else:
            ctx.attn_decode(q, kc, kn, vc, vn, ws=ws, out=out)

    fill(q, 100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    torch.cuda.synchronize()
    for r in range(5):
        fill(q, 200 + r)
        fill(vn, 300 + r, positive=True)
        graph.replay()
        torch.cuda.synchronize()
        got = to_np(out).copy()
        want = to_np(ctx.attn_decode(q, kc, kn, vc, vn, ws=ws_eager))
        assert np.isfinite(got).all()
        assert np.array_equal(got, want), "replay %d: max |diff| %.3g" % (r, float(np.abs(got - want).max()))
        launch()  # an eager call on the captured workspace between replays
        torch.cuda.synchronize()
        assert np.array_equal(to_np(out), want)
    print("noalloc=%s: 5 replays equal to eager calls" % noalloc)


def test_noalloc_scratch_across_batch_shapes():
    Hkv, Hq, T, bits = 8, 32, 3000, 2
    ctx = kvq.Context(Hkv, bits, seed=4)
    for i, B in enumerate([1, 24, 1, 3]):
        kc, kn = codes(20 + i, B, Hkv, T, bits)
        vc, vn = codes(40 + i, B, Hkv, T, bits)
        q = torch.from_numpy(synth.random_tensor(60 + i, (B, Hq, 128))).cuda()
        got = to_np(ctx.attn_decode_noalloc(q, kc, kn, vc, vn))
        want = to_np(ctx.attn_decode(q, kc, kn, vc, vn))
        err = float(np.abs(got - want).max())
        print("B=%d max |noalloc - workspace| %.3g" % (B, err))
        assert np.isfinite(got).all() and err <= 2e-3
