"""zha_route + zha_attn captured in a HIP graph and replayed.

The library never allocates, never synchronises and launches only kernels on
the caller's stream (no memset nodes), so a decode step or a block call can be
captured once and replayed.  Each case captures one call of each, replays the
graph several times with eager work and a synchronisation between replays,
and checks every replay bit for bit against the same calls run eagerly: a
decode call (the latency-shape router, the balanced attention path) and a
4096-head block call (the throughput router with its re-route list, the block
attention path).
"""
import sys

import numpy as np
import pytest

from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from hierarchical_tree_indexed_04_amd import zha
    zha.load()
    return zha


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name,kw,n_pos", [
    ("decode", dict(B=2, H_q=8, H_kv=2, T=8 ** 4 * 3 + 8 * 5 + 3, C=8, L=4, p=0.95), 1),
    ("block", dict(B=1, H_q=8, H_kv=1, T=32 ** 3 * 2 + 77, C=32, L=3, p=0.99), 512),
])
def test_captured_route_and_attention_replay_exactly(Z, name, kw, n_pos):
    import torch
    g = W.custom(f"graph-{name}", 190, dtype=W.BF16, **kw)
    say(f"graph capture: {name}, {g.B * n_pos * g.H_q} query heads")
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(n_pos))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    sel = torch.empty((g.B, n_pos, g.H_q, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((g.B, n_pos, g.H_q), dtype=torch.int32, device="cuda")
    stats = torch.empty((g.B, n_pos, g.H_q, g.L, 2), dtype=torch.int32, device="cuda")
    O = torch.empty((g.B, n_pos, g.H_q, g.d), dtype=torch.bfloat16, device="cuda")
    rs = torch.empty(max(Z.route_scratch_bytes(gm, n_pos, cap), 1), dtype=torch.uint8, device="cuda")
    asc = torch.empty(max(Z.attn_scratch_bytes(gm, n_pos, cap), 1), dtype=torch.uint8, device="cuda")

    def call(stream):
        Z.route(gm, tree, Qd, n_pos, g.p, cap, out=(sel, cnt, stats, None), scratch=rs,
                stream=stream)
        Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, O=O, scratch=asc, stream=stream)

    call(None)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (sel, cnt, stats, O)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        for x in (sel, cnt, stats, O):
            x.zero_()
        for buf in (rs, asc):  # whatever the scratch buffers held before must not matter
            buf.copy_(torch.randint(0, 255, (buf.numel(),), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        c = cnt.cpu()
        assert torch.equal(c, ref[1].cpu()), rep
        assert torch.equal(stats.cpu(), ref[2].cpu()), rep
        s_h, r_h = sel.cpu().numpy(), ref[0].cpu().numpy()
        for idx in np.ndindex(*c.shape):
            n = int(c[idx])
            assert np.array_equal(s_h[idx][:n], r_h[idx][:n]), (rep, idx)
        assert torch.equal(O.view(torch.int16), ref[3].view(torch.int16)), rep
        call(None)  # eager work between replays
        torch.cuda.synchronize()
    say(f"  4 replays identical to the eager call")
