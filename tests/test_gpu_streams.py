"""Sub-batch calls on two streams reproduce the full call.

A caller may run independent parts of a batch as calls of their own, each on
its own stream with its own scratch, pointing into the same KV cache and tree:
the sequences of a decode batch split in two halves (the tree of sequence b and
KV head k sits at (b H_kv + k) times the per-tree size, the cache rows of
sequence b at b H_kv T d elements), or a block of positions split by KV head
(one geometry of G query heads over one KV head per call, the queries laid out
per KV head).  Both schedules must give the full call's routes exactly and its
outputs up to fp32 summation order (the attention's split-KV plan differs with
the number of heads in a call).  The two halves run concurrently on two
streams, so the test also checks that concurrent calls with separate scratch
do not interfere, also when both route heads through device-memory frontier
slots (their locks are shared by every call on the device).
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


def _same_routes(sel_a, cnt_a, sel_b, cnt_b):
    import torch
    assert torch.equal(cnt_a, cnt_b)
    c = cnt_a.reshape(-1).cpu().numpy()
    sa = sel_a.reshape(len(c), -1).cpu().numpy()
    sb = sel_b.reshape(len(c), -1).cpu().numpy()
    assert (c >= 0).all()
    for i in range(len(c)):
        assert np.array_equal(sa[i, :c[i]], sb[i, :c[i]]), i


def test_half_batches_on_two_streams_equal_the_full_batch(Z):
    import torch
    g = W.custom("streams-halves", 310, dtype=W.BF16, B=4, H_q=8, H_kv=2,
                 T=8 ** 4 * 2 + 8 * 3 + 5, C=8, L=4, p=0.95)
    say(f"half batches on two streams: B={g.B}, {g.B * g.H_q} query heads per step")
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(1))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    sel, cnt, _, _ = Z.route(gm, tree, Qd, 1, g.p, cap, want_stats=False, want_gap=False)
    O = Z.attn(gm, Qd, 1, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()

    hb = g.B // 2
    gh = Z.geom(W.replace(g, B=hb))
    tbh, _ = Z.tree_bytes(gh)
    tb, _ = Z.tree_bytes(gm)
    assert 2 * tbh == tb
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    # Buffers used on the second stream stay referenced until the synchronisation
    # after each round (the allocator orders reuse on the current stream only).
    bufs = [(torch.empty(max(Z.route_scratch_bytes(gh, 1, cap), 1), dtype=torch.uint8,
                         device="cuda"),
             torch.empty(max(Z.attn_scratch_bytes(gh, 1, cap), 1), dtype=torch.uint8,
                         device="cuda")) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(2):  # the second round reuses the scratch buffers
        outs = []
        for h in range(2):
            sl = slice(h * hb, (h + 1) * hb)
            sh, ch, _, _ = Z.route(gh, tree[h * tbh:(h + 1) * tbh], Qd[sl], 1, g.p, cap,
                                   want_stats=False, want_gap=False, scratch=bufs[h][0],
                                   stream=streams[h])
            oh = Z.attn(gh, Qd[sl], 1, Kd[sl], Vd[sl], sh, ch, cap, scratch=bufs[h][1],
                        stream=streams[h])
            outs.append((sh, ch, oh))
        torch.cuda.synchronize()
        _same_routes(sel, cnt, torch.cat([o[0] for o in outs]), torch.cat([o[1] for o in outs]))
        err = float((torch.cat([o[2] for o in outs]).float() - O.float()).abs().max())
        say(f"round {rep}: routes equal, max |O_halves - O_full| = {err:.2e}")
        assert err <= 2e-2


def test_block_split_by_kv_head_on_two_streams_equals_the_single_call(Z):
    import torch
    g = W.custom("streams-kv", 311, dtype=W.BF16, B=1, H_q=16, H_kv=2,
                 T=32 ** 3 * 2 + 45, C=32, L=3, p=0.95)
    n_pos = 320  # 5,120 query heads: the throughput router and the block attention path
    say(f"block split by KV head: {n_pos * g.H_q} query heads in the single call")
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(n_pos))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    sel, cnt, _, _ = Z.route(gm, tree, Qd, n_pos, g.p, cap, want_stats=False, want_gap=False)
    O = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()

    g1 = Z.geom(W.replace(g, H_q=g.G, H_kv=1))
    tb1, _ = Z.tree_bytes(g1)
    tb, _ = Z.tree_bytes(gm)
    assert tb1 * g.H_kv == tb
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    # Every buffer a call on the second stream uses stays referenced until the
    # synchronisation below (the allocator orders reuse on the current stream only).
    qs = [Qd[:, :, k * g.G:(k + 1) * g.G].contiguous() for k in range(g.H_kv)]
    scr = [(torch.empty(max(Z.route_scratch_bytes(g1, n_pos, cap), 1), dtype=torch.uint8,
                        device="cuda"),
            torch.empty(max(Z.attn_scratch_bytes(g1, n_pos, cap), 1), dtype=torch.uint8,
                        device="cuda")) for _ in range(g.H_kv)]
    torch.cuda.synchronize()
    outs = []
    for k in range(g.H_kv):
        sk, ck, _, _ = Z.route(g1, tree[k * tb1:(k + 1) * tb1], qs[k], n_pos, g.p, cap,
                               want_stats=False, want_gap=False, scratch=scr[k][0],
                               stream=streams[k])
        ok = Z.attn(g1, qs[k], n_pos, Kd[:, k:k + 1], Vd[:, k:k + 1], sk, ck, cap,
                    scratch=scr[k][1], stream=streams[k])
        outs.append((sk, ck, ok))
    torch.cuda.synchronize()
    _same_routes(sel, cnt, torch.cat([o[0] for o in outs], dim=2),
                 torch.cat([o[1] for o in outs], dim=2))
    err = float((torch.cat([o[2] for o in outs], dim=2).float() - O.float()).abs().max())
    say(f"routes equal, max |O_split - O_single| = {err:.2e}")
    assert err <= 2e-2


def test_concurrent_calls_with_device_memory_frontiers(Z):
    # Weak queries at p = 0.99 keep nearly every candidate, so their level-1
    # frontiers (n_1 = 4,802) outgrow the on-chip capacity and are routed again
    # in device-memory frontier slots.  The slots' locks are one array per
    # device, shared by every call; each call's slots are in its own scratch.
    # Two calls of one sequence each, on two streams at once, must give the
    # routes of the single two-sequence call.
    import torch
    g = W.custom("streams-spill", 312, dtype=W.BF16, B=2, H_q=4, H_kv=1, C=16, L=2,
                 T=16 * 16 * 300 + 37, R=1, p=0.99)
    n_pos = 3
    say(f"concurrent spilling calls: n_1={g.n_level(1)}, {g.B} x {n_pos} x {g.H_q} query heads")
    K, _ = W.make_kv(g, want_v=False)
    Qn = W.make_query_block(g, K, range(n_pos))
    rng = np.random.default_rng(312)
    weak = rng.standard_normal((g.B, 2, g.H_q, g.d)).astype(np.float32) * np.float32(0.05)
    Qn[:, [0, 2]] = W.f32_to_bf16_bits(weak)
    gm = Z.geom(g)
    Kd, Qd = to_device(K, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    sel, cnt, stats, _ = Z.route(gm, tree, Qd, n_pos, g.p, cap, want_gap=False)
    torch.cuda.synchronize()
    assert int(stats[..., 0].max()) > Z.frontier_capacity(), "the case must spill"

    g1 = Z.geom(W.replace(g, B=1))
    tb1, _ = Z.tree_bytes(g1)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    scr = [torch.empty(max(Z.route_scratch_bytes(g1, n_pos, cap), 1), dtype=torch.uint8,
                       device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    outs = []
    for b in range(2):
        outs.append(Z.route(g1, tree[b * tb1:(b + 1) * tb1], Qd[b:b + 1], n_pos, g.p, cap,
                            want_gap=False, scratch=scr[b], stream=streams[b]))
    torch.cuda.synchronize()
    _same_routes(sel, cnt, torch.cat([o[0] for o in outs]), torch.cat([o[1] for o in outs]))
    assert torch.equal(stats, torch.cat([o[2] for o in outs]))
    say("  routes of the concurrent one-sequence calls equal the two-sequence call")
