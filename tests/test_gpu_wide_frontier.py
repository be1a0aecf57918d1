"""Routes whose frontier outgrows the router's on-chip capacity, against the oracle.

A frontier (the candidates of one level of one query head) larger than
zha_route_frontier_capacity() is routed again with the frontier in the
scratch buffer, so every valid head routes whatever its frontier's size.
Weak queries (small random vectors) score every summary alike, and with p =
0.99 nearly every candidate is kept at every level, so the level-1 frontier
approaches n_1 > 4096.  Strong queries (the workload's own) sit between them
in the same call and must route as before.  Each head is compared with the
oracle (paper §III-C top-p routing, App. E-E orphans); the many-head call
(throughput shape, latency shape, then device memory) must equal the same
positions routed in small calls, bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import (TOL, Parity, attend_on, compare_head, from_device, oracle_trees,
                          to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from hierarchical_tree_indexed_04_amd import zha
    zha.load()
    return zha


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def weaken(g, Qn, positions, seed):
    """Replaces the queries at the given positions by N(0, 0.05^2) vectors."""
    rng = np.random.default_rng(seed)
    weak = rng.standard_normal((g.B, len(positions), g.H_q, g.d)).astype(np.float32) * np.float32(0.05)
    Qn[:, positions] = W.f32_to_bf16_bits(weak) if g.dtype == W.BF16 else weak


def build(Z, g, K, V, chunked):
    import torch
    qref = W.make_qref(g, K)
    gm = Z.geom(g, Z.ZHA_KV_CHUNKED if chunked else Z.ZHA_KV_SPLIT)
    Kd, Vd = to_device(K, g.dtype), to_device(V, g.dtype)
    if chunked:
        Kd, Vd = Z.to_chunked(Kd, Vd, g.C), None
    tree = Z.build(gm, Kd, torch.from_numpy(qref).cuda())
    return gm, Kd, Vd, tree, qref


def check_heads(g, K, V, Qn, trees, sel, cnt, stats, Og, heads, gap):
    par = Parity()
    for (b, t, h) in heads:
        kvh = h // g.G
        Kf = W.to_float(K[b, kvh], g.dtype)
        Vf = W.to_float(V[b, kvh], g.dtype)
        q = W.to_float(Qn[b, t, h], g.dtype)
        r, o = O.zha_head(trees[(b, kvh)], q, Kf, Vf, g.p)
        compare_head(par, r, sel[b, t, h], int(cnt[b, t, h]), stats[b, t, h], Og[b, t, h], o,
                     TOL[g.dtype], (b, t, h), gap_row=gap[b, t, h],
                     attend_set=attend_on(q, Kf, Vf, g.C, g.T))
    say("  " + par.summary())
    par.check()
    return par


# n_1 > 4096 in every case; weak positions overflow the on-chip frontier.
WIDE = [
    ("two-level", dict(dtype=W.BF16, C=16, L=2, T=16 * 16 * 300 + 37, R=1), False),
    ("two-level-r2-fp32", dict(dtype=W.F32, C=16, L=2, T=16 * 16 * 300 + 37, R=2), True),
    ("one-level", dict(dtype=W.BF16, C=16, L=1, T=16 * 5000 + 5, R=1), False),
    ("three-level-c8", dict(dtype=W.BF16, C=8, L=3, T=8 ** 3 * 70 + 77, R=3), True),
]


@pytest.mark.parametrize("name,kw,chunked", WIDE, ids=[w[0] for w in WIDE])
def test_device_memory_frontier_matches_oracle(Z, name, kw, chunked):
    import torch
    g = W.custom(f"wide-{name}", 180, B=2, H_q=4, H_kv=1, p=0.99, **kw)
    say(f"{name}: T={g.T}, C={g.C}, L={g.L}, R={g.R}, n_1={g.n_level(1)}, "
        f"{'chunked' if chunked else 'split'} KV")
    K, V = W.make_kv(g)
    gm, Kd, Vd, tree, qref = build(Z, g, K, V, chunked)
    n_pos = 3
    Qn = W.make_query_block(g, K, range(n_pos))
    weaken(g, Qn, [0, 2], 180)
    Qd = to_device(Qn, g.dtype)
    cap = g.n_level(1)
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()
    sel, cnt, stats = sel.cpu().numpy(), cnt.cpu().numpy(), stats.cpu().numpy()
    gap = gap.cpu().numpy()
    assert (cnt >= 0).all()
    kmax = int(stats[..., 0].max())
    say(f"  largest frontier {kmax} (on-chip capacity {Z.frontier_capacity()})")
    assert kmax > Z.frontier_capacity(), "the case must exercise the device-memory frontier"
    if g.L > 1:  # strong queries stay on chip (with L = 1 the top level alone exceeds it)
        assert int(stats[:, 1, :, :, 0].max()) <= Z.frontier_capacity()
    trees = oracle_trees(g, K, qref, [(b, 0) for b in range(g.B)])
    heads = [(b, t, h) for b in range(g.B) for t in range(n_pos) for h in range(g.H_q)]
    check_heads(g, K, V, Qn, trees, sel, cnt, stats, from_device(Od, g.dtype), heads, gap)


@pytest.mark.parametrize("dtype,R,chunked", [(W.BF16, 1, False), (W.F32, 2, True)])
def test_device_memory_frontier_many_heads(Z, dtype, R, chunked):
    # 4096 query heads: the throughput shape lists every weak head, the latency
    # shape's list kernel outgrows its LDS on them too and routes them again
    # with the device-memory frontier.
    import torch
    g = W.custom("wide-many", 181, dtype=dtype, B=1, H_q=8, H_kv=1, C=16, L=2,
                 T=16 * 16 * 300 + 37, R=R, p=0.99)
    n_pos = 512
    say(f"many heads ({dtype}, R={R}): {n_pos} positions x {g.H_q} heads, n_1={g.n_level(1)}, "
        f"every 8th position weak")
    K, V = W.make_kv(g)
    gm, Kd, Vd, tree, qref = build(Z, g, K, V, chunked)
    Qn = W.make_query_block(g, K, range(n_pos))
    weak = list(range(0, n_pos, 8))
    weaken(g, Qn, weak, 181)
    Qd = to_device(Qn, g.dtype)
    cap = g.n_level(1)
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    parts = [Z.route(gm, tree, Qd[:, i:i + 64].contiguous(), 64, g.p, cap)
             for i in range(0, n_pos, 64)]
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()
    cnt_h, stats_h = cnt.cpu().numpy(), stats.cpu().numpy()
    assert (cnt_h >= 0).all()
    assert int(stats_h[:, weak, :, 0, 0].min()) > Z.frontier_capacity()
    for i, (s1, c1, st1, g1) in enumerate(parts):
        sl = slice(i * 64, (i + 1) * 64)
        assert np.array_equal(c1.cpu().numpy(), cnt_h[:, sl])
        assert np.array_equal(st1.cpu().numpy(), stats_h[:, sl])
        assert torch.equal(g1.cpu(), gap[:, sl].cpu())
        c = c1.cpu().numpy()
        for h in range(g.H_q):
            for t in range(64):
                n = int(c[0, t, h])
                assert torch.equal(s1[0, t, h, :n].cpu(), sel[0, i * 64 + t, h, :n].cpu())
    sel_h = sel.cpu().numpy()
    trees = oracle_trees(g, K, qref, [(0, 0)])
    rng = np.random.default_rng(181)
    heads = [(0, int(t), int(rng.integers(g.H_q))) for t in rng.choice(weak, 12, replace=False)]
    heads += [(0, int(rng.integers(n_pos)), int(rng.integers(g.H_q))) for _ in range(12)]
    check_heads(g, K, V, Qn, trees, sel_h, cnt_h, stats_h, from_device(Od, g.dtype), heads,
                gap.cpu().numpy())


def test_device_memory_frontier_causal_prefill(Z):
    # ctx_len per position: the last positions see nearly all of n_1 > 4096.
    import torch
    g = W.custom("wide-causal", 182, dtype=W.BF16, B=1, H_q=4, H_kv=1, C=16, L=2,
                 T=16 * 16 * 300 + 37, R=1, p=0.99)
    K, V = W.make_kv(g)
    gm, Kd, Vd, tree, qref = build(Z, g, K, V, False)
    lens = np.array([[g.T, g.T - 40, 5000, 17 * 16, g.T - 3000]], np.int32)
    n_pos = lens.shape[1]
    say(f"causal: visible lengths {lens[0].tolist()}, weak queries")
    Qn = W.make_query_block(g, K, range(n_pos))
    weaken(g, Qn, list(range(n_pos)), 182)
    Qd = to_device(Qn, g.dtype)
    ctx = torch.from_numpy(lens).cuda()
    cap = g.n_level(1)
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, g.p, cap, ctx_len=ctx)
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, ctx_len=ctx)
    torch.cuda.synchronize()
    sel, cnt, stats, gap = (sel.cpu().numpy(), cnt.cpu().numpy(), stats.cpu().numpy(),
                            gap.cpu().numpy())
    Og = from_device(Od, g.dtype)
    assert (cnt >= 0).all()
    assert int(stats[..., 0].max()) > Z.frontier_capacity()
    par = Parity()
    for t in range(n_pos):
        Tt = int(lens[0, t])
        gt = W.replace(g, T=Tt)
        tr = oracle_trees(gt, K[:, :, :Tt], qref, [(0, 0)])[(0, 0)]
        Kf = W.to_float(K[0, 0, :Tt], g.dtype)
        Vf = W.to_float(V[0, 0, :Tt], g.dtype)
        for h in range(g.H_q):
            q = W.to_float(Qn[0, t, h], g.dtype)
            r, o = O.zha_head(tr, q, Kf, Vf, g.p)
            compare_head(par, r, sel[0, t, h], int(cnt[0, t, h]), stats[0, t, h], Og[0, t, h], o,
                         TOL[g.dtype], (t, h), gap_row=gap[0, t, h],
                         attend_set=attend_on(q, Kf, Vf, g.C, Tt))
    say("  " + par.summary())
    par.check()


def test_frontier_slot_wait_gives_up_with_its_own_code(Z, monkeypatch):
    # The wait for a device-memory frontier slot is bounded.  Forced from the
    # host (ZHA_ROUTE_SPILL_WAIT < 0: give up at once, as if every slot were
    # held), each head that needs a slot ends with cnt = ZHA_ROUTE_SLOT_BUSY
    # (-2) and its attention row is NaN, while every other head routes as
    # before; with the default bound the same call routes every head.
    import torch
    g = W.custom("wide-busy", 183, dtype=W.BF16, B=1, H_q=4, H_kv=1, C=16, L=2,
                 T=16 * 16 * 300 + 37, R=1, p=0.99)
    K, V = W.make_kv(g)
    gm, Kd, Vd, tree, qref = build(Z, g, K, V, False)
    n_pos = 4
    Qn = W.make_query_block(g, K, range(n_pos))
    weaken(g, Qn, [1, 3], 183)
    Qd = to_device(Qn, g.dtype)
    cap = g.n_level(1)
    say("frontier slot wait: default bound, then none")
    ref = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    torch.cuda.synchronize()
    monkeypatch.setenv("ZHA_ROUTE_SPILL_WAIT", "-1")
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()
    monkeypatch.delenv("ZHA_ROUTE_SPILL_WAIT")
    again = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    torch.cuda.synchronize()
    rc, rst = ref[1].cpu().numpy(), ref[2].cpu().numpy()
    c, Og = cnt.cpu().numpy(), from_device(Od, g.dtype)
    spilled = rst[..., 0].max(axis=-1) > Z.frontier_capacity()  # [B, n_pos, H_q]
    say(f"  heads needing a slot: {int(spilled.sum())} of {spilled.size}")
    assert spilled.any() and not spilled.all()
    assert (rc >= 0).all()
    assert (c[spilled] == -2).all()
    assert np.isnan(Og[spilled]).all()
    assert np.array_equal(c[~spilled], rc[~spilled])
    s, rs = sel.cpu().numpy(), ref[0].cpu().numpy()
    for b, t, h in zip(*np.nonzero(~spilled)):
        n = int(rc[b, t, h])
        assert np.array_equal(s[b, t, h, :n], rs[b, t, h, :n])
        assert np.isfinite(Og[b, t, h]).all()
    assert np.array_equal(again[1].cpu().numpy(), rc)
