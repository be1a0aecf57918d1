"""zha_route_attn (routing and attention in one call) against the oracle and
against zha_route followed by zha_attn (GPU).

The fused launch must route every head exactly as zha_route does (sel, cnt,
level statistics and gaps bit for bit) and attend the same tokens; outputs
are checked against oracle attention over the routed set within the parity
tolerance, and against the separate calls' outputs (split points differ, so
the fp32 sums may differ in the last bits).  Calls run back to back, so the
launch's device-side queue and counters must come back cleared every time.
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


def run_fused(Z, g, steps, pairs=None, ctx=None, weak=(), chunked=False, reps=1):
    import torch
    pairs = pairs if pairs is not None else [(b, h) for b in range(g.B) for h in range(g.H_kv)]
    K, V = W.make_kv(g, slices=pairs)
    qref = W.make_qref(g, K)
    n_pos = len(steps)
    Qn = W.make_query_block(g, K, steps)
    if weak:
        rng = np.random.default_rng(77)
        w = rng.standard_normal((g.B, len(weak), g.H_q, g.d)).astype(np.float32) * np.float32(0.05)
        Qn[:, list(weak)] = W.f32_to_bf16_bits(w) if g.dtype == W.BF16 else w
    gm = Z.geom(g, Z.ZHA_KV_CHUNKED if chunked else Z.ZHA_KV_SPLIT)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    if chunked:
        Kd, Vd = Z.to_chunked(Kd, Vd, g.C), None
    tree = Z.build(gm, Kd, torch.from_numpy(qref).cuda())
    cap = g.n_level(1)
    cd = None if ctx is None else torch.from_numpy(np.ascontiguousarray(ctx, np.int32)).cuda()
    def filled():
        # Entries a call leaves unwritten (a failed position's statistics and
        # gaps) keep these values, so both entry points must leave the same ones.
        return (torch.full((g.B, n_pos, g.H_q, cap), -7, dtype=torch.int32, device="cuda"),
                torch.full((g.B, n_pos, g.H_q), -7, dtype=torch.int32, device="cuda"),
                torch.full((g.B, n_pos, g.H_q, g.L, 2), -7, dtype=torch.int32, device="cuda"),
                torch.full((g.B, n_pos, g.H_q, g.L), 1234.5, dtype=torch.float32, device="cuda"))

    # the separate calls, then the fused one (several times: counters must reset)
    s_sel, s_cnt, s_st, s_gap = Z.route(gm, tree, Qd, n_pos, g.p, cap, ctx_len=cd, out=filled())
    s_O = Z.attn(gm, Qd, n_pos, Kd, Vd, s_sel, s_cnt, cap, ctx_len=cd)
    outs = [Z.route_attn(gm, tree, Qd, n_pos, g.p, Kd, Vd, cap, ctx_len=cd, out=filled())
            for _ in range(reps)]
    torch.cuda.synchronize()
    s_cnt_h = s_cnt.cpu().numpy()
    for sel, cnt, st, gap, Od in outs:
        assert torch.equal(cnt.cpu(), s_cnt.cpu())
        assert torch.equal(st.cpu(), s_st.cpu())
        assert torch.equal(gap.cpu(), s_gap.cpu())
        sh, ssh = sel.cpu().numpy(), s_sel.cpu().numpy()
        for idx in np.ndindex(s_cnt_h.shape):
            n = min(max(int(s_cnt_h[idx]), 0), cap)
            assert np.array_equal(sh[idx][:n], ssh[idx][:n]), idx
        a, b = from_device(Od, g.dtype), from_device(s_O, g.dtype)
        fin = np.isfinite(b)
        assert np.array_equal(np.isnan(a), np.isnan(b))
        diff = float(np.abs(a[fin] - b[fin]).max()) if fin.any() else 0.0
        say(f"  fused vs separate: routes identical, max |O diff| {diff:.3g}")
        assert diff <= TOL[g.dtype]
    sel, cnt, st, gap, Od = outs[-1]
    sel, cnt, st, gap = sel.cpu().numpy(), cnt.cpu().numpy(), st.cpu().numpy(), gap.cpu().numpy()
    Og = from_device(Od, g.dtype)
    trees = oracle_trees(g, K, qref, pairs)
    par = Parity()
    for (b, kvh) in pairs:
        Kf, Vf = W.to_float(K[b, kvh], g.dtype), W.to_float(V[b, kvh], g.dtype)
        for t in range(n_pos):
            Tt = g.T if ctx is None else int(ctx[b, t])
            for h in range(kvh * g.G, (kvh + 1) * g.G):
                if not 1 <= Tt <= g.T:
                    assert cnt[b, t, h] == -1 and np.isnan(Og[b, t, h]).all()
                    continue
                tree_t = trees[(b, kvh)] if Tt == g.T else oracle_trees(
                    W.replace(g, T=Tt), K[:, :, :Tt], qref, [(b, kvh)])[(b, kvh)]
                q = W.to_float(Qn[b, t, h], g.dtype)
                r, o = O.zha_head(tree_t, q, Kf[:Tt], Vf[:Tt], g.p)
                compare_head(par, r, sel[b, t, h], int(cnt[b, t, h]), st[b, t, h], Og[b, t, h], o,
                             TOL[g.dtype], (b, t, h), gap_row=gap[b, t, h],
                             attend_set=attend_on(q, Kf[:Tt], Vf[:Tt], g.C, Tt))
    say("  " + par.summary())
    par.check()
    return par


def test_fused_tiny_fp32(Z):
    say("fused: config 1, fp32, 64 queries")
    run_fused(Z, W.CONFIGS[1], range(64), reps=3)


def test_fused_gqa_128k(Z):
    say("fused: config 2, 8 steps x 32 heads")
    run_fused(Z, W.CONFIGS[2], range(8))


def test_fused_deep_256k_full_batch(Z):
    g = W.CONFIGS[3]
    say("fused: config 3 at full size, 2 steps of 8 sequences x 32 heads (the bench's call)")
    K, V = W.make_kv(g)
    import torch
    gm = Z.geom(g)
    Kd, Vd = to_device(K, g.dtype), to_device(V, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    par = Parity()
    trees = {}
    for s in range(2):
        Qn = W.make_query_block(g, K, range(s, s + 1))
        Qd = to_device(Qn, g.dtype)
        s_sel, s_cnt, s_st, s_gap = Z.route(gm, tree, Qd, 1, g.p, cap)
        s_O = Z.attn(gm, Qd, 1, Kd, Vd, s_sel, s_cnt, cap)
        sel, cnt, st, gap, Od = Z.route_attn(gm, tree, Qd, 1, g.p, Kd, Vd, cap)
        torch.cuda.synchronize()
        assert torch.equal(cnt.cpu(), s_cnt.cpu()) and torch.equal(st.cpu(), s_st.cpu())
        assert torch.equal(gap.cpu(), s_gap.cpu())
        a, b = from_device(Od, g.dtype), from_device(s_O, g.dtype)
        diff = float(np.abs(a - b).max())
        say(f"  step {s}: routes identical, max |O diff| vs separate calls {diff:.3g}")
        assert diff <= TOL[g.dtype]
        sel, cnt, st, gap = sel.cpu().numpy(), cnt.cpu().numpy(), st.cpu().numpy(), gap.cpu().numpy()
        for b_ in (0, 7):
            for h in range(g.H_q):
                kvh = h // g.G
                if (b_, kvh) not in trees:
                    trees[(b_, kvh)] = (O.build_tree(W.to_float(K[b_, kvh], g.dtype).astype(np.float64),
                                                     np.zeros((1, g.d)), g.C, g.L, g.dtype),
                                        W.to_float(K[b_, kvh], g.dtype), W.to_float(V[b_, kvh], g.dtype))
                tr, Kf, Vf = trees[(b_, kvh)]
                q = W.to_float(Qn[b_, 0, h], g.dtype)
                r, o = O.zha_head(tr, q, Kf, Vf, g.p)
                compare_head(par, r, sel[b_, 0, h], int(cnt[b_, 0, h]), st[b_, 0, h], a[b_, 0, h], o,
                             TOL[g.dtype], (s, b_, h), gap_row=gap[b_, 0, h],
                             attend_set=attend_on(q, Kf, Vf, g.C, g.T))
    say("  " + par.summary())
    par.check()


@pytest.mark.parametrize("chunked", [False, True])
def test_fused_ragged_orphans_fp32(Z, chunked):
    say(f"fused: ragged T with orphans at every level, fp32, {'chunked' if chunked else 'split'} KV")
    g = W.custom("f-ragged", 171, dtype=W.F32, B=2, H_q=2, H_kv=1, T=4 ** 4 * 3 + 4 ** 3 * 2 + 4 * 3 + 2,
                 C=4, L=4, p=0.8)
    run_fused(Z, g, range(10), chunked=chunked, reps=2)


def test_fused_device_memory_frontier(Z):
    # n_1 > 4096 and weak queries at p = 0.99: those heads outgrow the on-chip
    # frontier and are routed again with a device-memory frontier inside the
    # fused launch; their attention covers nearly the whole cache (many pieces).
    say("fused: weak queries outgrow the on-chip frontier (device-memory frontier), many pieces")
    g = W.custom("f-wide", 172, dtype=W.BF16, B=2, H_q=4, H_kv=1, C=16, L=2, T=16 * 16 * 300 + 37,
                 p=0.99)
    run_fused(Z, g, range(3), weak=(0, 2))


def test_fused_causal_lengths_and_failed_rows(Z):
    say("fused: a visible length per position (causal prefill), invalid lengths give NaN rows")
    g = W.custom("f-causal", 173, dtype=W.BF16, B=2, H_q=8, H_kv=2, T=8 ** 4 + 8 * 3 + 5, C=8, L=4,
                 p=0.9)
    ctx = np.array([[g.T, 1, 9, 8 ** 3 + 3, 0, g.T - 100], [5000, g.T, 64, 2, g.T + 1, 777]],
                   np.int32)
    run_fused(Z, g, range(6), ctx=ctx, reps=2)


@pytest.mark.parametrize("name,kw", [
    ("R=3", dict(dtype=W.BF16, B=1, H_q=4, H_kv=2, T=8 ** 3 * 3 + 40, C=8, L=3, p=0.9, R=3)),
    ("C=6", dict(dtype=W.BF16, B=1, H_q=8, H_kv=2, T=6 ** 4 * 2 + 6 * 5 + 4, C=6, L=4, p=0.9)),
    ("p=1", dict(dtype=W.BF16, B=1, H_q=4, H_kv=1, T=16 ** 3 + 5, C=16, L=3, p=1.0)),
])
def test_fused_entry_falls_back_to_separate_calls(Z, name, kw):
    say(f"zha_route_attn where the single launch does not apply ({name}): route, then attention")
    g = W.custom(f"f-fb-{name}", 174, **kw)
    run_fused(Z, g, range(3))


@pytest.mark.parametrize("n_pos", [64, 65])
def test_fused_at_the_head_limit(Z, n_pos):
    """2048 query heads (64 positions x 32 heads: the most one launch takes, its
    queue nearly full of pieces) and 2080 (past the limit: route, then
    attention): routes bit for bit equal to zha_route's, outputs to zha_attn's
    within the parity tolerance, and sampled positions against the oracle."""
    import torch
    g = W.custom("f-limit", 175, dtype=W.BF16, B=1, H_q=32, H_kv=4, T=8 ** 5 + 21, C=8, L=5,
                 p=0.95)
    say(f"zha_route_attn with {n_pos * g.H_q} query heads ({n_pos} positions x {g.H_q} heads)")
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(n_pos))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    s_sel, s_cnt, s_st, s_gap = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    s_O = Z.attn(gm, Qd, n_pos, Kd, Vd, s_sel, s_cnt, cap)
    for rep in range(2):
        sel, cnt, st, gap, Od = Z.route_attn(gm, tree, Qd, n_pos, g.p, Kd, Vd, cap)
        torch.cuda.synchronize()
        assert torch.equal(cnt.cpu(), s_cnt.cpu()) and torch.equal(st.cpu(), s_st.cpu())
        assert torch.equal(gap.cpu(), s_gap.cpu())
        ch, sh = cnt.cpu().numpy(), sel.cpu().numpy()
        ssh = s_sel.cpu().numpy()
        for idx in np.ndindex(ch.shape):
            assert np.array_equal(sh[idx][:ch[idx]], ssh[idx][:ch[idx]]), idx
        a, b = from_device(Od, g.dtype), from_device(s_O, g.dtype)
        diff = float(np.abs(a - b).max())
        say(f"  call {rep}: routes identical, max |O diff| vs separate calls {diff:.3g}")
        assert diff <= TOL[g.dtype]
    trees = oracle_trees(g, K, np.zeros((g.H_kv, 1, g.d)), [(0, kvh) for kvh in range(g.H_kv)])
    sel, cnt, st, gap = sel.cpu().numpy(), cnt.cpu().numpy(), st.cpu().numpy(), gap.cpu().numpy()
    par = Parity()
    for kvh in range(g.H_kv):
        Kf, Vf = W.to_float(K[0, kvh], g.dtype), W.to_float(V[0, kvh], g.dtype)
        for t in (0, n_pos // 2, n_pos - 1):
            for h in range(kvh * g.G, (kvh + 1) * g.G):
                q = W.to_float(Qn[0, t, h], g.dtype)
                r, o = O.zha_head(trees[(0, kvh)], q, Kf, Vf, g.p)
                compare_head(par, r, sel[0, t, h], int(cnt[0, t, h]), st[0, t, h], a[0, t, h], o,
                             TOL[g.dtype], (t, h), gap_row=gap[0, t, h],
                             attend_set=attend_on(q, Kf, Vf, g.C, g.T))
    say("  " + par.summary())
    par.check()
