"""Causal prefill (every cached token is also a query) on the GPU against the fp64 oracle.

The query at cache position t sees the first t + 1 tokens: it routes through
the nodes complete within them and attends its own partial chunk (paper §V,
Q(T) = T).  The library takes one visible length per position (ctx_len); the
oracle builds the tree of each prefix and routes and attends over it, so the
two share nothing but the inputs.  Covered: a whole prompt as one call (the
many-head router shape and the block attention path), a chunk of positions in
the middle with several sequences of different lengths, the latency router
shape with few positions, and invalid lengths.
"""
import sys

import numpy as np
import pytest

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import TOL, Parity, attend_on, compare_head, from_device, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from hierarchical_tree_indexed_04_amd import zha
    zha.load()
    return zha


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def prefix_trees(g, K, qref, b, kvh, lengths):
    keys = W.to_float(K[b, kvh], g.dtype).astype(np.float64)
    return {n: O.build_tree(keys[:n], qref[kvh], g.C, g.L, g.dtype) for n in sorted(set(lengths))}


def run_prefill(Z, g, ctx, Qn, p, chunked=False, cap=None, qref=None):
    """Routes and attends positions with visible lengths ctx [B, n_pos]; checks every head."""
    import torch
    K, V = W.make_kv(g)
    qref = W.make_qref(g, K) if qref is None else qref
    n_pos = ctx.shape[1]
    gm = Z.geom(g, Z.ZHA_KV_CHUNKED if chunked else Z.ZHA_KV_SPLIT)
    Kd, Vd = to_device(K, g.dtype), to_device(V, g.dtype)
    if chunked:
        Kd, Vd = Z.to_chunked(Kd, Vd, g.C), None
    tree = Z.build(gm, Kd, torch.from_numpy(qref).cuda())
    Qd = to_device(Qn, g.dtype)
    cd = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).cuda()
    cap = max(g.n_level(1), 1) if cap is None else cap
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, p, cap, ctx_len=cd)
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, ctx_len=cd)
    torch.cuda.synchronize()
    sel, cnt, stats, gap = (sel.cpu().numpy(), cnt.cpu().numpy(), stats.cpu().numpy(),
                            gap.cpu().numpy())
    Og = from_device(Od, g.dtype)
    par = Parity()
    bad = []
    for b in range(g.B):
        for kvh in range(g.H_kv):
            lens = [int(x) for x in ctx[b] if 1 <= x <= g.T]
            trees = prefix_trees(g, K, qref, b, kvh, lens)
            Kf, Vf = W.to_float(K[b, kvh], g.dtype), W.to_float(V[b, kvh], g.dtype)
            for t in range(n_pos):
                n = int(ctx[b, t])
                for h in range(kvh * g.G, (kvh + 1) * g.G):
                    if not 1 <= n <= g.T:  # invalid length: failed route, NaN row
                        if cnt[b, t, h] != -1 or not np.isnan(Og[b, t, h]).all():
                            bad.append((b, t, h, n))
                        continue
                    q = W.to_float(Qn[b, t, h], g.dtype)
                    r, o = O.zha_head(trees[n], q, Kf[:n], Vf[:n], p)
                    compare_head(par, r, sel[b, t, h], int(cnt[b, t, h]), stats[b, t, h],
                                 Og[b, t, h], o, TOL[g.dtype], (b, t, h, n),
                                 gap_row=gap[b, t, h],
                                 attend_set=attend_on(q, Kf[:n], Vf[:n], g.C, n))
    say("  " + par.summary())
    assert not bad, bad[:5]
    par.check()
    return par


@pytest.mark.parametrize("dtype,chunked", [(W.BF16, False), (W.BF16, True), (W.F32, False)])
def test_whole_prompt_causal_prefill(Z, dtype, chunked):
    # 1061 positions x 4 heads = 4244 query heads in one call.
    g = W.custom("prefill", 200, dtype=dtype, B=1, H_q=4, H_kv=2, T=8 ** 3 * 2 + 37, C=8, L=3,
                 p=0.9, R=2)
    say(f"causal prefill of {g.T} tokens ({dtype}, {'chunked' if chunked else 'split'} KV)")
    K, _ = W.make_kv(g, want_v=False)
    Qn = W.make_query_block(g, K, range(g.T))
    ctx = np.arange(1, g.T + 1, dtype=np.int32)[None, :]
    run_prefill(Z, g, ctx, Qn, g.p, chunked=chunked)


def test_chunk_of_positions_several_sequences(Z):
    # Two sequences, positions [t0, t0 + 300) of each, with the second sequence
    # seeing fewer tokens (a batch of prompts of different lengths).
    g = W.custom("prefill-b2", 201, dtype=W.BF16, B=2, H_q=8, H_kv=2, T=16 ** 3 + 16 * 9 + 5,
                 C=16, L=3, p=0.95, R=1)
    say("chunked prefill, 2 sequences x 300 positions")
    K, _ = W.make_kv(g, want_v=False)
    Qn = W.make_query_block(g, K, range(300))
    ctx = np.stack([np.arange(3000, 3300), np.arange(700, 1000)]).astype(np.int32) + 1
    run_prefill(Z, g, ctx, Qn, g.p)


def test_few_positions_latency_shape_and_invalid_lengths(Z):
    g = W.custom("prefill-few", 202, dtype=W.BF16, B=2, H_q=4, H_kv=1, T=8 ** 3 + 8 * 3 + 1,
                 C=8, L=3, p=0.9, R=1)
    say("few positions: lengths 1, 7, 8, 9, 64, 512, T and invalid ones")
    K, _ = W.make_kv(g, want_v=False)
    Qn = W.make_query_block(g, K, range(9))
    ctx = np.array([[1, 7, 8, 9, 64, 512, g.T, 0, g.T + 1],
                    [g.T, 511, 513, 2, -5, 100, 65, 63, 300]], dtype=np.int32)
    run_prefill(Z, g, ctx, Qn, g.p)
    # p = 1 keeps every complete chunk of each prefix
    run_prefill(Z, g, ctx, Qn, 1.0)
