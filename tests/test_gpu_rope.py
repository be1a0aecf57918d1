"""RoPE re-anchoring of the tree build on the GPU against the fp64 oracle.

References are rotated to the last position of each node's span and children
are moved to the parent's reference before a merge (paper §III-B, reference
queries).  Stored trees must equal the oracle's bit for bit; routes and
outputs over those trees must meet the usual parity bar; decode-time updates
must reproduce the build.  The rotations use synthetic RoPE frequencies
theta_k = base^(-2k / dims), full and partial (half the dims rotated).
"""
import sys

import numpy as np
import pytest

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import (TOL, Parity, attend_on, compare_head, from_device, oracle_trees,
                          to_device, tree_mismatch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from hierarchical_tree_indexed_04_amd import zha
    zha.load()
    return zha


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def theta(dims, base):
    return base ** (-np.arange(dims // 2, dtype=np.float64) * 2.0 / dims)


def refs(g, K, R):
    # Non-zero references (a zero reference is unchanged by any rotation).
    q = W.make_qref(W.replace(g, R=max(R, 2)), K)
    return np.ascontiguousarray(q[:, :R])


CASES = [
    # name, dtype, R, rotated dims, base, chunked
    ("bf16-r1-full", W.BF16, 1, 128, 10000.0, False),
    ("bf16-r4-half", W.BF16, 4, 64, 1e6, True),
    ("f32-r2-full", W.F32, 2, 128, 500.0, False),
]


@pytest.mark.parametrize("name,dtype,R,dims,base,chunked", CASES)
def test_rope_tree_routes_and_outputs_match_oracle(Z, name, dtype, R, dims, base, chunked):
    import torch
    say(f"rope {name}: dims {dims}, base {base}, R={R}")
    g = W.custom(f"rope-{name}", 180 + R, dtype=dtype, B=1, H_q=8, H_kv=2,
                 T=8 ** 3 * 3 + 8 * 5 + 3, C=8, L=3, p=0.9, R=R)
    K, V = W.make_kv(g)
    qref = refs(g, K, R)
    th = theta(dims, base)
    rp = Z.rope(dims, th)
    gm = Z.geom(g, Z.ZHA_KV_CHUNKED if chunked else Z.ZHA_KV_SPLIT)
    Kd, Vd = to_device(K, dtype), to_device(V, dtype)
    if chunked:
        Kd, Vd = Z.to_chunked(Kd, Vd, g.C), None
    tree = Z.build(gm, Kd, torch.from_numpy(qref).cuda(), rope=rp)
    n_pos = 6
    Qn = W.make_query_block(g, K, range(n_pos))
    Qd = to_device(Qn, dtype)
    cap = g.n_level(1)
    sel, cnt, stats, gap = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()
    pairs = [(0, h) for h in range(g.H_kv)]
    trees = oracle_trees(g, K, qref, pairs, rope=(dims, th))
    bad_k, bad_b, total = tree_mismatch(Z, g, tree.cpu().numpy(), trees)
    say(f"  tree: {bad_k} k_hat and {bad_b} b_hat mismatches over {total} stored values")
    assert bad_k == 0 and bad_b == 0
    # the rotation matters: the plain tree differs
    plain = oracle_trees(g, K, qref, pairs[:1])[(0, 0)]
    assert not np.array_equal(plain.levels[1].k_store, trees[(0, 0)].levels[1].k_store)
    sel, cnt, stats, gap = (sel.cpu().numpy(), cnt.cpu().numpy(), stats.cpu().numpy(),
                            gap.cpu().numpy())
    Og = from_device(Od, dtype)
    par = Parity()
    for (b, kvh) in pairs:
        Kf, Vf = W.to_float(K[b, kvh], dtype), W.to_float(V[b, kvh], dtype)
        for t in range(n_pos):
            for h in range(kvh * g.G, (kvh + 1) * g.G):
                q = W.to_float(Qn[b, t, h], dtype)
                r, o = O.zha_head(trees[(b, kvh)], q, Kf, Vf, g.p)
                compare_head(par, r, sel[b, t, h], int(cnt[b, t, h]), stats[b, t, h],
                             Og[b, t, h], o, TOL[dtype], (b, t, h), gap_row=gap[b, t, h],
                             attend_set=attend_on(q, Kf, Vf, g.C, g.T))
    say("  " + par.summary())
    par.check()


def test_rope_decode_updates_equal_the_build(Z):
    # Appends across chunk, level-2 and level-3 completions with rotated
    # references: after each update the tree equals the oracle's at that length.
    import torch
    C, L, R, dims = 8, 3, 3, 96
    T0, grow = C ** L - 5, [1, 4, 3, 1, C * C + 2, C ** 3 - 40, 9]
    T_end = T0 + sum(grow)
    say(f"rope decode updates: T {T0} -> {T_end}, R={R}, {dims} rotated dims")
    g = W.custom("rope-dec", 190, dtype=W.BF16, B=1, H_q=4, H_kv=2, T=T_end, C=C, L=L, p=0.9,
                 R=R)
    K, V = W.make_kv(g)
    qref = refs(g, K, R)
    th = theta(dims, 10000.0)
    rp = Z.rope(dims, th)
    Kd = to_device(K, W.BF16)  # capacity T_end; rows past T are never read
    qd = torch.from_numpy(qref).cuda()
    gm = Z.geom(W.replace(g, T=T0), Z.ZHA_KV_SPLIT, T_cap=T_end)
    tb, sb = Z.tree_bytes(gm)
    tree = torch.zeros((tb,), dtype=torch.uint8, device="cuda")
    scratch = torch.empty((sb,), dtype=torch.uint8, device="cuda")
    Z.build(gm, Kd, qd, tree, scratch, rope=rp)
    T = T0
    pairs = [(0, h) for h in range(g.H_kv)]
    for n in grow:
        gm = Z.with_length(gm, T + n)
        Z.tree_update(gm, T, Kd, qd, tree, scratch, rope=rp)
        T += n
        gT = W.replace(g, T=T)
        trees = oracle_trees(gT, K[:, :, :T], qref, pairs, rope=(dims, th))
        bad_k, bad_b, total = tree_mismatch(Z, gT, tree.cpu().numpy(), trees, gm)
        say(f"  T={T}: {bad_k} k_hat and {bad_b} b_hat mismatches over {total}")
        assert bad_k == 0 and bad_b == 0
