"""The bench's attention byte accounting against brute-force token sets (no GPU).

bench.step_bytes gives the bytes the sparse gather of one decode step must
move: the K and V rows of every token some query head of a KV group attends,
counted once per group (the union of the heads' sets I(q) = {0} U selected
chunks' tokens U C_cur, summary page "Routing"), and, per head, the same rows
counted separately.  It counts with a closed form (chunks x C, plus the tail,
plus the sink unless chunk 0 is selected); here the sets are built token by
token with the oracle's token_set and their unions counted directly, on
random chunk lists that include and exclude chunk 0, empty lists, a ragged
tail and T < C.
"""
import numpy as np
import pytest

import bench
import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W


def _random_routes(g, rng):
    n1 = g.n_level(1)
    cap = max(n1, 1)
    sel = np.full((g.B, 1, g.H_q, cap), -1, np.int32)
    cnt = np.zeros((g.B, 1, g.H_q), np.int32)
    for b in range(g.B):
        for h in range(g.H_q):
            k = int(rng.integers(0, n1 + 1))
            ids = np.sort(rng.choice(n1, k, replace=False)).astype(np.int32) if n1 else []
            if n1 and h % 3 == 0 and 0 not in ids:  # chunk 0 selected: the sink lies in it
                ids = np.sort(np.append(ids, 0)).astype(np.int32)
            cnt[b, 0, h] = len(ids)
            sel[b, 0, h, :len(ids)] = ids
    stats = rng.integers(1, 9, size=(g.B, 1, g.H_q, g.L, 2)).astype(np.int32)
    return sel, cnt, stats


@pytest.mark.parametrize("T,C", [(8 ** 3 + 8 * 5 + 3, 8), (16 * 40, 16), (5, 8)])
def test_attention_bytes_equal_brute_force_unions(T, C):
    g = W.custom("acct", 950, dtype=W.BF16, B=2, H_q=6, H_kv=2, d=32, T=T, C=C, L=2)
    rng = np.random.default_rng(T)
    sel, cnt, stats = _random_routes(g, rng)
    got = bench.step_bytes(g, sel, cnt, stats)
    row = 2 * g.d * g.elem_bytes  # one token's K and V rows
    union_toks = per_head_toks = 0
    for b in range(g.B):
        for kvh in range(g.H_kv):
            group = set()
            for h in range(kvh * g.G, (kvh + 1) * g.G):
                toks = O.token_set(sel[b, 0, h, :cnt[b, 0, h]], g.C, g.T)
                assert toks.size == np.unique(toks).size and toks.max() < g.T
                per_head_toks += toks.size
                group.update(int(t) for t in toks)
            union_toks += len(group)
    io = g.B * g.H_q * 2 * g.d * g.elem_bytes + int(cnt.sum()) * 4  # q, o, chunk lists
    assert got["attn_union"] == union_toks * row + io
    assert got["attn_per_head"] == per_head_toks * row + io
    assert got["attn_union"] <= got["attn_per_head"]
