"""Balanced attention where the call's token count reaches 2^31 (GPU).

2048 query heads (the most the balanced split takes) each keep every chunk of
a 2^20-token cache, so the heads' attended tokens laid end to end number
exactly 2^31: a 32-bit prefix of per-head counts would wrap there.  With p = 1
the attended set is the whole cache (the sink lies in chunk 0), so each output
is dense attention; sampled heads are checked against the oracle's dense
attention, and every row must be finite.  d = 64 keeps the 2^31 token rows to
about 550 GB of K/V reads (mostly cache hits: the heads of a KV group read the
same rows).
"""
import sys

import numpy as np
import pytest

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import TOL, from_device, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_balanced_attention_total_of_2_pow_31_tokens():
    import torch
    from hierarchical_tree_indexed_04_amd import zha as Z
    Z.load()
    T, C = 1 << 20, 32
    g = W.custom("attn-2g", 150, dtype=W.BF16, B=1, H_q=16, H_kv=2, d=64, T=T, C=C, L=2, p=1.0)
    n_pos = 128
    n_heads = g.B * n_pos * g.H_q
    n1 = T // C
    assert n_heads == 2048 and n_heads * T == 1 << 31
    say(f"balanced attention: {n_heads} heads x {T} tokens = 2^31 positions, d = {g.d}")
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(n_pos))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    cap = n1
    sel = torch.arange(n1, dtype=torch.int32, device="cuda").repeat(n_heads, 1)
    sel = sel.reshape(g.B, n_pos, g.H_q, cap)
    cnt = torch.full((g.B, n_pos, g.H_q), n1, dtype=torch.int32, device="cuda")
    Od = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
    torch.cuda.synchronize()
    say("  attention done")
    del sel
    Og = from_device(Od, g.dtype)
    assert np.isfinite(Og).all()
    rng = np.random.default_rng(150)
    worst = 0.0
    Kf = [W.to_float(K[0, h], g.dtype) for h in range(g.H_kv)]
    Vf = [W.to_float(V[0, h], g.dtype) for h in range(g.H_kv)]
    # the first and last head of the call, plus random ones
    picks = [(0, 0), (n_pos - 1, g.H_q - 1)] + [
        (int(rng.integers(n_pos)), int(rng.integers(g.H_q))) for _ in range(30)]
    for t, h in picks:
        o = O.dense(W.to_float(Qn[0, t, h], g.dtype), Kf[h // g.G], Vf[h // g.G])
        worst = max(worst, float(np.abs(Og[0, t, h] - o).max()))
    say(f"  max abs err {worst:.3g} over {len(picks)} sampled heads")
    assert worst <= TOL[g.dtype]
