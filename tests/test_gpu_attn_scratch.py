"""zha_attn with scratch buffers holding leftover data (GPU).

The caller's scratch is not cleared between calls, so on entry it may hold
anything: an earlier call's plan and partials, or data of other tensors the
allocator handed the memory to before (chunk-id lists, whose int32 pairs are
small integers).  Outputs must not depend on it: every fill below must give
the same bits as a zero-filled scratch, twice in a row, and the zero-filled
run must match the oracle.
"""
import sys

import numpy as np
import pytest

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import TOL, from_device, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Z():
    from hierarchical_tree_indexed_04_amd import zha
    zha.load()
    return zha


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_split_merge_ignores_leftover_scratch(Z):
    import torch
    say("zha_attn: scratch words holding small-integer pairs, ones, earlier counters")
    g = W.custom("a-scratch", 181, dtype=W.BF16, B=2, H_q=16, H_kv=2, T=8 ** 5 + 77, C=8, L=5,
                 p=0.95)
    K, V = W.make_kv(g)
    n_pos = 2
    Qn = W.make_query_block(g, K, range(n_pos))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    sel, cnt, _, _ = Z.route(gm, tree, Qd, n_pos, g.p, cap)
    nbytes = Z.attn_scratch_bytes(gm, n_pos, cap)
    words = (nbytes + 7) // 8
    i = torch.arange(words, dtype=torch.int64, device="cuda")
    fills = {
        "zeros": torch.zeros(words, dtype=torch.int64, device="cuda"),
        # int32 pairs (k, k) and (k, k + 1) for small k: what a freed chunk-id list leaves
        "id pairs": ((i % 4096) << 32) | (i % 4096),
        "id pairs +1": ((i % 512) << 32) | ((i % 512) + 1),
        "ones": torch.full((words,), -1, dtype=torch.int64, device="cuda"),
    }
    outs = {}
    for name, f in fills.items():
        scr = f.clone().view(torch.uint8)[:nbytes]
        outs[name] = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, scratch=scr)
        torch.cuda.synchronize()
        # a second call over the first one's counters
        outs[name + ", again"] = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, scratch=scr)
    torch.cuda.synchronize()
    ref = outs["zeros"].view(torch.int16).cpu().numpy()
    for name, o in outs.items():
        same = np.array_equal(o.view(torch.int16).cpu().numpy(), ref)
        say(f"  {name}: {'same bits' if same else 'DIFFERENT'}")
        assert same, name
    # The reference run against the oracle, for every head with a route.
    Og = from_device(outs["zeros"], g.dtype)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    split_heads = 0
    worst = 0.0
    for b in range(g.B):
        for kvh in range(g.H_kv):
            Kf, Vf = W.to_float(K[b, kvh], g.dtype), W.to_float(V[b, kvh], g.dtype)
            for t in range(n_pos):
                for h in range(kvh * g.G, (kvh + 1) * g.G):
                    c = int(cnt_h[b, t, h])
                    assert 0 <= c <= cap
                    toks = O.token_set(sel_h[b, t, h, :c], g.C, g.T)
                    split_heads += len(toks) > 64
                    q = W.to_float(Qn[b, t, h], g.dtype)
                    err = float(np.max(np.abs(Og[b, t, h] - O.attend(q, Kf, Vf, toks))))
                    worst = max(worst, err)
                    assert err <= TOL[g.dtype], (b, t, h, err)
    say(f"  {split_heads} heads attend more than one 64-token range; max |err| {worst:.3g}")
    assert split_heads > 0
