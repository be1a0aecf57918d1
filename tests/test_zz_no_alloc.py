"""zha_attn_noalloc (the fixed-buffer variant of zha_attn) against zha_attn (GPU).

Two calls in a row through the C ABI, the second with a smaller input (fewer
sequences, positions and tokens, another chunk size), each compared with
zha_attn on the same routed inputs: the two entry points run the same kernels
on the same plan, so the outputs must be identical bit for bit; the second
call also finds the first call's contents in the shared buffer.  A third call
with a ragged visible length per position and failed routes (NaN rows) covers
the remaining input paths.
"""
import sys

import numpy as np
import pytest

from hierarchical_tree_indexed_04_amd import workload as W
from zha_testutil import to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _routed(Z, g, n_pos, seed_steps, ctx=None):
    import torch
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(seed_steps, seed_steps + n_pos))
    gm = Z.geom(g)
    Kd, Vd, Qd = to_device(K, g.dtype), to_device(V, g.dtype), to_device(Qn, g.dtype)
    tree = Z.build(gm, Kd, torch.zeros((g.H_kv, 1, g.d), device="cuda"))
    cap = g.n_level(1)
    sel, cnt, _, _ = Z.route(gm, tree, Qd, n_pos, g.p, cap, ctx_len=ctx)
    return gm, Kd, Vd, Qd, sel, cnt, cap


def _same(a, b):
    import torch
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 \
        else torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_noalloc_attention_equals_zha_attn_on_two_calls_in_a_row():
    import torch
    from hierarchical_tree_indexed_04_amd import zha as Z
    Z.load()
    big = W.custom("noalloc-a", 160, dtype=W.BF16, B=4, H_q=32, H_kv=4, T=8 ** 5 + 8 * 9 + 3,
                   C=8, L=5, p=0.95)
    small = W.custom("noalloc-b", 161, dtype=W.BF16, B=1, H_q=8, H_kv=2, T=16 ** 3 + 5, C=16,
                     L=3, p=0.9)
    for name, g, n_pos in (("first", big, 2), ("second, smaller", small, 1)):
        gm, Kd, Vd, Qd, sel, cnt, cap = _routed(Z, g, n_pos, 0)
        n_heads = g.B * n_pos * g.H_q
        say(f"{name} call: {n_heads} query heads, T={g.T}, C={g.C}")
        ref = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap)
        out = torch.full_like(ref, float("nan"))
        got = Z.attn_noalloc(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, O=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(ref.float()).all()
        assert _same(got, ref), float((got.float() - ref.float()).abs().max())


def test_noalloc_attention_ragged_lengths_and_failed_routes():
    import torch
    from hierarchical_tree_indexed_04_amd import zha as Z
    Z.load()
    g = W.custom("noalloc-c", 162, dtype=W.F32, B=2, H_q=4, H_kv=2, T=4 ** 5 * 3 + 21, C=4, L=5,
                 p=0.9)
    n_pos = 5
    lens = np.array([[g.T, 1, 3, 4 ** 3 + 2, g.T - 7], [5, g.T, 200, 17, 1024]], np.int32)
    ctx = torch.from_numpy(lens).cuda()
    gm, Kd, Vd, Qd, sel, cnt, cap = _routed(Z, g, n_pos, 3, ctx=ctx)
    cnt[0, 2, 1] = -1          # a failed route
    cnt[1, 4, 0] = cap + 1     # more chunks than cap
    say(f"ragged visible lengths {lens.tolist()}, two failed rows, fp32")
    ref = Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, ctx_len=ctx)
    got = Z.attn_noalloc(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, ctx_len=ctx)
    torch.cuda.synchronize()
    assert torch.isnan(got[0, 2, 1]).all() and torch.isnan(got[1, 4, 0]).all()
    assert _same(got, ref)
