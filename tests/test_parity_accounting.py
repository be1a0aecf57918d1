"""The parity accounting of the GPU tests, checked on the CPU with the oracle (no GPU).

compare_head is what decides whether a GPU route and output pass: these cases
feed it oracle results and hand-made "device" results, so that each branch
(exact match, gap comparison, fragile divergence with the output checked over
the device's own set, non-fragile mismatch) is exercised without a GPU.
"""
import math

import numpy as np

import oracle as O
from zha_testutil import GAP_TOL, Parity, attend_on, compare_head


def _case():
    # q = 0 over q_ref = 0: every score ties, so the p = 0.5 cut of 8 equal
    # candidates keeps exactly half of the mass (fragile by the mass margin).
    C, L, d = 4, 2, 8
    T = C ** L * 2
    g = np.random.default_rng(700)
    K = g.standard_normal((T, d))
    V = g.standard_normal((T, d))
    tree = O.build_tree(K, np.zeros((1, d)), C, L, O.F64)
    q = np.zeros(d)
    r, o = O.zha_head(tree, q, K, V, 0.5)
    return C, T, K, V, q, r, o


def _device_view(r, cap):
    sel = np.full(cap, -1, np.int32)
    sel[:len(r.S1)] = r.S1
    stats = np.array([[r.K[i], len(r.S[i])] for i in range(len(r.S))], np.int32)
    gap = np.array([math.inf if math.isinf(x) else x for x in r.gap], np.float32)
    return sel, stats, gap


def test_exact_route_compares_gaps_and_output():
    C, T, K, V, q, r, o = _case()
    sel, stats, gap = _device_view(r, 64)
    par = Parity()
    compare_head(par, r, sel, len(r.S1), stats, o.astype(np.float32), o, 2e-2, "a", gap_row=gap)
    assert par.exact == 1 and par.out_checked == 1 and not par.gap_bad
    bad = gap.copy()
    bad[np.isfinite(bad)] += 2 * GAP_TOL
    assert np.isfinite(gap).all()
    inf_claimed = gap.copy()  # the device reports the whole frontier kept where it was cut
    inf_claimed[0] = math.inf
    for row in (bad, inf_claimed):
        p2 = Parity()
        compare_head(p2, r, sel, len(r.S1), stats, o, o, 2e-2, "b", gap_row=row)
        assert p2.gap_bad


def test_fragile_divergence_checks_output_over_the_device_set():
    C, T, K, V, q, r, o = _case()
    assert any(r.fragile)
    sel, stats, gap = _device_view(r, 64)
    # the device kept other ids at the fragile level-1 cut (same count)
    other = np.setdiff1d(np.arange(T // C), r.S1)[:len(r.S1)].astype(np.int32)
    sel2 = sel.copy()
    sel2[:len(other)] = np.sort(other)
    want = O.attend(q, K, V, O.token_set(sel2[:len(other)], C, T))
    par = Parity()
    compare_head(par, r, sel2, len(other), stats, want.astype(np.float32), o, 2e-2, "c",
                 gap_row=gap, attend_set=attend_on(q, K, V, C, T))
    assert par.fragile_diverged == 1 and par.out_checked == 1 and not par.out_bad
    # a wrong output on that set is caught
    par = Parity()
    compare_head(par, r, sel2, len(other), stats, (want + 1.0).astype(np.float32), o, 2e-2, "d",
                 gap_row=gap, attend_set=attend_on(q, K, V, C, T))
    assert par.fragile_diverged == 1 and par.out_bad


def test_non_fragile_divergence_is_a_mismatch():
    C, L, d = 4, 2, 8
    T = C ** L * 2
    g = np.random.default_rng(701)
    K = 2 * g.standard_normal((T, d))
    V = g.standard_normal((T, d))
    tree = O.build_tree(K, np.zeros((1, d)), C, L, O.F64)
    q = 3 * K[5]
    r, o = O.zha_head(tree, q, K, V, 0.9)
    assert not any(r.fragile)
    sel, stats, gap = _device_view(r, 64)
    sel[0] = (sel[0] + 1) % (T // C)
    par = Parity()
    compare_head(par, r, sel, len(r.S1), stats, o, o, 2e-2, "e", gap_row=gap)
    assert par.mismatched and par.exact == 0
