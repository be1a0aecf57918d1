"""The MI355X roofline model of decode latency (host arithmetic, no GPU).

Pins: the two forms the paper gives for the amortized decode tree cost agree;
eq. (4)'s worker-wave term; the dense work and byte counts against a direct
count; the model's split count J(T) against the library's own plan (read back
through the C ABI's scratch-size query); the fit recovers parameters from data
the model generated; and, on the committed crossover measurement, the model
calibrated on four contexts predicts the other three and the crossover.
"""
import json
import math
import os

import pytest

from hierarchical_tree_indexed_04_amd import roofline as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("C,L", [(2, 2), (8, 6), (16, 3), (32, 4), (4, 9)])
def test_tree_decode_cost_sum_equals_closed_form(C, L):
    a = M.t_tree_decode_sum(9.6e-6, 5.1e-6, C, L)
    b = M.t_tree_decode_closed(9.6e-6, 5.1e-6, C, L)
    assert abs(a - b) <= 1e-12 * a


def test_worker_wave_term_and_max():
    # 300 tiles on 256 units, one resident each: two waves of tau.
    assert M.phi(0, 1, 0, 1, 2.0, 300, 256, 1) == 4.0
    assert M.phi(0, 1, 0, 1, 2.0, 256, 256, 1) == 2.0
    assert M.phi(10.0, 2.0, 0, 1, 1.0, 1, 256, 1) == 5.0  # compute-bound
    assert M.phi(0, 1, 12.0, 4.0, 1.0, 1, 256, 1) == 3.0  # memory-bound


def test_dense_counts_match_a_direct_count():
    w = M.Workload(B=2, H_q=8, H_kv=2, d=16, T=100, C=4, L=2)
    x = M.dense_terms(w)
    J = x["J"]
    n_qtiles = sum(1 for b in range(w.B) for kvh in range(w.H_kv))  # G = 4 rows: one tile each
    kv = sum(w.s * w.d * 2 for _tile in range(n_qtiles) for _t in range(w.T))
    per_head = sum(w.s * w.d + w.s_acc * J * (w.d + 2) for _h in range(w.B * w.H_q))
    assert x["n_qtiles"] == n_qtiles and x["bytes_partial"] == kv + per_head
    assert x["flops_partial"] == sum(2 * 2 * w.d for _h in range(w.B * w.H_q) for _t in range(w.T))


@pytest.mark.parametrize("T,B", [(4096, 8), (65536, 8), (262144, 8), (1 << 20, 1), (3000, 1)])
def test_split_count_matches_the_library_plan(T, B):
    from hierarchical_tree_indexed_04_amd import zha as Z
    w = M.Workload(B=B, H_q=32, H_kv=4, d=128, T=T, C=8, L=3)
    gm = Z.Geom(B, 32, 4, 128, T, 8, 3, 1, Z.ZHA_BF16, Z.ZHA_KV_SPLIT, 0)
    J = M.dense_splits(w)
    lib = Z.dense_scratch_bytes(gm, 1)
    assert lib == (0 if J == 1 else B * 32 * J * (128 + 2) * 4)


def test_fit_recovers_parameters_of_model_generated_points():
    true = M.Calibration(lam=4e-6, bw_stream=6e12, bw_gather=5e12, tau_level=0.7e-6,
                         tau_log=1.1e-6, tau_attn=9e-6, tau_dense=15e-6,
                         tau_merge_attn=4e-6, tau_merge_dense=5e-6)
    pts = []
    for T, L, ks, tok, union in [(4096, 4, [9, 8, 8, 1], 50, 6e6), (16384, 4, [52, 9, 8, 4], 300, 4e7),
                                 (65536, 5, [309, 52, 9, 8, 2], 2000, 2.2e8),
                                 (262144, 6, [307, 52, 9, 8, 8, 1], 1960, 2.5e8),
                                 (1 << 20, 6, [900, 120, 30, 8, 8, 4], 3000, 9e8)]:
        w = M.Workload(B=8, H_q=32, H_kv=4, d=128, T=T, C=8, L=L)
        z = M.t_zha(w, ks, tok, union, cal=true)
        d = M.t_dense(w, cal=true)
        pts.append(M.Point(w=w, K_levels=ks, tokens_per_head=tok, union_bytes=union,
                           route=z["route"], attn=z["attn"], dense=d["total"]))
    got = M.fit(pts, lam=true.lam, tau_merge_attn=true.tau_merge_attn,
                tau_merge_dense=true.tau_merge_dense)
    for name in ("tau_level", "tau_log", "tau_attn", "bw_gather", "bw_stream", "tau_dense"):
        assert math.isclose(getattr(got, name), getattr(true, name), rel_tol=1e-6), name


def test_committed_crossover_is_predicted_within_its_calibration():
    path = os.path.join(ROOT, "profiles", "crossover_deep-decode.json")
    rec = json.loads(open(path).read().strip().splitlines()[-1])
    pts = M.points_from_crossover(rec)
    train_T = (4096, 16384, 65536, 262144)
    cal = M.fit([p for p in pts if p.w.T in train_T])
    for p in pts:
        if p.w.T in train_T:
            continue
        q = M.predict(p, cal)
        assert abs(q["zha"] / (p.route + p.attn) - 1) < 0.15, p.w.T
        assert abs(q["dense"] / p.dense - 1) < 0.25, p.w.T
    srt = sorted(pts, key=lambda p: p.w.T)
    measured = next(srt[k].w.T for k in range(len(srt))
                    if all(p.route + p.attn < p.dense for p in srt[k:]))
    assert M.crossover(pts, cal) == measured
