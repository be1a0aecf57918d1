"""Roofline latency model of ZHA decode and of dense decode, instantiated for MI355X.

Follows "Subquadratic Attention with a Hierarchical Tree-Structured Indexer" §V-A
(eq. (3): t_ZHA = t_tree + lambda_A + Phi_attn + sum over levels of
[lambda_l + Phi_routing,l + Phi_scan,l]; eq. (4): each stage is the largest of
its compute time, its memory time and its worker-wave time) and App. D (D-A the
dense model, D-B1 worker-aware execution with the per-level work and byte
counts, D-B2 tree construction and its amortized decode cost).

The pages model an H100 and separate routing, scan and attention kernels.  The
instance here describes this library's kernels on MI355X:

* one router launch walks every level (so the per-level launch terms collapse
  into one lambda and the scan runs inside the routing workgroup: its frontier
  scores never leave LDS, bytes_scan = 0); one workgroup per query head, so the
  router's worker-wave term is a per-level latency tau_route(K_l) =
  tau_level + tau_log * log2(K_l) for the mean frontier K_l: a level's rows
  load in one round (up to 2,048 in flight per workgroup), and the cut's
  reductions, histogram and radix passes deepen with the frontier;
* attention is one balanced split-KV launch over ZHA_ATTN_BLOCKS workgroups
  plus a merge launch; its memory term moves the union of the attended K/V rows
  over the G heads of each group (the paper's "grouped union") at the gather
  bandwidth of leaf-chunk pieces;
* dense decode is the matrix-core kernel: N_qtiles = B H_kv ceil(Q G / 16)
  16-row query tiles per cache, J(T) splits each, then a merge launch.

Hardware limits are MI355X's published figures; the effective rates (stream
and gather bandwidth, per-launch overhead, per-block latencies) are calibrated
from measurements by ``fit``.  Host-only arithmetic: nothing here runs on the
GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np


@dataclass(frozen=True)
class Hardware:
    """MI355X full-device limits (published figures)."""
    n_cu: int = 256
    hbm_bw: float = 8.0e12       # bytes/s
    mfma_bf16: float = 2.5e15    # dense FLOP/s
    valu_fp32: float = 157.3e12  # FLOP/s


@dataclass(frozen=True)
class Calibration:
    """Effective rates of this library's kernels (fitted)."""
    lam: float = 4e-6            # per-launch overhead lambda_x (s)
    bw_stream: float = 5.8e12    # dense decode's K/V stream (bytes/s)
    bw_gather: float = 5.0e12    # attention's gather of leaf-chunk pieces (bytes/s)
    tau_level: float = 0.5e-6    # router: fixed latency of one level (s)
    tau_log: float = 1.0e-6      # router: latency per doubling of the frontier (s)
    tau_attn: float = 12e-6      # attention workgroup latency at its residency (s)
    tau_dense: float = 10e-6     # dense wave latency floor (s)
    tau_merge_attn: float = 4.1e-6   # attention merge launch: one workgroup per head (s)
    tau_merge_dense: float = 4.7e-6  # dense merge launch (s)


@dataclass(frozen=True)
class Workload:
    """Decode geometry (Tables V-VI): B, Q(T) = 1, heads, dims, storage bytes."""
    B: int
    H_q: int
    H_kv: int
    d: int
    T: int
    C: int
    L: int
    R: int = 1
    Q: int = 1
    s: int = 2       # s_QKV: bf16
    s_acc: int = 4   # s_accum: fp32 partials and statistics

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def heads(self) -> int:
        return self.B * self.Q * self.H_q


# Launch shapes of the library (see the kernel sources).
ATTN_BLOCKS = 512                       # balanced attention workgroups
ATTN_RESIDENT = 2                       # of them per CU
DENSE_WAVES = 2048


def phi(flops: float, P: float, nbytes: float, BW: float, tau: float, n_tiles: int,
        n_cu: int, c: int) -> float:
    """Eq. (4): max of compute time, memory time and worker waves tau ceil(N_tiles / (N_CU c))."""
    return max(flops / P, nbytes / BW, tau * math.ceil(n_tiles / (n_cu * c)))


# ----------------------------------------------------------------------------
# Dense decode (App. D-A)
# ----------------------------------------------------------------------------

def dense_splits(w: Workload) -> int:
    """J(T): splits per query tile, as the library plans them (fill DENSE_WAVES waves)."""
    units = w.B * w.H_kv * math.ceil(w.Q * w.G / 16)
    s = min(math.ceil(DENSE_WAVES / units), math.ceil(w.T / 32))
    tps = math.ceil(math.ceil(w.T / max(s, 1)) / 32) * 32
    return math.ceil(w.T / tps)


def dense_terms(w: Workload) -> dict:
    """Work and traffic of the split partial and merge stages (App. D-A formulas)."""
    n_qtiles = w.B * w.H_kv * math.ceil(w.Q * w.G / 16)
    J = dense_splits(w)
    bq = w.B * w.Q * w.H_q
    return {
        "n_qtiles": n_qtiles, "J": J,
        "flops_partial": 2 * bq * (w.d + w.d) * w.T,
        "bytes_partial": w.s * (w.d + w.d) * n_qtiles * w.T + bq * (w.s * w.d + w.s_acc * J * (w.d + 2)),
        "tiles_partial": n_qtiles * J,
        "flops_merge": bq * (2 * J * w.d + 3 * J - 1),
        "bytes_merge": bq * (w.s_acc * J * (w.d + 2) + w.s * w.d),
        "tiles_merge": bq,
    }


def t_dense(w: Workload, hw: Hardware = Hardware(), cal: Calibration = Calibration()) -> dict:
    x = dense_terms(w)
    # A wave is the worker of the matrix-core kernel: 4 per workgroup, 8 per CU resident.
    partial = phi(x["flops_partial"], hw.mfma_bf16, x["bytes_partial"], cal.bw_stream,
                  cal.tau_dense, x["tiles_partial"], hw.n_cu, 8)
    merge = phi(x["flops_merge"], hw.valu_fp32, x["bytes_merge"], cal.bw_stream,
                cal.tau_merge_dense, x["tiles_merge"], hw.n_cu, 8)
    lam = 2 * cal.lam if x["J"] > 1 else cal.lam
    return {"partial": partial, "merge": merge if x["J"] > 1 else 0.0, "launch": lam,
            "total": lam + partial + (merge if x["J"] > 1 else 0.0)}


# ----------------------------------------------------------------------------
# ZHA decode (App. D-B1)
# ----------------------------------------------------------------------------

def routing_terms(w: Workload, K_l: float) -> dict:
    """Per-level routing work: R scores of d_k MACs per candidate, compressed keys and biases
    read once per query tile (one query head per tile here), plus the queries."""
    bq = w.B * w.Q * w.H_q
    return {"flops": 2 * bq * w.R * w.d * K_l,
            "bytes": w.R * w.s * (w.d + 1) * bq * K_l + w.s * w.d * bq,
            "tiles": bq}


def t_route_level(w: Workload, K_l: float, hw: Hardware, cal: Calibration) -> float:
    x = routing_terms(w, K_l)
    tau = cal.tau_level + cal.tau_log * math.log2(max(K_l, 1.0)) if K_l > 0 else 0.0
    # Scan: in the routing workgroup, scores stay in LDS (no bytes of its own).
    return phi(x["flops"], hw.valu_fp32, x["bytes"], hw.hbm_bw, tau, x["tiles"], hw.n_cu, 1)


def attn_terms(w: Workload, tokens_per_head: float, union_bytes: float) -> dict:
    """Attention over K_0 retained tokens per head; bytes: the grouped union of K/V rows
    (measured) plus the queries and outputs, and the split partials written and read."""
    bq = w.B * w.Q * w.H_q
    part = 2 * w.s_acc * (ATTN_BLOCKS + bq) * (w.d + 2)
    return {"flops": 2 * bq * (w.d + w.d) * tokens_per_head,
            "bytes": union_bytes + w.s * 2 * w.d * bq + part,
            "tiles": ATTN_BLOCKS}


def t_zha(w: Workload, K_levels, tokens_per_head: float, union_bytes: float,
          hw: Hardware = Hardware(), cal: Calibration = Calibration(),
          t_tree: float = 0.0) -> dict:
    """Eq. (3) for this library: one router launch over L levels, one attention launch and
    its merge.  K_levels: mean frontier size per level (level 1 first)."""
    levels = [t_route_level(w, k, hw, cal) for k in K_levels]
    x = attn_terms(w, tokens_per_head, union_bytes)
    attn = phi(x["flops"], hw.valu_fp32, x["bytes"], cal.bw_gather, cal.tau_attn, x["tiles"],
               hw.n_cu, ATTN_RESIDENT)
    merge = phi(0.0, hw.valu_fp32, 0.0, cal.bw_gather, cal.tau_merge_attn, w.heads, hw.n_cu, 8)
    route = cal.lam + sum(levels)
    attn_total = 2 * cal.lam + attn + merge
    return {"route_levels": levels, "route": route, "attn": attn_total, "tree": t_tree,
            "total": t_tree + route + attn_total}


# ----------------------------------------------------------------------------
# Tree construction (App. D-B2)
# ----------------------------------------------------------------------------

def t_tree_decode_sum(t_summ: float, t_merge: float, C: int, L: int) -> float:
    """Amortized maintenance per decoded token: t_summ(1)/C + sum_{l=2..L} t_merge(1)/C^l."""
    return t_summ / C + sum(t_merge / C ** l for l in range(2, L + 1))


def t_tree_decode_closed(t_summ: float, t_merge: float, C: int, L: int) -> float:
    """The same in closed form: t_summ/C + t_merge / (C (C - 1)) (1 - C^-(L - 1))."""
    return t_summ / C + t_merge / (C * (C - 1)) * (1.0 - float(C) ** -(L - 1))


def tree_build_terms(w: Workload, n: int, level: int) -> dict:
    """Work and traffic of one tree kernel processing n full nodes per sequence (Table VIII
    counts, per KV group; the leaf kernel reads its chunk's keys twice)."""
    if level == 1:
        return {"flops": 4 * w.B * w.H_q * n * w.R * w.C * w.d,
                "bytes": w.B * w.H_q * n * (2 * w.s * w.d * (w.C / w.G + w.R)
                                            + w.s_acc * w.R * (w.d + 3)),
                "tiles": w.B * w.H_kv * n}
    return {"flops": 2 * w.B * w.H_q * n * w.R * w.C * w.d,
            "bytes": w.B * w.H_q * n * w.R * (w.s_acc * w.C * (w.d + 4) + w.s_acc * (w.d + 3)
                                              + w.s * w.d),
            "tiles": w.B * w.H_q * n}


# ----------------------------------------------------------------------------
# Calibration
# ----------------------------------------------------------------------------

@dataclass
class Point:
    """One measured decode step: geometry, frontier statistics and times (s)."""
    w: Workload
    K_levels: list
    tokens_per_head: float
    union_bytes: float
    route: float
    attn: float
    dense: float
    extra: dict = field(default_factory=dict)


def _nnls(A, y):
    """Least squares with non-negative coefficients (latencies cannot be negative)."""
    from scipy.optimize import nnls
    sol, _ = nnls(np.asarray(A, float), np.asarray(y, float))
    return sol


def fit(points, hw: Hardware = Hardware(), lam: float = 4.1e-6, tau_merge_attn: float = 4.1e-6,
        tau_merge_dense: float = 4.7e-6) -> Calibration:
    """Fits the effective rates to measured steps.

    lambda (per launch) and the two merge launches' durations are measured directly (a
    trivial kernel's and the merge kernels' rocprof durations) and passed in.  Router:
    t_route - lambda = sum_l [tau_level + tau_log log2 K_l], linear in (tau_level, tau_log).
    Attention: t_attn - 2 lambda - tau_merge is the larger of bytes/bw_gather and tau_attn,
    so tau_attn is the floor seen at small contexts and bw_gather comes from the points
    well above it.  Dense likewise with bytes/bw_stream and tau_dense.
    """
    A, y = [], []
    for p in points:
        ks = [k for k in p.K_levels if k > 0]
        A.append([float(len(ks)), sum(math.log2(max(k, 1.0)) for k in ks)])
        y.append(p.route - lam)
    tau_level, tau_log = (float(v) for v in _nnls(A, y))
    # Attention: floor from the smallest-byte point, bandwidth from the others.
    att = sorted(points, key=lambda p: p.union_bytes)
    body = [p.attn - 2 * lam - tau_merge_attn for p in att]
    tau_attn = min(body)
    big = [(attn_terms(p.w, p.tokens_per_head, p.union_bytes)["bytes"], b)
           for p, b in zip(att, body) if b > 1.5 * tau_attn]
    bw_gather = (sum(x for x, _ in big) / sum(b for _, b in big)) if big else 5e12
    # Dense: stream bandwidth from the points well above the floor.
    dd = [(dense_terms(p.w)["bytes_partial"], p.dense - 2 * lam - tau_merge_dense)
          for p in points]
    floor = min(b for _, b in dd)
    big = [(x, b) for x, b in dd if b > 2 * floor]
    bw_stream = (sum(x for x, _ in big) / sum(b for _, b in big)) if big else 5.8e12
    return Calibration(lam=lam, bw_stream=bw_stream, bw_gather=bw_gather, tau_level=tau_level,
                       tau_log=tau_log, tau_attn=tau_attn, tau_dense=floor,
                       tau_merge_attn=tau_merge_attn, tau_merge_dense=tau_merge_dense)


def predict(p: Point, cal: Calibration, hw: Hardware = Hardware()) -> dict:
    z = t_zha(p.w, p.K_levels, p.tokens_per_head, p.union_bytes, hw, cal)
    d = t_dense(p.w, hw, cal)
    return {"route": z["route"], "attn": z["attn"], "zha": z["total"], "dense": d["total"]}


def crossover(points, cal: Calibration, hw: Hardware = Hardware()):
    """Smallest measured T from which the model has ZHA faster than dense at every larger T."""
    pts = sorted(points, key=lambda p: p.w.T)
    pred = [predict(p, cal, hw) for p in pts]
    for k in range(len(pts)):
        if all(q["zha"] < q["dense"] for q in pred[k:]):
            return pts[k].w.T
    return None


def points_from_crossover(record: dict, B=8, H_q=32, H_kv=4, d=128, C=8) -> list:
    """Points from the JSON line of ``bench.py --crossover`` (deep-decode geometry)."""
    out = []
    for r in record["crossover"]:
        w = Workload(B=B, H_q=H_q, H_kv=H_kv, d=d, T=r["T"], C=C, L=r["L"])
        out.append(Point(w=w, K_levels=list(r["frontier_per_level"]),
                         tokens_per_head=r["keys_attended_frac"] * r["T"],
                         union_bytes=r["attn_union_bytes"], route=r["route_us"] * 1e-6,
                         attn=r["attn_us"] * 1e-6, dense=r["dense_us"] * 1e-6))
    return out


def replace_T(w: Workload, T: int, L: int) -> Workload:
    return replace(w, T=T, L=L)


def report(record: dict, train_T=(4096, 16384, 65536, 262144)) -> str:
    """Markdown table of model against measurement for a ``bench.py --crossover`` record,
    calibrated on the contexts in train_T and checked on the others."""
    pts = points_from_crossover(record)
    cal = fit([p for p in pts if p.w.T in train_T])
    rows = ["| T | L | mean frontier per level (1..L) | route model / measured (us) | attention "
            "model / measured (us) | ZHA step model / measured (us) | e | dense model / measured "
            "(us) | e | set |",
            "|---|---|---|---|---|---|---|---|---|---|"]
    for p in pts:
        q = predict(p, cal)
        ez = 100 * (q["zha"] / (p.route + p.attn) - 1)
        ed = 100 * (q["dense"] / p.dense - 1)
        rows.append(f"| {p.w.T:,} | {p.w.L} | {', '.join(f'{k:.0f}' for k in p.K_levels)} | "
                    f"{q['route'] * 1e6:.1f} / {p.route * 1e6:.1f} | {q['attn'] * 1e6:.1f} / "
                    f"{p.attn * 1e6:.1f} | {q['zha'] * 1e6:.1f} / {(p.route + p.attn) * 1e6:.1f} | "
                    f"{ez:+.0f} % | {q['dense'] * 1e6:.1f} / {p.dense * 1e6:.1f} | {ed:+.0f} % | "
                    f"{'calibration' if p.w.T in train_T else 'held out'} |")
    measured = None
    srt = sorted(pts, key=lambda p: p.w.T)
    for k in range(len(srt)):
        if all(p.route + p.attn < p.dense for p in srt[k:]):
            measured = srt[k].w.T
            break
    c = cal
    rows.append("")
    rows.append(f"Calibrated: lambda {c.lam * 1e6:.1f} us per launch (measured), router "
                f"tau_level {c.tau_level * 1e6:.2f} us + tau_log {c.tau_log * 1e6:.2f} us per "
                f"doubling of the frontier, attention floor {c.tau_attn * 1e6:.1f} us and gather "
                f"{c.bw_gather / 1e12:.2f} TB/s, dense floor {c.tau_dense * 1e6:.1f} us and stream "
                f"{c.bw_stream / 1e12:.2f} TB/s, merges {c.tau_merge_attn * 1e6:.1f} / "
                f"{c.tau_merge_dense * 1e6:.1f} us (measured).")
    rows.append(f"Crossover (smallest T from which ZHA is faster at every larger T): model "
                f"{crossover(pts, cal):,}, measured {measured:,}.")
    return "\n".join(rows)


if __name__ == "__main__":
    import json
    import sys
    rec = json.loads(open(sys.argv[1]).read().strip().splitlines()[-1])
    print(report(rec))
