"""Helpers shared by the tests: device transfer, tree unpacking, oracle runs, parity accounting."""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

import oracle as O
from hierarchical_tree_indexed_04_amd import workload as W

TOL = {W.BF16: 2e-2, W.F32: 1e-4}


def to_device(a: np.ndarray, dtype: str):
    import torch
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.cuda()


def from_device(t, dtype: str) -> np.ndarray:
    """Device tensor of the storage dtype -> float32 numpy values."""
    import torch
    if dtype == W.BF16:
        return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy()


def unpack_tree(Z, g: W.Geometry, tree_np: np.ndarray, b: int, kvh: int, gm=None):
    """Level arrays (k_hat [n, R, d] float, b_hat [n, R] float32) of one tree from the blob;
    ``gm`` gives the layout when it has a capacity beyond g.T."""
    gm = Z.geom(g) if gm is None else gm
    out = []
    for ell in range(1, g.L + 1):
        ko, bo, stride = Z.level_offset(gm, ell)
        base = (b * g.H_kv + kvh) * stride
        n = g.n_level(ell)
        nk = n * g.R * g.d
        if g.dtype == W.BF16:
            k = W.bf16_bits_to_f32(tree_np[base + ko: base + ko + 2 * nk].view(np.uint16))
        else:
            k = tree_np[base + ko: base + ko + 4 * nk].view(np.float32)
        bh = tree_np[base + bo: base + bo + 4 * n * g.R].view(np.float32)
        out.append((k.reshape(n, g.R, g.d), bh.reshape(n, g.R)))
    return out


# The route's gap output s_(m) - s_(m+1) is a difference of two fp32 scores
# (each a 128-term dot product of magnitude up to ~50 nats), the oracle's is fp64
# on the same stored summaries: they agree to a few fp32 ulps of the scores.
GAP_TOL = 1e-3


@dataclass
class Parity:
    heads: int = 0
    exact: int = 0  # S_1 and every level's (K, m) equal
    fragile_diverged: int = 0  # differ, oracle flagged a fragile level at/above the divergence
    mismatched: list = field(default_factory=list)  # non-fragile divergences (must stay empty)
    fragile_levels: int = 0  # fragile levels seen by the oracle (reported)
    max_err: float = 0.0  # over every head with a route (oracle attention on the GPU's set)
    out_checked: int = 0
    out_bad: list = field(default_factory=list)
    gaps_checked: int = 0  # levels whose finite gap was compared with the oracle's
    max_gap_err: float = 0.0
    gap_bad: list = field(default_factory=list)

    def summary(self) -> str:
        return (f"heads={self.heads} exact={self.exact} fragile_diverged={self.fragile_diverged} "
                f"mismatched={len(self.mismatched)} fragile_levels={self.fragile_levels} "
                f"outputs_checked={self.out_checked} max_abs_err={self.max_err:.3g} "
                f"out_bad={len(self.out_bad)} gaps_checked={self.gaps_checked} "
                f"max_gap_err={self.max_gap_err:.3g} gap_bad={len(self.gap_bad)}")

    def check(self, min_exact: float = 0.98):
        """The parity bar: no non-fragile divergence, every output and gap within
        tolerance, and at most 2 % of the heads fragile-diverged (0 measured so far)."""
        assert not self.mismatched, self.mismatched[:5]
        assert not self.out_bad, self.out_bad[:5]
        assert not self.gap_bad, self.gap_bad[:5]
        assert self.exact >= min_exact * self.heads, self.summary()


def compare_head(par: Parity, r: O.Route, sel_row: np.ndarray, cnt: int, stats: np.ndarray,
                 o_gpu: np.ndarray | None, o_ref: np.ndarray | None, tol: float, tag,
                 gap_row: np.ndarray | None = None, attend_set=None):
    """Accumulates the parity verdict of one query head (route, gap, then output).

    The output is compared with o_ref (oracle attention over the oracle's set)
    when the routes agree; when they diverge at a fragile cut, with
    attend_set(gpu_S1), oracle attention over the GPU's own set (summary page
    "Routing": o(q) = Attn(q, K_I, V_I) for whatever set the route produced).
    gap_row (the route's gap output, per level) is compared with the oracle's
    gap at every level of an exactly matching route: +inf exactly where the whole
    frontier is kept, within GAP_TOL elsewhere."""
    par.heads += 1
    L = len(r.S)
    par.fragile_levels += sum(r.fragile)
    gpu_S1 = sel_row[:cnt] if cnt >= 0 else None
    first_div = None
    for ell in range(L, 0, -1):
        if stats[ell - 1, 0] != r.K[ell - 1] or stats[ell - 1, 1] != len(r.S[ell - 1]):
            first_div = ell
            break
    same_S1 = gpu_S1 is not None and np.array_equal(gpu_S1, r.S1)
    if first_div is None and same_S1:
        par.exact += 1
        if gap_row is not None:
            for ell in range(1, L + 1):
                want, got = r.gap[ell - 1], float(gap_row[ell - 1])
                if math.isinf(want) or math.isinf(got):
                    if not (math.isinf(want) and math.isinf(got) and got > 0):
                        par.gap_bad.append((tag, ell, got, want))
                    continue
                err = abs(got - want)
                par.gaps_checked += 1
                par.max_gap_err = max(par.max_gap_err, err)
                if not err <= GAP_TOL:
                    par.gap_bad.append((tag, ell, got, want))
    else:
        lim = first_div if first_div is not None else 1
        if any(r.fragile[ell - 1] for ell in range(lim, L + 1)):
            par.fragile_diverged += 1
        else:
            par.mismatched.append((tag, first_div, cnt, len(r.S1)))
            return
        if attend_set is None or gpu_S1 is None:
            return
        o_ref = attend_set(gpu_S1)
    if o_gpu is not None:
        err = float(np.max(np.abs(o_gpu.astype(np.float64) - o_ref)))
        par.out_checked += 1
        par.max_err = max(par.max_err, err)
        if not err <= tol:
            par.out_bad.append((tag, err))


def attend_on(q, Kf, Vf, C: int, T: int):
    """Oracle attention of q over the token set of a given S_1 (sink, chunks, C_cur)."""
    return lambda S1: O.attend(q, Kf, Vf, O.token_set(S1, C, T))


def oracle_trees(g: W.Geometry, K: np.ndarray, qref: np.ndarray, pairs, rope=None):
    """Oracle trees per (b, kvh); rope = (dims, theta) or None."""
    trees = {}
    for b, kvh in pairs:
        keys = W.to_float(K[b, kvh], g.dtype).astype(np.float64)
        trees[(b, kvh)] = O.build_tree(keys, qref[kvh], g.C, g.L, g.dtype, rope=rope)
    return trees


def tree_mismatch(Z, g, tree_np, trees, gm=None):
    """Counts of stored k_hat / b_hat entries where the device tree differs from the oracle's."""
    bad_k = bad_b = total = 0
    for (b, kvh), t in trees.items():
        levels = unpack_tree(Z, g, tree_np, b, kvh, gm)
        for ell, (k, bh) in enumerate(levels, start=1):
            lv = t.levels[ell - 1]
            bad_k += int(np.count_nonzero(k.astype(np.float64) != lv.k_store))
            bad_b += int(np.count_nonzero(bh.astype(np.float64) != lv.b_store))
            total += k.size
    return bad_k, bad_b, total


def ceil_div(a, b):
    return -(-a // b)


def log2i(x):
    return int(round(math.log2(x)))
