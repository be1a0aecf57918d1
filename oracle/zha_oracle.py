"""Plain fp64 CPU oracle for the ZHA hot path: tree build, top-p routing, sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from the product package; callers hand it plain
NumPy arrays (bf16 inputs already widened to float values).

Sources (titles of the pages this follows):

* "Subquadratic Attention with a Hierarchical Tree-Structured Indexer"
  (the full paper): §II-A (top-p set, eq. (1)), §III-A (chunk log-mass F_C,
  tangent summaries), §III-B (shared reference queries, frontier-normalised
  chunk probabilities), §III-C (top-p routing per level), App. D-B2 (baseline
  stable-state merge: per reference, rescale and sum the children's weighted
  sums), App. E-E (frontier expansion adds nodes whose parent is incomplete,
  final reads include the first key and the partial chunk).
* The condensed summary page of the same paper (picx.dev): "Tree
  Construction" (k_hat_r, b_hat_r, max over tangents) and "Routing"
  (m_ell(q), the final index set I(q), o(q) = Attn(q, K_I, V_I)).

Readings taken where the pages leave a step open (each one also listed in the
design notes of the repository):

* Scores carry the 1/sqrt(d) factor of the tangent t_r(q).
* Candidates are ordered by score descending, ties to the lower node id.
* The cut is the first prefix m with W_m >= p * Z, where W is one running sum
  in that order and Z = W_K; p >= 1 keeps the whole frontier.  p is taken as
  the fp32 value the library receives.
* The softmax of a level runs over that level's frontier only.
* Stored summaries k_hat are rounded (nearest-even) to the storage dtype, the
  biases b_hat to fp32; merges use the unrounded fp64 child values.
* Token 0 (the sink) and the tokens after the last complete leaf chunk are
  always attended; the sink is a set union, never counted twice.
* RoPE re-anchoring (paper §III-B, reference queries): token t sits at position
  t; a node's reference queries are rotated to the last position of its span;
  the rotation pairs dim k with dim k + dims/2 (k < dims/2) at angle
  position * theta_k, with the theta_k given (the model's frequencies), and
  leaves dims >= dims unrotated.

Fragility (reported, used by parity tests): a level's cut is fragile when
(G) m < K and the score gap s_(m) - s_(m+1) is below EPS = 1e-3, or (M) a
prefix-mass ratio sits within a relative EPS_MASS = 1e-4 of p on either side
of the cut: W_m / Z < p (1 + EPS_MASS) or W_{m-1} / Z >= p (1 - EPS_MASS).
EPS_MASS is a hundred times the relative error of an fp32 evaluation of the
same sums (exp of fp32 scores and running sums over at most a few thousand
terms), the same safety factor EPS has over fp32 score error.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

EPS = 1e-3
EPS_MASS = 1e-4

F64 = "f64"  # no storage rounding (used by the pins only)
F32 = "f32"
BF16 = "bf16"


# ----------------------------------------------------------------------------
# Storage rounding
# ----------------------------------------------------------------------------

def round_to_bf16(x) -> np.ndarray:
    """Nearest-even rounding of fp64 values to bf16 (8 significant bits), returned as fp64.

    Written from the definition: the spacing of bf16 values in [2^e, 2^{e+1}) is 2^{e-7};
    x / spacing is rounded half-to-even.  Values below the normal range use the fixed
    subnormal spacing 2^-133.  Overflow saturates to +-inf like any IEEE conversion.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    ax = np.abs(x[nz])
    e = np.floor(np.log2(ax))
    # log2 can be off by one next to powers of two; fix the exponent exactly.
    e = np.where(np.exp2(e) > ax, e - 1, e)
    e = np.where(np.exp2(e + 1) <= ax, e + 1, e)
    e = np.maximum(e, -126.0)
    spacing = np.exp2(e - 7)
    r = np.round(ax / spacing) * spacing  # np.round is half-to-even
    r = np.where(r > 3.3895313892515355e38, np.inf, r)
    out[nz] = np.sign(x[nz]) * r
    return out


def round_to_store(x, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if dtype == BF16:
        return round_to_bf16(x)
    if dtype == F32:
        return x.astype(np.float32).astype(np.float64)
    if dtype == F64:
        return x.copy()
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Tree construction (paper §III-A, App. D-B2; summary page "Tree Construction")
# ----------------------------------------------------------------------------

def chunk_log_mass(q, keys) -> float:
    """F_C(q) = LSE_j (q . k_j / sqrt(d)) over one chunk (paper §III-A)."""
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    s = keys @ q / math.sqrt(q.shape[-1])
    m = s.max()
    return float(m + math.log(np.exp(s - m).sum()))


def rope_rotate(x, pos, dims: int, theta):
    """Rotary position embedding (RoFormer rotation) of vectors x [..., d] to positions pos.

    pos: a scalar or one position per leading index of x ([n] for x [n, ...]).  For
    k < dims/2, the pair (x_k, x_{k + dims/2}) is rotated by the angle pos * theta_k; dims
    from `dims` on are left as they are.  dims = 0 returns x unchanged.
    """
    x = np.array(x, dtype=np.float64)
    if dims == 0:
        return x
    h = dims // 2
    theta = np.asarray(theta, np.float64).reshape(h)
    pos = np.asarray(pos, np.float64)
    ang = pos.reshape(pos.shape + (1,) * (x.ndim - 1 - pos.ndim) + (1,)) * theta
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h].copy(), x[..., h:dims].copy()
    x[..., :h] = a * c - b * s
    x[..., h:dims] = a * s + b * c
    return x


def node_references(qref, ell: int, n: int, C: int, rope):
    """Reference queries [n, R, d] of the first n nodes of level ell: the shared qref [R, d],
    or with rope = (dims, theta) qref rotated to the last position of each node's span,
    (i + 1) C^ell - 1 (paper §III-B)."""
    qref = np.asarray(qref, np.float64)
    q = np.broadcast_to(qref, (n,) + qref.shape).copy()
    if rope is None or rope[0] == 0:
        return q
    last = (np.arange(n, dtype=np.float64) + 1) * float(C) ** ell - 1
    return rope_rotate(q, last, rope[0], rope[1])


def leaf_summaries(keys, qref):
    """Tangent summaries of leaf chunks.

    keys: [n, C, d] (n chunks of C raw keys), qref: [R, d] shared by all chunks, or [n, R, d]
    one set per chunk (rotated references).
    For each chunk and reference r (summary page "Tree Construction"; paper §III-A):
      s_j = q_r . k_j / sqrt(d),  F = LSE_j s_j,
      k_hat = sum_j softmax_j(s) k_j,  b_hat = F - q_r . k_hat / sqrt(d).
    Returns F [n, R], k_hat [n, R, d], b_hat [n, R], all fp64.
    """
    keys = np.asarray(keys, np.float64)
    n, _, d = keys.shape
    qref = np.asarray(qref, np.float64)
    if qref.ndim == 2:
        qref = np.broadcast_to(qref, (n,) + qref.shape)
    s = np.einsum("ncd,nrd->nrc", keys, qref) / math.sqrt(d)  # [n, R, C]
    m = s.max(axis=-1, keepdims=True)
    w = np.exp(s - m)
    Z = w.sum(axis=-1)  # [n, R]
    F = m[..., 0] + np.log(Z)
    k_hat = np.einsum("nrc,ncd->nrd", w, keys) / Z[..., None]
    b_hat = F - np.einsum("nrd,nrd->nr", k_hat, qref) / math.sqrt(d)
    return F, k_hat, b_hat


def merge_summaries(F_child, k_child, qref, q_child=None):
    """Parent summaries from C children each (paper App. D-B2 baseline stable-state merge).

    F_child: [n, C, R], k_child: [n, C, R, d]; qref: the parents' references, [R, d] shared
    or [n, R, d].  Per reference r, independently:
      F_P = LSE_c F_c,  k_hat_P = sum_c exp(F_c - F_P) k_hat_c,
      b_hat_P = F_P - q_r . k_hat_P / sqrt(d).
    The sum is evaluated the way App. D-B2 keeps its statistics, a maximum m and a weight sum
    Z = sum_c exp(F_c - m): k_hat_P = sum_c exp(F_c - m) k_hat_c / Z and F_P = m + ln Z (the
    same quantity; with equal child masses every weight is exactly 1).
    With q_child [n, C, R, d] (children summarised at their own rotated references), every
    child's log-mass is first moved to the parent's reference (paper §III-B re-anchoring):
      F_c <- F_c + <k_hat_c, q_P - q_c> / sqrt(d).
    """
    F_child = np.asarray(F_child, np.float64)
    k_child = np.asarray(k_child, np.float64)
    n, C, R, d = k_child.shape
    qref = np.asarray(qref, np.float64)
    if qref.ndim == 2:
        qref = np.broadcast_to(qref, (n,) + qref.shape)
    if q_child is not None:
        dq = qref[:, None, :, :] - np.asarray(q_child, np.float64)  # [n, C, R, d]
        F_child = F_child + np.einsum("ncrd,ncrd->ncr", k_child, dq) / math.sqrt(d)
    m = F_child.max(axis=1, keepdims=True)  # [n, 1, R]
    e = np.exp(F_child - m)  # [n, C, R]
    Z = e.sum(axis=1)  # [n, R]
    F_P = m[:, 0, :] + np.log(Z)
    k_P = np.einsum("ncr,ncrd->nrd", e, k_child) / Z[..., None]
    b_P = F_P - np.einsum("nrd,nrd->nr", k_P, qref) / math.sqrt(d)
    return F_P, k_P, b_P


@dataclass
class Level:
    F: np.ndarray  # [n, R] fp64
    k_hat: np.ndarray  # [n, R, d] fp64 (unrounded)
    b_hat: np.ndarray  # [n, R] fp64 (unrounded)
    k_store: np.ndarray  # [n, R, d] k_hat rounded to the storage dtype (as fp64)
    b_store: np.ndarray  # [n, R] b_hat rounded to fp32 (as fp64)


@dataclass
class Tree:
    C: int
    T: int
    d: int
    dtype: str
    levels: list = field(default_factory=list)  # levels[ell-1] is level ell

    @property
    def L(self) -> int:
        return len(self.levels)

    def n(self, ell: int) -> int:
        return self.levels[ell - 1].F.shape[0]


def build_tree(keys, qref, C: int, L: int, dtype: str, rope=None) -> Tree:
    """Full tree over one KV head's keys [T, d] (paper §III-A: recursive summaries).

    Level 1 has n_1 = floor(T / C) chunk summaries; level ell has n_ell = floor(T / C^ell)
    nodes, each built from its C children at level ell - 1.  rope = (dims, theta) summarises
    every node at its rotated references and re-anchors children to their parent's (paper
    §III-B); None (or dims 0) uses the shared references everywhere.
    """
    keys = np.asarray(keys, np.float64)
    T, d = keys.shape
    qref = np.asarray(qref, np.float64).reshape(-1, d)
    R = qref.shape[0]
    roped = rope is not None and rope[0] != 0
    bias_dtype = F64 if dtype == F64 else F32
    tree = Tree(C=C, T=T, d=d, dtype=dtype)
    n1 = T // C
    q1 = node_references(qref, 1, n1, C, rope)
    F, k, b = leaf_summaries(keys[: n1 * C].reshape(n1, C, d), q1)
    tree.levels.append(Level(F, k, b, round_to_store(k, dtype), round_to_store(b, bias_dtype)))
    q_prev = q1
    for ell in range(2, L + 1):
        prev = tree.levels[-1]
        n = T // C ** ell
        q_ell = node_references(qref, ell, n, C, rope)
        q_child = q_prev[: n * C].reshape(n, C, R, d) if roped else None
        F, k, b = merge_summaries(prev.F[: n * C].reshape(n, C, R),
                                  prev.k_hat[: n * C].reshape(n, C, R, d), q_ell, q_child)
        tree.levels.append(Level(F, k, b, round_to_store(k, dtype), round_to_store(b, bias_dtype)))
        q_prev = q_ell
    return tree


# ----------------------------------------------------------------------------
# Routing (paper §III-C; summary page "Routing")
# ----------------------------------------------------------------------------

def node_scores(q, k_store, b_store) -> np.ndarray:
    """s_i = max_r (q . k_hat_{r,i} / sqrt(d) + b_hat_{r,i}) (max over tangents, §III-A)."""
    q = np.asarray(q, np.float64)
    d = q.shape[-1]
    t = np.einsum("nrd,d->nr", k_store, q) / math.sqrt(d) + b_store
    return t.max(axis=1)


@dataclass
class Cut:
    order: np.ndarray  # candidate positions sorted by (score desc, id asc)
    m: int  # number kept
    K: int  # frontier size
    gap: float  # s_(m) - s_(m+1), +inf when m == K
    ratio_m: float  # W_m / Z
    ratio_prev: float  # W_{m-1} / Z (0 when m == 1)
    fragile_gap: bool
    fragile_mass: bool


def topp_cut(scores, ids, p: float) -> Cut:
    """Smallest prefix (by score, ties to lower id) whose softmax mass reaches p.

    m = min{ m : W_m >= p * Z } with W the running sum of exp(s - s_max) in sorted order and
    Z = W_K (summary page "Routing", m_ell(q); paper §III-C).  p >= 1 keeps all candidates.
    """
    scores = np.asarray(scores, np.float64)
    ids = np.asarray(ids)
    K = scores.shape[0]
    if K == 0:
        return Cut(np.zeros(0, np.int64), 0, 0, math.inf, 1.0, 0.0, False, False)
    p32 = float(np.float32(p))
    order = np.lexsort((ids, -scores))
    s = scores[order]
    w = np.exp(s - s[0])
    W = np.cumsum(w)
    Z = W[-1]
    if p32 >= 1.0:
        m = K
    else:
        m = int(np.argmax(W >= p32 * Z)) + 1
    gap = float(s[m - 1] - s[m]) if m < K else math.inf
    ratio_m = float(W[m - 1] / Z)
    ratio_prev = float(W[m - 2] / Z) if m >= 2 else 0.0
    fragile_gap = m < K and gap < EPS
    fragile_mass = p32 < 1.0 and (ratio_m < p32 * (1.0 + EPS_MASS)
                                  or ratio_prev >= p32 * (1.0 - EPS_MASS))
    return Cut(order, m, K, gap, ratio_m, ratio_prev, fragile_gap, fragile_mass)


@dataclass
class Route:
    S: list  # S[ell-1]: selected ids at level ell, ascending
    K: list  # frontier size per level
    gap: list
    fragile: list  # per level: (fragile_gap or fragile_mass)
    fragile_kind: list  # per level: "", "G", "M" or "GM"

    @property
    def S1(self) -> np.ndarray:
        return self.S[0]


def route(tree: Tree, q, p: float) -> Route:
    """Top-down routing of one query head through one tree (paper §III-C, App. E-E).

    The top level's frontier is every top node.  Below, the frontier is the children of the
    selected nodes, plus nodes whose parent is incomplete (they have no parent to select them).
    """
    L = tree.L
    C = tree.C
    res = Route([None] * L, [0] * L, [0.0] * L, [False] * L, [""] * L)
    frontier = np.arange(tree.n(L))
    for ell in range(L, 0, -1):
        lv = tree.levels[ell - 1]
        s = node_scores(q, lv.k_store[frontier], lv.b_store[frontier])
        cut = topp_cut(s, frontier, p)
        S = np.sort(frontier[cut.order[: cut.m]])
        res.S[ell - 1] = S
        res.K[ell - 1] = cut.K
        res.gap[ell - 1] = cut.gap
        res.fragile[ell - 1] = cut.fragile_gap or cut.fragile_mass
        res.fragile_kind[ell - 1] = ("G" if cut.fragile_gap else "") + ("M" if cut.fragile_mass else "")
        if ell > 1:
            children = (S[:, None] * C + np.arange(C)[None, :]).reshape(-1)
            orphans = np.arange(tree.n(ell) * C, tree.n(ell - 1))
            frontier = np.concatenate([children, orphans])
    return res


# ----------------------------------------------------------------------------
# Attention (summary page "Routing": I(q) and o(q))
# ----------------------------------------------------------------------------

def token_set(S1, C: int, T: int) -> np.ndarray:
    """I(q) = {0} U tokens of the selected leaf chunks U C_cur, ascending.

    C_cur is every token after the last complete leaf chunk: [floor(T/C) C, T).
    """
    S1 = np.asarray(S1, np.int64)
    n1 = T // C
    toks = (S1[:, None] * C + np.arange(C)[None, :]).reshape(-1)
    cur = np.arange(n1 * C, T)
    return np.union1d(np.union1d(np.array([0]), toks), cur)


def attend(q, K, V, idx=None) -> np.ndarray:
    """Exact softmax attention of one query over the rows idx of K, V (all rows if None), fp64."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K if idx is None else K[idx], np.float64)
    V = np.asarray(V if idx is None else V[idx], np.float64)
    s = K @ q / math.sqrt(q.shape[-1])
    e = np.exp(s - s.max())
    return (e @ V) / e.sum()


def dense(q, K, V) -> np.ndarray:
    """Full attention over all T keys (the dense-decode baseline)."""
    return attend(q, K, V, None)


def zha_head(tree: Tree, q, K, V, p: float):
    """One query head end to end: route, then attention over I(q).  Returns (Route, o fp64)."""
    r = route(tree, q, p)
    o = attend(q, K, V, token_set(r.S1, tree.C, tree.T))
    return r, o
