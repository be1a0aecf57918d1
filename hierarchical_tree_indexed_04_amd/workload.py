"""Seeded synthetic workloads for the ZHA hot path.

This module is the one piece shared by the CPU oracle's tests and the HIP
path: it draws inputs and holds none of the method's arithmetic.

Workloads (the five geometries of the hot-path scope, plus small custom ones)
follow the hierarchical Gaussian-mixture recipe used throughout this repo:

* Every node of a virtual tree over the T key positions owns a centre drawn
  i.i.d. from N(0, sigma_k^2 I_d), where k = 1 is the level just below the
  (single or virtual) root and sigma_k = 2^-(k-1) (1.0, 0.5, 0.25, ...).
  Keys are the deepest nodes, so a key is the sum of its ancestors' centres,
  its own centre and N(0, 0.1^2 I_d) noise.  The key's own centre and the
  noise are drawn as one normal of standard deviation sqrt(sigma_D^2 + 0.01)
  (a sum of independent normals has exactly that law).
* Values are N(0, 1).
* A decode query of head h is 3 * k_{j*} + N(0, 0.3^2 I_d) with j* uniform on
  [0, T) and drawn independently per (sequence, step, head); k_{j*} is the
  stored (rounded) key of KV head h // G.
* Reference queries default to R = 1 and q_ref = 0.  With R > 1 they are drawn
  like queries (3 * a random key + N(0, 0.3^2)), kept in fp32.

Streams are independent and reproducible: every block of rows has its own
``SeedSequence([cfg_id, stream, ...])`` (stream 0 keys, 1 values, 2 queries,
3 reference queries, 4 random chunk sets), so any slice can be regenerated
alone and blocks are drawn in parallel threads.

bf16 tensors are returned as ``np.uint16`` bit patterns, rounded to nearest
even from fp32.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

_BLK = 65536  # rows per seeded block

F32 = "f32"
BF16 = "bf16"


@dataclass(frozen=True)
class Geometry:
    """One ZHA workload: cache shape, tree shape, threshold and query count."""

    name: str
    cfg_id: int
    dtype: str  # "f32" or "bf16": K, V, Q, O and stored summaries
    B: int
    H_q: int
    H_kv: int
    d: int
    T: int
    C: int
    L: int
    p: float
    n_steps: int  # decode steps per sequence (or block positions when block=True)
    block: bool = False  # all n_steps positions are routed in one call
    R: int = 1

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    def n_level(self, ell: int) -> int:
        """Full nodes at level ell (1 = leaf chunks of C keys)."""
        return self.T // (self.C ** ell)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4


# The five workloads of the hot-path scope.
CONFIGS = {
    1: Geometry("tiny-fp32-4k", 1, F32, B=1, H_q=1, H_kv=1, d=128, T=4096, C=16, L=3, p=0.9,
                n_steps=64),
    2: Geometry("gqa-decode-128k", 2, BF16, B=1, H_q=32, H_kv=4, d=128, T=131072, C=32, L=3,
                p=0.95, n_steps=256),
    3: Geometry("deep-decode-256k", 3, BF16, B=8, H_q=32, H_kv=4, d=128, T=262144, C=8, L=6,
                p=0.95, n_steps=128),
    4: Geometry("wide-block-1m", 4, BF16, B=1, H_q=16, H_kv=2, d=128, T=1048576, C=32, L=4,
                p=0.95, n_steps=2048, block=True),
    5: Geometry("extreme-16m", 5, BF16, B=1, H_q=8, H_kv=1, d=128, T=16777216, C=16, L=6,
                p=0.9, n_steps=64),
}


def custom(name: str, cfg_id: int, **kw) -> Geometry:
    """A small geometry for tests; unspecified fields follow config 1."""
    return replace(CONFIGS[1], name=name, cfg_id=cfg_id, **kw)


# ----------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def to_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor (bf16 bits or float32) as float32 values."""
    return bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a, dtype=np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, np.float32)


# ----------------------------------------------------------------------------
# Seeded blocks
# ----------------------------------------------------------------------------

def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) for w in words])))


def _normal_rows(seed: tuple, nrows: int, d: int, scale: float, out: np.ndarray | None = None):
    g = _rng(*seed)
    if out is None:
        out = np.empty((nrows, d), np.float32)
    g.standard_normal(out=out, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def _threads() -> int:
    env = os.environ.get("ZHA_GEN_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def centre_spans(g: Geometry) -> list[int]:
    """Key-span of each centre depth k = 1..D (last entry is 1: the key itself)."""
    top = g.L if g.n_level(g.L) > 1 else g.L - 1
    return [g.C ** e for e in range(top, -1, -1)]


def centre_scales(g: Geometry) -> list[float]:
    return [2.0 ** (-k) for k in range(len(centre_spans(g)))]


def _key_rows(g: Geometry, b: int, kvh: int, centres: list[np.ndarray], r0: int, r1: int,
              blk: int) -> np.ndarray:
    spans = centre_spans(g)
    sd = centre_scales(g)[-1]
    x = _normal_rows((g.cfg_id, 0, b, kvh, len(spans), blk), r1 - r0, g.d,
                     math.sqrt(sd * sd + 0.01))
    rows = np.arange(r0, r1)
    for k, span in enumerate(spans[:-1]):
        x += centres[k][rows // span]
    return x


def _centres(g: Geometry, b: int, kvh: int, pool: ThreadPoolExecutor) -> list[np.ndarray]:
    spans = centre_spans(g)
    scales = centre_scales(g)
    out = []
    for k, span in enumerate(spans[:-1]):
        n = -(-g.T // span)
        arr = np.empty((n, g.d), np.float32)
        jobs = []
        for blk, r0 in enumerate(range(0, n, _BLK)):
            r1 = min(n, r0 + _BLK)
            jobs.append(pool.submit(_normal_rows, (g.cfg_id, 0, b, kvh, k + 1, blk), r1 - r0, g.d,
                                    scales[k], arr[r0:r1]))
        for j in jobs:
            j.result()
        out.append(arr)
    return out


def make_kv(g: Geometry, want_v: bool = True, slices=None):
    """K (and V) as [B, H_kv, T, d] stored arrays (uint16 bf16 bits or float32).

    ``slices`` optionally restricts generation to a list of (b, kvh) pairs; the
    others are left zero (used to keep host work bounded for spot checks).
    """
    sdt = np.uint16 if g.dtype == BF16 else np.float32
    K = np.zeros((g.B, g.H_kv, g.T, g.d), sdt)
    V = np.zeros((g.B, g.H_kv, g.T, g.d), sdt) if want_v else None
    pairs = slices if slices is not None else [(b, h) for b in range(g.B) for h in range(g.H_kv)]
    with ThreadPoolExecutor(_threads()) as pool:
        for b, kvh in pairs:
            cent = _centres(g, b, kvh, pool)
            jobs = []
            for blk, r0 in enumerate(range(0, g.T, _BLK)):
                r1 = min(g.T, r0 + _BLK)

                def kjob(r0=r0, r1=r1, blk=blk, b=b, kvh=kvh, cent=cent):
                    K[b, kvh, r0:r1] = _store(_key_rows(g, b, kvh, cent, r0, r1, blk), g.dtype)

                jobs.append(pool.submit(kjob))
                if want_v:
                    def vjob(r0=r0, r1=r1, blk=blk, b=b, kvh=kvh):
                        V[b, kvh, r0:r1] = _store(
                            _normal_rows((g.cfg_id, 1, b, kvh, blk), r1 - r0, g.d, 1.0), g.dtype)

                    jobs.append(pool.submit(vjob))
            for j in jobs:
                j.result()
            del cent
    return K, V


def make_queries(g: Geometry, K: np.ndarray, step: int) -> np.ndarray:
    """Queries of one decode step (or one block position): [B, H_q, d] stored."""
    Kf_row = lambda b, kvh, j: to_float(K[b, kvh, j], g.dtype)  # noqa: E731
    out = np.empty((g.B, g.H_q, g.d), np.float32)
    for b in range(g.B):
        rng = _rng(g.cfg_id, 2, b, step)
        js = rng.integers(0, g.T, size=g.H_q)
        noise = rng.standard_normal((g.H_q, g.d), dtype=np.float32) * np.float32(0.3)
        for h in range(g.H_q):
            out[b, h] = np.float32(3.0) * Kf_row(b, h // g.G, js[h]) + noise[h]
    return _store(out, g.dtype)


def make_query_block(g: Geometry, K: np.ndarray, steps) -> np.ndarray:
    """Queries for several steps/positions: [B, len(steps), H_q, d] stored."""
    steps = list(steps)
    sdt = np.uint16 if g.dtype == BF16 else np.float32
    out = np.empty((g.B, len(steps), g.H_q, g.d), sdt)
    for i, s in enumerate(steps):
        out[:, i] = make_queries(g, K, s)
    return out


def make_qref(g: Geometry, K: np.ndarray, R: int | None = None) -> np.ndarray:
    """Reference queries [H_kv, R, d] fp32; R = 1 gives the zero reference."""
    R = g.R if R is None else R
    out = np.zeros((g.H_kv, R, g.d), np.float32)
    if R == 1:
        return out
    for kvh in range(g.H_kv):
        rng = _rng(g.cfg_id, 3, kvh)
        js = rng.integers(0, g.T, size=R)
        noise = rng.standard_normal((R, g.d), dtype=np.float32) * np.float32(0.3)
        for r in range(R):
            out[kvh, r] = np.float32(3.0) * to_float(K[0, kvh, js[r]], g.dtype) + noise[r]
    return out


def random_chunk_sets(g: Geometry, n_heads: int, max_chunks: int, seed: int, cap: int):
    """Random ascending level-1 chunk-id lists, for tests of attention alone.

    Returns (sel [n_heads, cap] int32 padded with -1, cnt [n_heads] int32).  Counts are uniform
    on [0, max_chunks] (so empty sets occur).
    """
    n1 = g.n_level(1)
    rng = _rng(g.cfg_id, 4, seed)
    sel = np.full((n_heads, cap), -1, np.int32)
    cnt = np.zeros(n_heads, np.int32)
    for h in range(n_heads):
        m = int(rng.integers(0, min(max_chunks, n1) + 1))
        ids = np.sort(rng.choice(n1, size=m, replace=False)).astype(np.int32)
        cnt[h] = m
        sel[h, :min(m, cap)] = ids[:cap]
    return sel, cnt
