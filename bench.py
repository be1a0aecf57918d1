#!/usr/bin/env python3
"""ZHA decode benchmark on one MI355X.

A step is one decode step of the whole hot path over one batch: zha_route
(top-down top-p routing of every query head through its tree) followed by
zha_attn (exact attention over the routed tokens), on seeded synthetic inputs
already resident in HBM.  The batch's sequences are independent, so the timed
steps run it as two micro-batches (B/2 sequences each) on two streams, each a
chain of zha_route then zha_attn per step: one half's latency-bound routing
overlaps the other half's bandwidth-bound attention.  The same steps on one
stream are reported beside it.  The tree is built once before timing (its time
is reported separately).  Default workload: deep-tree decode at 256K context,
B = 8 sequences, 32 query heads over 4 KV heads, d = 128, C = 8, L = 6,
p = 0.95, bf16.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from hierarchical_tree_indexed_04_amd import workload as W  # noqa: E402

METRIC = "ZHA decode queries/sec per layer at 256K and 1M ctx; % of HBM peak"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "hierarchical_tree_indexed_04_amd", "csrc")
# Sources that determine the decode step's kernels; measured traffic is
# reported only while their hash matches the one recorded with the counters.
STEP_SOURCES = ["zha_route.hip", "zha_route_impl.inc", "zha_attn.hip", "zha_attn_impl.hpp",
                "zha_plan.hpp", "zha_internal.hpp", "zha_common.hpp", "zha_wave.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode-step_deep-decode-256k.json")


def step_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per zha_route and per zha_attn call (dict) from the committed counter
    runs, or None when the kernels' sources changed since."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != step_source_hash():
        return None
    return rec


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample, over host cores.
# ----------------------------------------------------------------------------
_CB = None


def _cb_head(item):
    import oracle as O
    g, trees, Kf, Vf = _CB
    q, kvh = item
    r = O.route(trees[kvh], q, g.p)
    O.attend(q, Kf[kvh], Vf[kvh], O.token_set(r.S1, g.C, g.T))
    return 1


def _one_thread():
    # One BLAS thread per worker process: `cores` is then the thread count used.
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def cpu_baseline(g, K, V, seconds: float, procs: int):
    """Oracle route + attention per query head of sequence 0; rate in queries/s."""
    global _CB
    import multiprocessing as mp

    import oracle as O
    trees, Kf, Vf = {}, {}, {}
    for kvh in range(g.H_kv):
        Kf[kvh] = W.to_float(K[0, kvh], g.dtype)
        Vf[kvh] = W.to_float(V[0, kvh], g.dtype)
        trees[kvh] = O.build_tree(Kf[kvh].astype(np.float64), reference_queries(g, K)[kvh],
                                  g.C, g.L, g.dtype)
    items = []
    for step in range(8192):
        Q = W.make_queries(g, K, step)
        for h in range(g.H_q):
            items.append((W.to_float(Q[0, h], g.dtype), h // g.G))
    _CB = (g, trees, Kf, Vf)
    ctx = mp.get_context("fork")
    done = 0
    with ctx.Pool(procs, initializer=_one_thread) as pool:
        t0 = time.perf_counter()
        for _ in pool.imap_unordered(_cb_head, items, chunksize=2):
            done += 1
            if time.perf_counter() - t0 > seconds:
                break
        elapsed = time.perf_counter() - t0
        pool.terminate()
    _CB = None
    heads_per_s = done / elapsed
    return {"value": heads_per_s / g.H_q, "unit": "queries/s", "cores": procs, "kind": "oracle",
            "sample": f"{done} query heads (sequence 0, decode steps in order, all {g.H_q} heads "
                      f"per step) of the same workload, fp64 NumPy route + attention, "
                      f"{elapsed:.1f} s wall over {procs} single-threaded processes; tree build "
                      f"excluded"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------
# Byte accounting (algorithmic bytes, per step)
# ----------------------------------------------------------------------------

def step_bytes(g, sel, cnt, stats):
    """Bytes the routing and the sparse gather must touch in one step.

    Attention: K and V rows of the attended tokens, counted once per KV head (union over the
    G query heads of the group, the minimum any implementation moves) and summed per head;
    plus each head's query read, output write and chunk-list read.  Routing: per query head,
    the summary row (R d storage elements + R fp32 biases) of every candidate at every level,
    the query, and the route outputs.
    """
    s = g.elem_bytes
    row_kv = 2 * g.d * s
    n1 = g.n_level(1)
    tail = g.T - n1 * g.C
    attn_union = attn_sum = 0
    heads = g.B * g.H_q
    for b in range(g.B):
        for kvh in range(g.H_kv):
            ids = []
            for h in range(kvh * g.G, (kvh + 1) * g.G):
                c = int(cnt[b, 0, h])
                ch = sel[b, 0, h, :c]
                ids.append(ch)
                # The sink is a token of its own unless chunk 0 is selected or,
                # with no complete chunk, the partial chunk already holds it.
                toks = c * g.C + tail + (0 if (n1 == 0 or (c > 0 and ch[0] == 0)) else 1)
                attn_sum += toks * row_kv
            u = np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)
            toks_u = u.size * g.C + tail + (0 if (n1 == 0 or (u.size and u[0] == 0)) else 1)
            attn_union += toks_u * row_kv
    per_head_io = heads * (2 * g.d * s) + int(cnt.sum()) * 4
    attn_union += per_head_io
    attn_sum += per_head_io
    route_row = g.R * g.d * s + 4 * g.R
    K_levels = stats[..., 0].astype(np.int64)  # [B, 1, H_q, L]
    route = int(K_levels.sum()) * route_row + heads * g.d * s + int(cnt.sum()) * 4 + heads * (
        4 + 8 * g.L)
    return {"attn_union": attn_union, "attn_per_head": attn_sum, "route": route,
            "tokens_per_head": float((cnt.astype(np.int64) * g.C).mean())}


# ----------------------------------------------------------------------------
# GPU part
# ----------------------------------------------------------------------------

def to_dev(torch, a, dtype):
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def device_wait(torch, us: float = 300.0):
    """Queues a spin of about `us` on the device, so that the launches queued
    behind it are all submitted before the first of them can start: events
    recorded after it then time device work alone, not the host's submission."""
    torch.cuda._sleep(int(us * 2400))


def layer_count(layer_bytes: int) -> int:
    """Synthetic layers the timed decode steps cycle through: at least 4, and
    enough for 4 GiB of caches and trees in all (at most 16)."""
    return int(min(16, max(4, -(-(4 << 30) // layer_bytes))))


def reference_queries(g, K):
    """[H_kv, R, d] fp32: the zero reference for R = 1 (tangents are the span means), else R
    reference queries per KV head drawn like queries from the head's keys."""
    if g.R == 1:
        return np.zeros((g.H_kv, 1, g.d), np.float32)
    return W.make_qref(g, K)


def run_gpu(g, K, V, steps, warmup, dense_steps, lean=False):
    """The decode-step measurements of workload g.  lean: only the timed steps, the build and
    dense decode (no cache-cold repeats, copy rate or tree-maintenance timings)."""
    import torch

    from hierarchical_tree_indexed_04_amd import zha as Z
    Z.load()
    torch.cuda.set_device(0)
    gm = Z.geom(g)
    n = warmup + steps
    t0 = time.perf_counter()
    Qs = np.stack([W.make_queries(g, K, i) for i in range(n)])[:, :, None]  # [n, B, 1, H_q, d]
    log(f"[bench] queries for {n} steps: {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    Kd, Vd = to_dev(torch, K, g.dtype), to_dev(torch, V, g.dtype)
    Qd = to_dev(torch, Qs, g.dtype)
    # R = 1 builds take no reference queries (the zero reference); R > 1 draws them.
    qref = None if g.R == 1 else torch.from_numpy(reference_queries(g, K)).cuda()
    torch.cuda.synchronize()
    log(f"[bench] upload {Kd.numel() * 2 * Kd.element_size() / 1e9:.2f} GB: "
        f"{time.perf_counter() - t0:.1f} s")

    tb, sb = Z.tree_bytes(gm)
    tree = torch.empty(tb, dtype=torch.uint8, device="cuda")
    bscratch = torch.empty(max(sb, 1), dtype=torch.uint8, device="cuda")
    Z.build(gm, Kd, qref, tree, bscratch)  # first call: code load
    torch.cuda.synchronize()
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    device_wait(torch)
    eb0.record()
    Z.build(gm, Kd, qref, tree, bscratch)
    eb1.record()
    torch.cuda.synchronize()
    build_ms = eb0.elapsed_time(eb1)
    log(f"[bench] tree build {build_ms:.2f} ms ({tb / 1e6:.1f} MB tree)")

    # Decode visits every layer's cache and tree in turn, so a layer's rows are
    # long gone from L2 and the 256 MB memory-side cache when its next step
    # comes.  The timed steps do the same: step i uses layer i mod n_layers, each
    # layer its own copy of K, V and the tree in HBM, with at least 4 GiB of them
    # in all.
    n_layers = layer_count(Kd.numel() * 2 * Kd.element_size() + tb)
    layers = [(Kd, Vd, tree)]
    for _ in range(n_layers - 1):
        layers.append((Kd.clone(), Vd.clone(), tree.clone()))
    torch.cuda.synchronize()
    log(f"[bench] steps cycle through {n_layers} layers' caches and trees")

    # Chunk-list capacity: every leaf chunk when the lists of all steps fit in 2 GiB.
    cap = g.n_level(1) if n * g.B * g.H_q * g.n_level(1) * 4 <= (2 << 30) else 8192
    sel = torch.empty((n, g.B, 1, g.H_q, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((n, g.B, 1, g.H_q), dtype=torch.int32, device="cuda")
    stats = torch.empty((n, g.B, 1, g.H_q, g.L, 2), dtype=torch.int32, device="cuda")
    O = torch.empty((n, g.B, 1, g.H_q, g.d), dtype=Kd.dtype, device="cuda")
    rscratch = torch.empty(max(Z.route_scratch_bytes(gm, 1, cap), 1), dtype=torch.uint8,
                           device="cuda")
    ascratch = torch.zeros(max(Z.attn_scratch_bytes(gm, 1, cap), 1), dtype=torch.uint8,
                           device="cuda")
    fscratch = torch.zeros(max(Z.route_attn_scratch_bytes(gm, 1, cap), 1), dtype=torch.uint8,
                           device="cuda")

    # Timed loop: direct C-ABI calls with pointers marshalled once, so host
    # overhead stays far below the GPU time of a step.
    import ctypes
    lib = Z.load()
    gref = ctypes.byref(gm)
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    lp = [(vp(t.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr())) for (k, v, t) in layers]
    rs_p, as_p = vp(rscratch.data_ptr()), vp(ascratch.data_ptr())
    args_r = [(gref, lp[i % n_layers][0], vp(Qd[i].data_ptr()), 1, None, ctypes.c_float(g.p),
               vp(sel[i].data_ptr()),
               vp(cnt[i].data_ptr()), cap, vp(stats[i].data_ptr()), None, rs_p, stream)
              for i in range(n)]
    args_a = [(gref, vp(Qd[i].data_ptr()), 1, None, lp[i % n_layers][1], lp[i % n_layers][2],
               vp(sel[i].data_ptr()), vp(cnt[i].data_ptr()), cap, vp(O[i].data_ptr()), as_p,
               stream) for i in range(n)]
    fs_p = vp(fscratch.data_ptr())
    args_f = [(gref, lp[i % n_layers][0], vp(Qd[i].data_ptr()), 1, None, ctypes.c_float(g.p),
               lp[i % n_layers][1], lp[i % n_layers][2], vp(sel[i].data_ptr()),
               vp(cnt[i].data_ptr()), cap, vp(stats[i].data_ptr()), None, vp(O[i].data_ptr()),
               fs_p, stream) for i in range(n)]
    zr, za, zf = lib.zha_route, lib.zha_attn, lib.zha_route_attn

    def step(i):
        if zr(*args_r[i]) != 0 or za(*args_a[i]) != 0:
            raise RuntimeError("launch failed")

    def timed(calls):
        """Device time of the given launches, back to back, between two events."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        device_wait(torch)
        e0.record()
        for fn, a in calls:
            if fn(*a) != 0:
                raise RuntimeError("launch failed")
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    for i in range(warmup):
        step(i)
        if zf(*args_f[i]) != 0:
            raise RuntimeError("launch failed")
    torch.cuda.synchronize()
    # The timed steps: zha_route followed by zha_attn per step, no event
    # between them (an event recorded between two launches costs the stream
    # ~3.5 us).  Then the same steps as one zha_route_attn call each (routing
    # and attention in one launch).
    timed_ids = range(warmup, warmup + steps)
    total_ms = timed([c for i in timed_ids for c in ((zr, args_r[i]), (za, args_a[i]))])
    fused_ms = timed([(zf, args_f[i]) for i in timed_ids])
    # The same steps as two micro-batches, sequences [0, B/2) and [B/2, B), each
    # a chain of zha_route then zha_attn per step on a stream of its own (both at
    # the default priority): one half's routing, bound by its dependent levels,
    # runs beside the other half's attention, bound by HBM.  The sequences are
    # independent, so a decode loop can run them this way layer after layer; the
    # routes are those of the full-batch calls, the outputs equal theirs up to
    # fp32 summation order (the balanced split differs).
    pipe_ms = None
    if g.B >= 2 and g.B % 2 == 0:
        hb = g.B // 2
        gmh = Z.geom(W.replace(g, B=hb))
        tbh, _ = Z.tree_bytes(gmh)
        if 2 * tbh != tb:
            raise RuntimeError("half-batch tree layout does not split the full one")
        seq_kv = Kd[0].numel() * Kd.element_size()
        s_half = [torch.cuda.current_stream(), torch.cuda.Stream()]
        scr = [(torch.empty(max(Z.route_scratch_bytes(gmh, 1, cap), 1), dtype=torch.uint8,
                            device="cuda"),
                torch.zeros(max(Z.attn_scratch_bytes(gmh, 1, cap), 1), dtype=torch.uint8,
                            device="cuda")) for _ in range(2)]
        gref_h = ctypes.byref(gmh)
        half_calls = []
        for i in range(n):
            k, v, t = layers[i % n_layers]
            for h in range(2):
                o = h * hb
                st = vp(s_half[h].cuda_stream)
                half_calls.append((
                    (zr, (gref_h, vp(t.data_ptr() + h * tbh), vp(Qd[i, o].data_ptr()), 1, None,
                          ctypes.c_float(g.p), vp(sel[i, o].data_ptr()), vp(cnt[i, o].data_ptr()),
                          cap, vp(stats[i, o].data_ptr()), None, vp(scr[h][0].data_ptr()), st)),
                    (za, (gref_h, vp(Qd[i, o].data_ptr()), 1, None,
                          vp(k.data_ptr() + o * seq_kv), vp(v.data_ptr() + o * seq_kv),
                          vp(sel[i, o].data_ptr()), vp(cnt[i, o].data_ptr()), cap,
                          vp(O[i, o].data_ptr()), vp(scr[h][1].data_ptr()), st))))

        def run_half(ids):
            for i in ids:
                for h in range(2):
                    for fn, a in half_calls[2 * i + h]:
                        if fn(*a) != 0:
                            raise RuntimeError("launch failed")

        run_half(range(warmup))
        torch.cuda.synchronize()
        p0 = torch.cuda.Event(enable_timing=True)
        p_end = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        device_wait(torch)
        p0.record(s_half[0])
        s_half[1].wait_event(p0)
        run_half(timed_ids)
        for h in range(2):
            p_end[h].record(s_half[h])
        torch.cuda.synchronize()
        pipe_ms = max(p0.elapsed_time(e) for e in p_end)
        log(f"[bench] {steps} steps as two micro-batches on two streams: "
            f"{pipe_ms / steps * 1e3:.1f} us per step")
        del scr

    # The split, each call kind timed back to back over the same steps (the
    # attention calls reuse the routes computed above).
    route_ms = np.full(steps, timed([(zr, args_r[i]) for i in timed_ids]) / steps)
    attn_ms = np.full(steps, timed([(za, args_a[i]) for i in timed_ids]) / steps)
    log(f"[bench] {steps} steps: {total_ms:.3f} ms total ({total_ms / steps * 1e3:.1f} us per step "
        f"as zha_route + zha_attn, {fused_ms / steps * 1e3:.1f} us in zha_route_attn); "
        f"route alone {route_ms.mean() * 1e3:.1f} us, attn alone {attn_ms.mean() * 1e3:.1f} us per call")

    # The same calls fully cache-cold: 1 GiB written before each call (outside
    # its timing) evicts L2 and the memory-side cache; each call between two
    # events of its own.
    flush = None if lean else torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    n_cold = 0 if lean else min(steps, 10)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_cold)]
    for j in range(n_cold):
        i = warmup + j
        for k, (fn, a) in enumerate(((zr, args_r[i]), (za, args_a[i]), (zf, args_f[i]))):
            flush.fill_((3 * j + k) & 255)
            evc[j][2 * k].record()
            if fn(*a) != 0:
                raise RuntimeError("launch failed")
            evc[j][2 * k + 1].record()
    torch.cuda.synchronize()
    cold_route = np.array([e[0].elapsed_time(e[1]) for e in evc])
    cold_attn = np.array([e[2].elapsed_time(e[3]) for e in evc])
    cold_fused = np.array([e[4].elapsed_time(e[5]) for e in evc])
    copy_gbs = None
    if not lean:
        log(f"[bench] {n_cold} cold steps: route {cold_route.mean() * 1e3:.1f} us, "
            f"attn {cold_attn.mean() * 1e3:.1f} us, zha_route_attn "
            f"{cold_fused.mean() * 1e3:.1f} us per step")
        # Streaming-copy bandwidth of this device (read + write bytes of a 1 GiB copy).
        dst = torch.empty_like(flush)
        dst.copy_(flush)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            dst.copy_(flush)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * 5 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del dst
    del flush, layers
    torch.cuda.empty_cache()

    cnt_h = cnt.cpu().numpy()
    if (cnt_h[warmup:] < 0).any() or (cnt_h[warmup:] > cap).any():
        raise RuntimeError("a route failed (cnt < 0) or its count exceeds the chunk-list cap")
    sel_h = sel.cpu().numpy()
    stats_h = stats.cpu().numpy()
    acc = {"attn_union": 0, "attn_per_head": 0, "route": 0, "tokens_per_head": 0.0}
    for j in range(steps):
        i = warmup + j
        b = step_bytes(g, sel_h[i], cnt_h[i], stats_h[i])
        for k in acc:
            acc[k] += b[k]
    for k in acc:
        acc[k] /= steps
    if not np.isfinite(O.float().cpu().numpy()).all():
        raise RuntimeError("non-finite attention output")

    dense_ms = None
    if dense_steps > 0:
        dscratch = torch.zeros(max(Z.dense_scratch_bytes(gm, 1), 1), dtype=torch.uint8,
                               device="cuda")
        Od = torch.empty((g.B, 1, g.H_q, g.d), dtype=Kd.dtype, device="cuda")
        Z.dense_decode(gm, Qd[0], 1, Kd, Vd, O=Od, scratch=dscratch)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        device_wait(torch)
        d0.record()
        for j in range(dense_steps):
            Z.dense_decode(gm, Qd[warmup + j % steps], 1, Kd, Vd, O=Od, scratch=dscratch)
        d1.record()
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / dense_steps
        log(f"[bench] dense decode {dense_ms * 1e3:.1f} us per step")
    maint = None if lean else decode_maintenance(Z, g, gm, Kd, qref, tree, bscratch)
    return {"total_ms": total_ms, "fused_ms": fused_ms, "pipe_ms": pipe_ms,
            "cold_fused_ms": cold_fused,
            "route_ms": route_ms, "attn_ms": attn_ms, "bytes": acc,
            "build_ms": build_ms, "dense_ms": dense_ms, "cap": cap, "cold_route_ms": cold_route,
            "cold_attn_ms": cold_attn, "copy_gbs": copy_gbs, "maintenance": maint,
            "n_layers": n_layers}


def run_decode_leg(cfg: int, warmup: int = 3, dense_steps: int = 2):
    """One of the other decode workloads at its own size: every one of its decode steps timed
    back to back (route + attention per step, the same calls as the headline), its tree build,
    zha_route_attn over the same steps and dense decode of the same cache."""
    g = W.CONFIGS[cfg]
    t0 = time.perf_counter()
    K, V = W.make_kv(g)
    log(f"[bench] {g.name}: generated K, V ({2 * K.nbytes / 1e9:.2f} GB) in "
        f"{time.perf_counter() - t0:.1f} s")
    r = run_gpu(g, K, V, g.n_steps, warmup, dense_steps, lean=True)
    del K, V
    us = r["total_ms"] / g.n_steps * 1e3
    by = r["bytes"]
    union = by["attn_union"] + by["route"]
    return {"workload": f"{g.name}: B={g.B}, H_q={g.H_q}/H_kv={g.H_kv}, d={g.d}, T={g.T}, "
                        f"C={g.C}, L={g.L}, p={g.p}, {g.dtype}, {g.n_steps} decode steps",
            "steps": g.n_steps,
            "queries_per_s": g.B / (us * 1e-6),
            "us_per_step": us,
            "route_us": float(r["route_ms"].mean() * 1e3),
            "attn_us": float(r["attn_ms"].mean() * 1e3),
            "route_attn_us_per_step": r["fused_ms"] / g.n_steps * 1e3,
            "build_ms": r["build_ms"],
            "step_bytes_union": union,
            "step_hbm_frac": union / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
            "tokens_per_head": by["tokens_per_head"],
            "dense_us_per_step": r["dense_ms"] * 1e3 if r["dense_ms"] else None,
            "speedup_vs_dense": (r["dense_ms"] * 1e3 / us) if r["dense_ms"] else None,
            "n_layers": r["n_layers"]}


def decode_maintenance(Z, g, gm, Kd, qref, tree, bscratch, reps: int = 200):
    """Tree-maintenance cost of decode (the paper App. D-B2, amortized decode tree cost):
    t_summ(1) is a zha_tree_update whose appended token completes one leaf per tree, t_full one
    that completes a node at every level; t_merge(1) = (t_full - t_summ) / (L - 1).  The amortized
    cost per decoded token is t_summ / C + t_merge * sum_{l=2..L} C^-l.  The updates rewrite nodes
    that already hold the same values, so the tree stays valid."""
    import torch
    C, L, T = g.C, g.L, g.T
    t_leaf = (T // C) * C
    if L > 1 and t_leaf % (C * C) == 0:
        t_leaf -= C
    t_top = (T // C ** L) * C ** L

    import ctypes
    lib = Z.load()
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)

    def timed(t_new):
        gt = Z.with_length(gm, t_new)
        Z.tree_update(gt, t_new - 1, Kd, qref, tree, bscratch)  # checked once through the binding
        torch.cuda.synchronize()
        args = (ctypes.byref(gt), ctypes.c_int64(t_new - 1), vp(Kd.data_ptr()),
                None if qref is None else vp(qref.data_ptr()), None, vp(tree.data_ptr()),
                vp(bscratch.data_ptr()), stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # A short device-side wait first, so that every call is queued before the first
        # runs: the events then time the device work, not the host's submission rate.
        torch.cuda._sleep(int(1e7))
        e0.record()
        for _ in range(reps):
            if lib.zha_tree_update(*args) != 0:
                raise RuntimeError("zha_tree_update failed")
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    t_summ = timed(t_leaf)
    t_full = timed(t_top)
    t_merge = (t_full - t_summ) / (L - 1) if L > 1 else 0.0
    amort = t_summ / C + t_merge * sum(C ** -l for l in range(2, L + 1))
    log(f"[bench] decode maintenance: one leaf per tree {t_summ:.1f} us, a node at all {L} levels "
        f"{t_full:.1f} us; amortized {amort:.2f} us per decoded token")
    return {"t_summ_us": t_summ, "t_full_update_us": t_full, "t_merge_us": t_merge,
            "amortized_us_per_token": amort,
            "how": f"mean of {reps} zha_tree_update C-ABI calls queued behind a device-side wait "
                   f"(device time, launches included), {g.B * g.H_kv} trees; "
                   "amortized = t_summ / C + t_merge * sum over l = 2..L of C^-l"}


def run_block_1m(reps: int = 3):
    """Secondary figure: the 1M-token cache with a block of 2048 new positions (16 query heads
    over 2 KV heads, C=32, L=4, p=0.95) routed and attended as one call pair per KV head on two
    streams, and as one call pair for all heads; the tree is built from scratch on the cache.
    Queries/s counts the 2048 positions."""
    import torch

    from hierarchical_tree_indexed_04_amd import zha as Z
    g = W.CONFIGS[4]
    t0 = time.perf_counter()
    K, V = W.make_kv(g)
    Qn = W.make_query_block(g, K, range(g.n_steps))
    log(f"[bench] {g.name}: inputs {time.perf_counter() - t0:.1f} s")
    gm = Z.geom(g)
    Kd, Vd, Qd = to_dev(torch, K, g.dtype), to_dev(torch, V, g.dtype), to_dev(torch, Qn, g.dtype)
    n_pos = g.n_steps
    cap = 2048
    tb, sb = Z.tree_bytes(gm)
    tree = torch.empty(tb, dtype=torch.uint8, device="cuda")
    bsc = torch.empty(max(sb, 1), dtype=torch.uint8, device="cuda")
    qref = None  # the zero reference (R = 1)
    sel = torch.empty((g.B, n_pos, g.H_q, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((g.B, n_pos, g.H_q), dtype=torch.int32, device="cuda")
    stats = torch.empty((g.B, n_pos, g.H_q, g.L, 2), dtype=torch.int32, device="cuda")
    O = torch.empty((g.B, n_pos, g.H_q, g.d), dtype=Kd.dtype, device="cuda")
    asc = torch.empty(max(Z.attn_scratch_bytes(gm, n_pos, cap), 1), dtype=torch.uint8, device="cuda")

    def once():
        Z.build(gm, Kd, qref, tree, bsc)
        e1.record()
        Z.route(gm, tree, Qd, n_pos, g.p, cap, out=(sel, cnt, stats, None))
        e2.record()
        Z.attn(gm, Qd, n_pos, Kd, Vd, sel, cnt, cap, O=O, scratch=asc)

    e0, e1, e2, e3 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    once()
    torch.cuda.synchronize()
    tb_ms, tr_ms, ta_ms = [], [], []
    for _ in range(reps):
        device_wait(torch)
        e0.record()
        once()
        e3.record()
        torch.cuda.synchronize()
        tb_ms.append(e0.elapsed_time(e1))
        tr_ms.append(e1.elapsed_time(e2))
        ta_ms.append(e2.elapsed_time(e3))
    # The same block as one call pair per KV head (8 query heads over 1 KV head
    # each), the two pairs on two streams: the KV groups share nothing, so one
    # group's routing (VALU-bound) and bookkeeping run beside the other group's
    # attention (HBM-bound).  The queries are laid out per KV head beforehand
    # (outside the timing); routes and outputs are those of the single call.
    g1 = W.replace(g, H_q=g.G, H_kv=1)
    gm1 = Z.geom(g1)
    tb1, _ = Z.tree_bytes(gm1)
    if tb1 * g.H_kv != tb:
        raise RuntimeError("per-KV-head tree layout does not split the full one")
    kv_head = Kd[0, 0].numel() * Kd.element_size()
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(g.H_kv - 1)]
    per = []
    for k in range(g.H_kv):
        qk = Qd[:, :, k * g.G:(k + 1) * g.G].contiguous()
        sk = torch.empty((g.B, n_pos, g.G, cap), dtype=torch.int32, device="cuda")
        ck = torch.empty((g.B, n_pos, g.G), dtype=torch.int32, device="cuda")
        ok = torch.empty((g.B, n_pos, g.G, g.d), dtype=Kd.dtype, device="cuda")
        rk = torch.empty(max(Z.route_scratch_bytes(gm1, n_pos, cap), 1), dtype=torch.uint8,
                         device="cuda")
        ak = torch.empty(max(Z.attn_scratch_bytes(gm1, n_pos, cap), 1), dtype=torch.uint8,
                         device="cuda")
        per.append((qk, sk, ck, ok, rk, ak))
    tree_k = [tree[k * tb1:(k + 1) * tb1] for k in range(g.H_kv)]
    K_k = [Kd[:, k:k + 1] for k in range(g.H_kv)]
    V_k = [Vd[:, k:k + 1] for k in range(g.H_kv)]

    def split_once():
        for k in range(g.H_kv):
            qk, sk, ck, ok, rk, ak = per[k]
            Z.route(gm1, tree_k[k], qk, n_pos, g.p, cap, out=(sk, ck, None, None), scratch=rk,
                    stream=streams[k])
            Z.attn(gm1, qk, n_pos, K_k[k], V_k[k], sk, ck, cap, O=ok, scratch=ak,
                   stream=streams[k])

    split_once()
    torch.cuda.synchronize()
    ts_ms = []
    for _ in range(reps):
        s0 = torch.cuda.Event(enable_timing=True)
        s_end = [torch.cuda.Event(enable_timing=True) for _ in range(g.H_kv)]
        device_wait(torch, 1000.0)  # covers the host's submission of the four calls
        s0.record(streams[0])
        for st in streams[1:]:
            st.wait_event(s0)
        split_once()
        for k in range(g.H_kv):
            s_end[k].record(streams[k])
        torch.cuda.synchronize()
        ts_ms.append(max(s0.elapsed_time(e) for e in s_end))
    split_ms = float(np.median(ts_ms))
    c_split = torch.cat([per[k][2] for k in range(g.H_kv)], dim=2)
    o_split = torch.cat([per[k][3] for k in range(g.H_kv)], dim=2)
    if not torch.equal(c_split, cnt) or float((o_split.float() - O.float()).abs().max()) > 2e-2:
        raise RuntimeError("1M block: the per-KV-head calls disagree with the single call")
    log(f"[bench] 1M block as one call pair per KV head on {g.H_kv} streams: "
        f"{split_ms:.3f} ms (route + attn)")

    c = cnt.cpu().numpy()
    if (c < 0).any() or (c > cap).any():
        raise RuntimeError("1M block: a route overflowed")
    s_h = sel.cpu().numpy()
    n1 = g.n_level(1)
    union = 0
    for kvh in range(g.H_kv):
        mark = np.zeros(n1, bool)
        for h in range(kvh * g.G, (kvh + 1) * g.G):
            for t in range(n_pos):
                mark[s_h[0, t, h, :c[0, t, h]]] = True
        # Tokens of the group's selected chunks, the partial chunk, and the sink
        # where no head selected chunk 0.
        toks = int(mark.sum()) * g.C + (g.T - n1 * g.C) + (0 if mark[0] else 1)
        union += toks * 2 * g.d * g.elem_bytes
    per_head = int(c.sum()) * g.C * 2 * g.d * g.elem_bytes
    route_rows = int(stats.cpu().numpy()[..., 0].sum()) * (g.d * g.elem_bytes + 4)
    # Summary rows touched by some head: at most the whole tree (the heads'
    # frontiers overlap; their per-head sum counts shared rows many times).
    route_union = min(route_rows, tb)
    b_ms, r_ms, a_ms = (float(np.median(x)) for x in (tb_ms, tr_ms, ta_ms))
    log(f"[bench] 1M block: build {b_ms:.3f} ms, route {r_ms:.3f} ms, attn {a_ms:.3f} ms")
    return {"workload": f"{g.name}: B={g.B}, H_q={g.H_q}/H_kv={g.H_kv}, d={g.d}, T={g.T}, C={g.C}, "
                        f"L={g.L}, p={g.p}, {n_pos} positions per call",
            "schedule": f"one zha_route + zha_attn pair per KV head ({g.G} query heads each), "
                        f"the {g.H_kv} pairs on {g.H_kv} streams",
            "queries_per_s": n_pos / (split_ms * 1e-3),
            "route_attn_ms": split_ms,
            "queries_per_s_with_build": n_pos / ((b_ms + split_ms) * 1e-3),
            "single_call": {"queries_per_s": n_pos / ((r_ms + a_ms) * 1e-3),
                            "route_ms": r_ms, "attn_ms": a_ms,
                            "hbm_frac_union": (union + route_union) / ((r_ms + a_ms) * 1e-3)
                            / (HBM_PEAK_GBS * 1e9)},
            "build_ms": b_ms, "route_ms": r_ms, "attn_ms": a_ms,
            "bytes_union": union + route_union, "bytes_kv_union": union,
            "bytes_route_rows_per_head_sum": route_rows, "bytes_tree": tb,
            "bytes_per_head_sum": per_head + route_rows,
            "hbm_frac_union": (union + route_union) / (split_ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
            "how_union": "K/V rows of the tokens any head of a KV group attends (its selected "
                         "chunks, the partial chunk and the sink), plus the summary rows touched "
                         "(at most the tree's bytes)"}


CROSSOVER_T = [4096, 8192, 16384, 32768, 65536, 131072, 262144]


def crossover_geometry(T: int):
    """The deep-decode geometry (B=8, 32/4 heads, d=128, C=8, p=0.95, bf16) at context T, with the
    deepest L such that C^L <= T (T / C^L top nodes)."""
    from dataclasses import replace
    base = W.CONFIGS[3]
    L = 1
    while base.C ** (L + 1) <= T:
        L += 1
    return replace(base, name=f"deep-decode-{T // 1024}k", T=T, L=L)


def run_crossover(steps: int):
    """ZHA route + attention against dense decode, one decode step per call, cache-cold (1 GiB
    written between calls, outside the timed region), over CROSSOVER_T."""
    import torch

    from hierarchical_tree_indexed_04_amd import zha as Z
    Z.load()
    torch.cuda.set_device(0)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def ev():
        return torch.cuda.Event(enable_timing=True)

    rows = []
    for T in CROSSOVER_T:
        g = crossover_geometry(T)
        K, V = W.make_kv(g)
        Qs = np.stack([W.make_queries(g, K, i) for i in range(steps)])[:, :, None]
        gm = Z.geom(g)
        Kd, Vd, Qd = to_dev(torch, K, g.dtype), to_dev(torch, V, g.dtype), to_dev(torch, Qs, g.dtype)
        del K, V
        tree = Z.build(gm, Kd, torch.zeros((g.H_kv, g.R, g.d), dtype=torch.float32, device="cuda"))
        cap = g.n_level(1)
        sel = torch.empty((g.B, 1, g.H_q, cap), dtype=torch.int32, device="cuda")
        cnt = torch.empty((g.B, 1, g.H_q), dtype=torch.int32, device="cuda")
        stats = torch.empty((g.B, 1, g.H_q, g.L, 2), dtype=torch.int32, device="cuda")
        O = torch.empty((g.B, 1, g.H_q, g.d), dtype=Kd.dtype, device="cuda")
        rsc = torch.empty(max(Z.route_scratch_bytes(gm, 1, cap), 1), dtype=torch.uint8,
                          device="cuda")
        asc = torch.empty(max(Z.attn_scratch_bytes(gm, 1, cap), 1), dtype=torch.uint8,
                          device="cuda")
        dsc = torch.empty(max(Z.dense_scratch_bytes(gm, 1), 1), dtype=torch.uint8, device="cuda")

        def zha(i):
            Z.route(gm, tree, Qd[i], 1, g.p, cap, want_stats=False, want_gap=False,
                    out=(sel, cnt, stats, None), scratch=rsc)
            return Z.attn(gm, Qd[i], 1, Kd, Vd, sel, cnt, cap, O=O, scratch=asc)

        zha(0)
        Z.dense_decode(gm, Qd[0], 1, Kd, Vd, O=O, scratch=dsc)
        torch.cuda.synchronize()
        er = [[ev() for _ in range(3)] for _ in range(steps)]
        ed = [[ev() for _ in range(2)] for _ in range(steps)]
        toks = 0
        k_lv, s_lv, k0_union = np.zeros(g.L), np.zeros(g.L), 0.0
        for i in range(steps):
            flush.fill_(i & 255)
            er[i][0].record()
            Z.route(gm, tree, Qd[i], 1, g.p, cap, want_stats=False, want_gap=False,
                    out=(sel, cnt, stats, None), scratch=rsc)
            er[i][1].record()
            Z.attn(gm, Qd[i], 1, Kd, Vd, sel, cnt, cap, O=O, scratch=asc)
            er[i][2].record()
            toks += int(cnt.sum().item()) * g.C
            st = stats.cpu().numpy().reshape(-1, g.L, 2)
            k_lv += st[:, :, 0].mean(axis=0) / steps
            s_lv += st[:, :, 1].mean(axis=0) / steps
            k0_union += step_bytes(g, sel.cpu().numpy(), cnt.cpu().numpy(),
                                   stats.cpu().numpy())["attn_union"] / steps
            flush.fill_((i + 7) & 255)
            ed[i][0].record()
            Z.dense_decode(gm, Qd[i], 1, Kd, Vd, O=O, scratch=dsc)
            ed[i][1].record()
        torch.cuda.synchronize()
        r_us = float(np.median([e[0].elapsed_time(e[1]) for e in er]) * 1e3)
        a_us = float(np.median([e[1].elapsed_time(e[2]) for e in er]) * 1e3)
        z_us = float(np.median([e[0].elapsed_time(e[2]) for e in er]) * 1e3)
        d_us = float(np.median([e[0].elapsed_time(e[1]) for e in ed]) * 1e3)
        row = {"T": T, "L": g.L, "top_nodes": g.n_level(g.L), "zha_us": z_us, "route_us": r_us,
               "attn_us": a_us, "dense_us": d_us, "speedup_vs_dense": d_us / z_us,
               "keys_attended_frac": toks / steps / (g.B * g.H_q) / T,
               "frontier_per_level": [float(x) for x in k_lv],  # K_l, level 1 first
               "kept_per_level": [float(x) for x in s_lv],
               "attn_union_bytes": float(k0_union)}
        log(f"[crossover] T={T:7d} L={g.L}: zha {z_us:8.1f} us (route {r_us:6.1f}, attn "
            f"{a_us:6.1f}), dense {d_us:8.1f} us, x{d_us / z_us:.2f}")
        rows.append(row)
        del Kd, Vd, Qd, tree
        torch.cuda.empty_cache()
    # Smallest T from which ZHA is faster at every larger T measured.
    crossing = None
    for k in range(len(rows)):
        if all(r["zha_us"] < r["dense_us"] for r in rows[k:]):
            crossing = rows[k]["T"]
            break
    print(json.dumps({"crossover": rows, "zha_faster_from_T": crossing,
                      "workload": "deep-decode geometry (B=8, H_q=32/H_kv=4, d=128, C=8, p=0.95, "
                                  "bf16), L = deepest with 8^L <= T, one decode step per call",
                      "timing": f"median over {steps} steps, cache-cold (1 GiB written between "
                                "calls)"}), flush=True)


def run_prefill(block: int, reps: int):
    """Causal prefill of the 128K GQA workload (B=1, H_q=32/H_kv=4, d=128, T=131072, C=32,
    L=3, p=0.95): every cached token is also a query seeing the tokens up to itself (ctx_len =
    t + 1), routed and attended in calls of `block` positions over a tree built once on the
    prompt.  Queries 3 k_j + N(0, 0.3^2) with j uniform over the visible tokens, drawn on the
    device from a seeded generator."""
    import torch

    from hierarchical_tree_indexed_04_amd import zha as Z
    Z.load()
    torch.cuda.set_device(0)
    g = W.CONFIGS[2]
    K, V = W.make_kv(g)
    gm = Z.geom(g)
    Kd, Vd = to_dev(torch, K, g.dtype), to_dev(torch, V, g.dtype)
    del K, V
    T = g.T
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20240)
    t = torch.arange(T, device="cuda")
    j = torch.minimum((torch.rand((T, g.H_q), generator=gen, device="cuda")
                       * (t[:, None] + 1)).long(), t[:, None])
    kvh = (torch.arange(g.H_q, device="cuda") // g.G)[None, :]
    Qd = (3.0 * Kd[0][kvh, j].float() + 0.3 * torch.randn((T, g.H_q, g.d), generator=gen,
                                                            device="cuda")).to(Kd.dtype)[None]
    ctx = (t + 1).to(torch.int32)[None].contiguous()
    del j
    qref = None  # the zero reference (R = 1)
    tb, sb = Z.tree_bytes(gm)
    tree = torch.empty(tb, dtype=torch.uint8, device="cuda")
    bsc = torch.empty(max(sb, 1), dtype=torch.uint8, device="cuda")
    cap = 1024
    sel = torch.empty((1, block, g.H_q, cap), dtype=torch.int32, device="cuda")
    cnt_all = torch.empty((1, T, g.H_q), dtype=torch.int32, device="cuda")
    O = torch.empty((1, T, g.H_q, g.d), dtype=Kd.dtype, device="cuda")
    rsc = torch.empty(max(Z.route_scratch_bytes(gm, block, cap), 1), dtype=torch.uint8,
                      device="cuda")
    asc = torch.empty(max(Z.attn_scratch_bytes(gm, block, cap), 1), dtype=torch.uint8,
                      device="cuda")
    starts = list(range(0, T, block))

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def prefill(evs=None):
        Z.build(gm, Kd, qref, tree, bsc)
        if evs:
            evs[0].record()
        for i, t0 in enumerate(starts):
            n = min(block, T - t0)
            Qb, cb = Qd[:, t0:t0 + n], ctx[:, t0:t0 + n]
            sb_, cnt = sel[:, :n], cnt_all[:, t0:t0 + n]
            Z.route(gm, tree, Qb, n, g.p, cap, want_stats=False, want_gap=False,
                    out=(sb_, cnt, None, None), scratch=rsc, ctx_len=cb)
            if evs:
                evs[1 + 2 * i].record()
            Z.attn(gm, Qb, n, Kd, Vd, sb_, cnt, cap, O=O[:, t0:t0 + n], scratch=asc, ctx_len=cb)
            if evs:
                evs[2 + 2 * i].record()

    prefill()
    torch.cuda.synchronize()
    c = cnt_all.cpu().numpy()
    if (c < 0).any() or (c > cap).any():
        raise RuntimeError("prefill: a route failed (cnt < 0) or its count exceeds the list cap")
    if not torch.isfinite(O).all():
        raise RuntimeError("prefill: non-finite output")
    tail = (np.arange(1, T + 1) % g.C)[None, :, None]
    toks = c.astype(np.int64) * g.C + tail  # + the sink when chunk 0 is not selected
    e_start, e_end = ev(), ev()
    totals, builds, routes, attns = [], [], [], []
    for _ in range(reps):
        evs = [ev() for _ in range(1 + 2 * len(starts))]
        e_start.record()
        prefill(evs)
        e_end.record()
        torch.cuda.synchronize()
        totals.append(e_start.elapsed_time(e_end))
        builds.append(e_start.elapsed_time(evs[0]))
        routes.append(sum(evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(len(starts))))
        attns.append(sum(evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(len(starts))))
    tot, b_ms, r_ms, a_ms = (float(np.median(x)) for x in (totals, builds, routes, attns))
    log(f"[prefill] {T} tokens in {len(starts)} calls of {block}: {tot:.2f} ms (build {b_ms:.2f}, "
        f"route {r_ms:.2f}, attn {a_ms:.2f}); {T / (tot * 1e-3) / 1e6:.2f} M tokens/s")

    # The same calls alternated over two streams (each with its own chunk lists
    # and scratch), after the build: the calls are independent, so one call's
    # routing (bound by instruction issue) runs beside the other's attention
    # (bound by HBM).
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    bufs = [(sel, rsc, asc)] + [(torch.empty_like(sel), torch.empty_like(rsc),
                                 torch.empty_like(asc))]

    def prefill2():
        Z.build(gm, Kd, qref, tree, bsc)
        built = torch.cuda.Event()
        built.record(streams[0])
        streams[1].wait_event(built)
        for i, t0 in enumerate(starts):
            n = min(block, T - t0)
            Qb, cb = Qd[:, t0:t0 + n], ctx[:, t0:t0 + n]
            sl, rs, as_ = bufs[i % 2]
            sb_, cnt = sl[:, :n], cnt_all[:, t0:t0 + n]
            Z.route(gm, tree, Qb, n, g.p, cap, want_stats=False, want_gap=False,
                    out=(sb_, cnt, None, None), scratch=rs, ctx_len=cb, stream=streams[i % 2])
            Z.attn(gm, Qb, n, Kd, Vd, sb_, cnt, cap, O=O[:, t0:t0 + n], scratch=as_,
                   ctx_len=cb, stream=streams[i % 2])

    O_serial = O.clone()
    cnt_serial = cnt_all.clone()
    prefill2()
    torch.cuda.synchronize()
    if not torch.equal(cnt_all, cnt_serial) or float((O.float() - O_serial.float()).abs().max()) > 2e-2:
        raise RuntimeError("prefill on two streams disagrees with the serial calls")
    del O_serial, cnt_serial
    totals2 = []
    for _ in range(reps):
        e0 = ev()
        ends = [ev(), ev()]
        device_wait(torch)
        e0.record(streams[0])
        prefill2()
        for e, st in zip(ends, streams):
            e.record(st)
        torch.cuda.synchronize()
        totals2.append(max(e0.elapsed_time(e) for e in ends))
    tot2 = float(np.median(totals2))
    log(f"[prefill] the same calls alternated over two streams: {tot2:.2f} ms; "
        f"{T / (tot2 * 1e-3) / 1e6:.2f} M tokens/s")
    print(json.dumps({
        "prefill": {"tokens_per_s": T / (tot * 1e-3), "ms": tot, "build_ms": b_ms,
                    "route_ms": r_ms, "attn_ms": a_ms, "calls": len(starts),
                    "two_streams_ms": tot2, "two_streams_tokens_per_s": T / (tot2 * 1e-3),
                    "positions_per_call": block, "cap": cap,
                    "keys_attended_frac_mean": float(np.mean(toks / np.arange(1, T + 1)[None, :, None])),
                    "tokens_per_query_head_mean": float(toks.mean())},
        "workload": f"causal prefill of {g.name}: B={g.B}, H_q={g.H_q}/H_kv={g.H_kv}, d={g.d}, "
                    f"T={T}, C={g.C}, L={g.L}, p={g.p}, bf16; query at position t sees t + 1 tokens",
        "timing": f"median of {reps} full prefills (tree build + every call), HIP events"}),
        flush=True)


def copy_calibration():
    """One plain copy of 1 GiB: reads and writes 2^30 bytes each, for scaling HBM counters."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: 256K)")
    ap.add_argument("--dense-steps", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the oracle baseline (0 disables)")
    ap.add_argument("--refs", type=int, default=0, metavar="R",
                    help="reference queries per KV head (0: the workload's own R = 1 with the zero "
                         "reference; R > 1 draws them like queries)")
    ap.add_argument("--with-1m", type=int, default=1,
                    help="also time the 1M-context block workload (2048 positions routed at once)")
    ap.add_argument("--with-configs", type=int, default=1,
                    help="also time the other decode workloads (4K fp32, 128K GQA, 16.7M) at "
                         "their own sizes and step counts")
    ap.add_argument("--crossover", action="store_true",
                    help="only run the context-length sweep of ZHA against dense decode")
    ap.add_argument("--prefill", type=int, default=0, metavar="BLOCK",
                    help="only run a causal prefill of the 128K workload in calls of BLOCK "
                         "positions")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.crossover:
        run_crossover(max(3, min(args.steps, 20)))
        return
    if args.prefill:
        run_prefill(args.prefill, max(1, min(args.steps, 5)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU: the hot path has no multi-GPU mode "
            "(run with --gpus 1)")
        sys.exit(2)
    g = W.CONFIGS[args.config]
    if args.refs > 0:
        g = W.replace(g, R=args.refs)
    if g.block:
        log("the chunked-query block workload is not a decode-step benchmark yet")
        sys.exit(2)
    t0 = time.perf_counter()
    K, V = W.make_kv(g)
    log(f"[bench] {g.name}: generated K, V ({2 * K.nbytes / 1e9:.2f} GB) in "
        f"{time.perf_counter() - t0:.1f} s")

    cpu = None
    if args.cpu_seconds > 0:
        procs = max(1, min(16, os.cpu_count() or 1))
        t0 = time.perf_counter()
        cpu = cpu_baseline(g, K, V, args.cpu_seconds, procs)
        one = cpu_baseline(g, K, V, max(2.0, args.cpu_seconds / 3), 1)
        cpu["one_core_value"] = one["value"]
        cpu["one_core_sample"] = one["sample"]
        cpu["host_cpus"] = os.cpu_count()
        cpu["cpu_model"] = cpu_model()
        log(f"[bench] oracle baseline {cpu['value']:.2f} queries/s on {procs} processes, "
            f"{one['value']:.2f} on one ({time.perf_counter() - t0:.1f} s)")

    r = run_gpu(g, K, V, args.steps, args.warmup, args.dense_steps)
    # The step: the batch as two micro-batches on two streams where it splits
    # (run_gpu), else the full-batch calls on one stream.
    step_ms = r["pipe_ms"] if r["pipe_ms"] is not None else r["total_ms"]
    ms_per_step = step_ms / args.steps
    queries_per_step = g.B  # one query = one token position x all H_q heads
    value = queries_per_step * args.steps / (step_ms / 1e3)
    by = r["bytes"]
    attn_us = float(r["attn_ms"].mean() * 1e3)
    route_us = float(r["route_ms"].mean() * 1e3)
    step_union = by["attn_union"] + by["route"]
    achieved = step_union / (ms_per_step * 1e-3) / 1e9
    achieved_attn = by["attn_union"] / (attn_us * 1e-6) / 1e9
    # The committed counter record covers the default workload (256K, R = 1) only.
    tr = measured_traffic() if args.config == 3 and args.refs == 0 else None
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": g.dtype,
        "data": "synthetic",
        "config": {"workload": f"{g.name}: B={g.B}, H_q={g.H_q}/H_kv={g.H_kv}, d={g.d}, T={g.T}, "
                               f"C={g.C}, L={g.L}, R={g.R}, p={g.p}, one decode step per call, "
                               f"steps cycling through {r['n_layers']} layers' KV caches and trees",
                   "global_batch": g.B, "seq_len": g.T, "parallelism": "single GPU"},
        # The step as a whole: the bytes routing and attention must move (step_bytes)
        # over the timed step (zha_route then zha_attn, back to back, HIP events).
        "step_schedule": ("two micro-batches of B/2 sequences on two streams, each zha_route "
                          "then zha_attn per step" if r["pipe_ms"] is not None else
                          "zha_route then zha_attn per step, one stream"),
        "ms_per_step_one_stream": r["total_ms"] / args.steps,
        "value_one_stream": g.B * args.steps / (r["total_ms"] / 1e3),
        "roofline": {"bound": "hbm",
                     "kernel": "decode step (the step_schedule above): zha_route "
                               "(lat::route_kernel) + zha_attn (attn_balanced_kernel + "
                               "merge_balanced_kernel)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": tr["step_bytes"] if tr else None,
                     "bytes": step_union},
        # The dominant call alone: attention's union bytes over the zha_attn call time.
        "roofline_attn": {"bound": "hbm",
                          "kernel": "zha_attn call (attn_balanced_kernel + merge_balanced_kernel)",
                          "achieved": achieved_attn, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": achieved_attn / HBM_PEAK_GBS,
                          "traffic": tr["attn_bytes_per_call"] if tr else None,
                          "bytes": by["attn_union"]},
        "cpu_baseline": cpu,
        "route_attn_us_per_step": r["fused_ms"] / args.steps * 1e3,
        "route_us": route_us,
        "attn_us": attn_us,
        "step_bytes_union": step_union,
        "attn_bytes_union": by["attn_union"],
        "route_bytes": by["route"],
        "step_bytes_how": "attention: K/V rows of the union of chunks over each KV group's heads, "
                          "plus q, o and chunk lists; routing: each query head's frontier summary "
                          "rows (heads of a group share many of them, so this overcounts HBM)",
        "step_bytes_per_head_sum": by["attn_per_head"] + by["route"],
        "step_hbm_frac": step_union / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "query_heads_per_s": value * g.H_q,
        "stream_copy_GBs": r["copy_gbs"],
        "attn_frac_of_copy": achieved_attn / r["copy_gbs"],
        "cold": {"route_attn_us": float(r["cold_fused_ms"].mean() * 1e3),
                 "route_us": float(r["cold_route_ms"].mean() * 1e3),
                 "attn_us": float(r["cold_attn_ms"].mean() * 1e3),
                 "us_per_step": float((r["cold_route_ms"] + r["cold_attn_ms"]).mean() * 1e3),
                 "queries_per_s": g.B / float((r["cold_route_ms"] + r["cold_attn_ms"]).mean()
                                              * 1e-3),
                 "step_hbm_frac": step_union / float((r["cold_route_ms"] + r["cold_attn_ms"]).mean()
                                                     * 1e-3) / (HBM_PEAK_GBS * 1e9),
                 "steps": int(len(r["cold_route_ms"])),
                 "how": "1 GiB written before each route and each attention call, outside its "
                        "timing; each call between two events of its own"},
        "tokens_per_head": by["tokens_per_head"],
        "keys_attended_frac": by["tokens_per_head"] / g.T,
        "build_ms": r["build_ms"],
        "decode_maintenance": dict(r["maintenance"], frac_of_step=r["maintenance"][
            "amortized_us_per_token"] / (ms_per_step * 1e3)),
        "dense_ms_per_step": r["dense_ms"],
        "speedup_vs_dense": (r["dense_ms"] / ms_per_step) if r["dense_ms"] else None,
        "at_1m": run_block_1m() if args.with_1m else None,
        "other_decode": ({W.CONFIGS[c].name: run_decode_leg(c) for c in (1, 2, 5)}
                         if args.with_configs and args.config == 3 and args.refs == 0 else None),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
