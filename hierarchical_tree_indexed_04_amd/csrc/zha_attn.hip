// Exact attention over the routed token set, and the dense decode baseline.
//
// Sparse path (summary page of the paper, "Routing": I(q) = {0} U selected
// leaf chunks U C_cur, o(q) = Attn(q, K_I, V_I)).  Balanced split-KV: the
// attended tokens of all query heads of the call, laid end to end, are cut
// into equal ranges, one per workgroup (every workgroup computes the same
// prefix of per-head token counts in LDS).  A workgroup streams the K and V
// rows of its range (one 16-byte slice per lane, LPR lanes per row, 8 rows in
// flight per lane, q . k with packed bf16 dot products), keeps an online
// softmax per row group and combines the row groups in LDS in a fixed order.
// A head whose tokens fall in one range is written directly; otherwise each
// range writes a partial (a d-vector plus max and sum, paper App. D-B) to slot
// (workgroup + head), which is unique, and a second launch merges the
// partials of each head in range order, so results are bit-reproducible.
// (Merging inside the first launch would need a device-scope release/acquire
// per workgroup, which on a multi-XCD part means an L2 write-back and
// invalidate each time: far slower than the extra launch.)
//
// With more query heads than a workgroup can prefix-sum in LDS, each head is
// one workgroup (no split).
//
// Dense path (paper App. D-A decode model): the same structure over all T
// keys; a workgroup serves the G query heads of one KV head so each K/V row
// is read once per group.

#include "zha_attn_impl.hpp"

namespace zha {
namespace {
// Split-KV merge as its own launch: one workgroup per query head (or per
// dense head tile); the kernel boundary makes the partials visible without
// device-wide fences.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ part,
                                                         const int32_t* __restrict__ cnt,
                                                         int32_t cap, T* __restrict__ O, int S) {
  const int64_t head = blockIdx.x;
  if (cnt != nullptr) {
    const int c = cnt[head];
    if (c < 0 || c > cap) return;  // NaN row already written by the partial kernel
  }
  merge_partials<T, D>(part + head * (int64_t)S * (D + 2), S, O + head * D);
}

// Attention of one query head (split `split` of a.S) by one workgroup.
template <typename T, int D, bool POW2, bool BUF>
__device__ __forceinline__ void attend_one_head(const T* __restrict__ Q, const T* __restrict__ K,
                                                const T* __restrict__ V,
                                                const int32_t* __restrict__ sel,
                                                const int32_t* __restrict__ cnt,
                                                T* __restrict__ O, float* __restrict__ part,
                                                const AttnArgs& a, int64_t head, int split) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = kThreads / LPR;
  __shared__ float s_m[RPB], s_l[RPB];
  __shared__ float s_acc[RPB * D];
  __shared__ int32_t s_ids[kIds];
  const int tid = threadIdx.x;
  const int sub = tid % LPR, grp = tid / LPR;
  const int64_t Th = visible_len(a, head);  // tokens this head may see
  const int c = Th < 0 ? -1 : cnt[head];
  if (c < 0 || c > a.cap) {  // overflowed or failed route: the row is NaN
    if (split == 0)
      for (int t = tid; t < D; t += kThreads) store_elem(O + head * D, t, __int_as_float(0x7fc00000));
    return;
  }
  const int h = (int)(head % a.H_q);
  const int64_t b = head / ((int64_t)a.n_pos * a.H_q);
  const int64_t tr = b * a.H_kv + h / a.G;
  const int32_t* ids = sel + head * a.cap;
  const KvBlock<T, D, BUF> kvb(K, V, tr, a.Tc, a.C, a.chunked, sub);

  // This split's chunks, plus (last split) the sink when chunk 0 is not selected
  // and C_cur.  Token positions and ids fit in 31 bits (T < 2^31).
  const int Cc = a.C, log2C = a.log2C;
  const int c0 = (int)(((int64_t)split * c) / a.S);
  const int c1 = (int)(((int64_t)(split + 1) * c) / a.S);
  const int ct = (c1 - c0) * Cc;  // chunk tokens come first, then the extras
  int n_extra = 0;
  bool sink = false;
  const int n1 = (int)(Th / Cc);  // full chunks within the visible tokens
  if (split == a.S - 1) {
    sink = n1 > 0 && ((c == 0) || (ids[0] != 0));  // with no full chunk, C_cur holds token 0
    n_extra = (sink ? 1 : 0) + (int)(Th - (int64_t)n1 * Cc);
  }
  const int ntok = ct + n_extra;

  const uint4 qv = ld16c(Q + head * D + sub * VEC);
  const float inv = 1.0f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  // Chunk ids are staged in LDS, kIds at a time, so the address of every K/V
  // row comes from LDS and all loads of an iteration issue back to back (a
  // global id load between them would wait, in order, for every earlier row).
  const int nc = c1 - c0;
  for (int r0 = 0;; r0 += kIds) {
    const int rn = min(kIds, nc - r0);
    const bool final_round = r0 + kIds >= nc;
    if (rn > 0) {
      __syncthreads();
      for (int i = tid; i < rn; i += kThreads) s_ids[i] = ids[c0 + r0 + i];
      __syncthreads();
    }
    const int xb = r0 * Cc;
    const int xe = final_round ? ntok : (r0 + rn) * Cc;
    for (int base = xb; base < xe; base += RPB * kUA) {
      int row[kUA];
#pragma unroll
      for (int u = 0; u < kUA; ++u) {
        const int x = base + u * RPB + grp;
        const int ci = POW2 ? (x >> log2C) : x / Cc;
        row[u] = s_ids[min(max(ci - r0, 0), kIds - 1)];
      }
#pragma unroll
      for (int u = 0; u < kUA; ++u) {
        const int x = base + u * RPB + grp;
        const int ci = POW2 ? (x >> log2C) : x / Cc;
        const int e = x - ct;
        const bool is_sink = sink && e == 0;
        const int chunk = x < ct ? row[u] : (is_sink ? 0 : n1);
        const int j = x < ct ? x - ci * Cc : (is_sink ? 0 : e - (sink ? 1 : 0));
        row[u] = kvb.key_row(chunk, j);
      }
      uint4 kv[kUA], vv[kUA];
#pragma unroll
      for (int u = 0; u < kUA; ++u) kvb.load(row[u], base + u * RPB + grp < xe, kv[u], vv[u]);
      __builtin_amdgcn_sched_barrier(0);
      float s[kUA];
#pragma unroll
      for (int u = 0; u < kUA; ++u) {
        const float dot = group_allreduce<LPR>(slice_dot<T>(kv[u], qv), OpAdd()) * inv;
        s[u] = (base + u * RPB + grp < xe) ? dot : -INFINITY;
      }
      online_update<T, kUA>(m, l, acc, s, vv);
    }
    if (final_round) break;
  }
  float* prow = (a.S > 1) ? part + (head * a.S + split) * (int64_t)(D + 2) : nullptr;
  combine_groups<T, D, RPB>(m, l, acc, grp, sub, s_m, s_l, s_acc, O + head * D, prow);
}

template <typename T, int D, bool POW2, bool BUF>
__global__ __launch_bounds__(kThreads) void attn_partial_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, T* __restrict__ O,
    float* __restrict__ part, AttnArgs a) {
  attend_one_head<T, D, POW2, BUF>(Q, K, V, sel, cnt, O, part, a, (int64_t)blockIdx.x,
                                   (int)blockIdx.y);
}

// Balanced split-KV over all heads of the call: workgroup w owns tokens
// [w W, (w + 1) W) of the concatenated per-head token lists.  POW2: C is a
// power of two (chunk index by shift).
// The launch keeps ZHA_ATTN_WAVES waves per SIMD resident (ZHA_ATTN_BLOCKS
// workgroups of 4 waves); telling the compiler so lets it keep every row load
// of an iteration in flight instead of trimming registers for occupancy that
// the launch cannot use.
template <typename T, int D, bool POW2, bool BUF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ZHA_ATTN_WAVES, ZHA_ATTN_WAVES))) void attn_balanced_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, T* __restrict__ O,
    float* __restrict__ part, int64_t* __restrict__ plan, AttnArgs a) {
  constexpr int kE = kBalMaxHeads / kThreads;
  __shared__ int64_t s_pre[kBalMaxHeads + 1];
  __shared__ SegSmem<T, D> sm;
  __shared__ uint64_t s_wtot[kWaves];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nh = (int)a.n_heads;
  const int E = (nh + kThreads - 1) / kThreads;

  // 1. Prefix of per-head token counts (thread tid owns heads [tid E, tid E + E)),
  // 64-bit: a head attends up to T < 2^31 tokens, so the call's total can
  // pass 2^31 (the plan arithmetic lives in zha_plan.hpp).
  int cv[kE], fv[kE];
  int64_t lv[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    const int h = tid * E + e;
    cv[e] = -1;
    fv[e] = 0;
    lv[e] = -1;
    if (e < E && h < nh) {
      cv[e] = cnt[h];
      fv[e] = sel[(int64_t)h * a.cap];  // read even when unused: the buffer has it
      lv[e] = visible_len(a, h);
    }
  }
  int64_t tv[kE];
  uint64_t run = 0;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    tv[e] = (e < E && tid * E + e < nh) ? bal_head_tokens(cv[e], fv[e], lv[e], a.C, a.cap) : 0;
    run += (uint64_t)tv[e];
  }
  const uint64_t incl = wave_incl_scan_u64(run);
  if (lane == kWave - 1) s_wtot[wave] = incl;
  __syncthreads();
  uint64_t excl = incl - run;
  uint64_t total_u = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) excl += s_wtot[w];
    total_u += s_wtot[w];
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    const int h = tid * E + e;
    if (e < E && h < nh) {
      s_pre[h] = (int64_t)excl;
      excl += (uint64_t)tv[e];
    }
  }
  const int64_t total = (int64_t)total_u;
  if (tid == 0) s_pre[nh] = total;
  __syncthreads();
  const int64_t Wtok = bal_width(total, gridDim.x);
  if (blockIdx.x == 0) {
    for (int h = tid; h <= nh; h += kThreads) plan[h] = s_pre[h];
    if (tid == 0) plan[nh + 1] = Wtok;
  }
  // Range index, XCD-major: consecutive ranges (the heads of one KV group,
  // which share many chunks) run on one XCD and meet in its L2 (256K call
  // 49.1 -> 48.7 us).  The merge finds a head's partials by range index.
  const int64_t rng = xcd_major_index(blockIdx.x, gridDim.x);
  const int64_t lo = rng * Wtok;
  const int64_t hi = min(lo + Wtok, total);
  if (lo >= hi) return;

  // 2. First head of the range.
  const int h0 = bal_first_head(s_pre, nh, lo);

  // 3. One segment per head overlapping the range.  Token positions and ids
  // fit in 31 bits (T < 2^31), so the index math is 32-bit; only the final
  // row address is 64-bit.
  for (int h = h0; h < nh && s_pre[h] < hi; ++h) {
    const int64_t P0 = s_pre[h], P1 = s_pre[h + 1];
    if (P1 <= lo || P1 == P0) continue;  // before the range, or a failed route (no tokens)
    const BalSegment seg = bal_segment(P0, P1, lo, hi);
    const bool whole = seg.x0 == 0 && (int64_t)seg.x1 == P1 - P0;
    attend_segment<T, D, POW2, BUF>(Q, K, V, sel + (int64_t)h * a.cap, cnt[h], visible_len(a, h),
                                    a, h, seg.x0, seg.x1, O + (int64_t)h * D,
                                    whole ? nullptr : part + bal_slot(rng, h) * (D + 2), sm);
  }
}

// Merge for the balanced split: head h's ranges are workgroups
// [P_h / W, (P_{h+1} - 1) / W]; their partials sit at slots (workgroup + h).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_balanced_kernel(
    const float* __restrict__ part, const int64_t* __restrict__ plan,
    const int32_t* __restrict__ cnt, AttnArgs a, T* __restrict__ O) {
  const int h = blockIdx.x;
  const int cap = a.cap, nh = (int)a.n_heads;
  // Independent loads, issued together.
  const int c = cnt[h];
  const int64_t Th = visible_len(a, h);
  const int64_t P0 = plan[h], P1 = plan[h + 1], W = plan[nh + 1];
  if (c < 0 || c > cap || Th < 0) {  // failed or overflowed route: NaN row
    for (int t = threadIdx.x; t < D; t += kThreads)
      store_elem(O + (int64_t)h * D, t, __int_as_float(0x7fc00000));
    return;
  }
  const BalSpan sp = bal_head_span(P0, P1, W);
  if (sp.first == sp.last) return;  // written whole by its workgroup
  merge_partials<T, D>(part + bal_slot(sp.first, h) * (D + 2), (int)(sp.last - sp.first + 1),
                       O + (int64_t)h * D);
}

// Dense decode: one workgroup per (b, t, kvh, head tile of GT) and split; GT
// query heads share every K/V row.
template <typename T, int D, int GT>
__global__ __launch_bounds__(kThreads) void dense_partial_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    T* __restrict__ O, float* __restrict__ part, DenseArgs a) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = kThreads / LPR;
  __shared__ float s_m[RPB], s_l[RPB];
  __shared__ float s_acc[RPB * D];
  const int tid = threadIdx.x;
  const int sub = tid % LPR, grp = tid / LPR;
  const int tiles = a.G / GT;
  const int64_t blk = blockIdx.x;
  const int tile = (int)(blk % tiles);
  const int64_t bk = blk / tiles;  // (b * n_pos + t) * H_kv + kvh
  const int kvh = (int)(bk % a.H_kv);
  const int64_t bt = bk / a.H_kv;
  const int64_t b = bt / a.n_pos;
  const int split = blockIdx.y;
  const int64_t head0 = bt * a.H_q + (int64_t)kvh * a.G + tile * GT;
  // Key row of token t: t (split) or t + (t / C) C (chunked pages of C key
  // rows then C value rows, the value row C rows further).
  const int64_t nblk = kv_block_elems(a.Tc, a.C, D, a.chunked);
  const T* Kt = K + (b * a.H_kv + kvh) * nblk;
  const T* Vt = a.chunked ? Kt + (int64_t)a.C * D : V + (b * a.H_kv + kvh) * nblk;
  const int64_t t0 = (a.T * split) / a.S, t1 = (a.T * (split + 1)) / a.S;

  uint4 qv[GT];
  const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int g = 0; g < GT; ++g) qv[g] = ld16c(Q + (head0 + g) * D + sub * VEC);
  float m[GT], l[GT], acc[GT][VEC];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[g][e] = 0.f;
  }
  for (int64_t base = t0; base < t1; base += (int64_t)RPB * kUD) {
    uint4 kv[kUD], vv[kUD];
    bool ok[kUD];
#pragma unroll
    for (int u = 0; u < kUD; ++u) {
      const int64_t tok = base + u * RPB + grp;
      ok[u] = tok < t1;
      if (ok[u]) {
        const int64_t ci = a.log2C >= 0 ? (tok >> a.log2C) : tok / a.C;
        const int64_t row = a.chunked ? tok + ci * a.C : tok;
        kv[u] = ld16(Kt + row * D + sub * VEC);
        vv[u] = ld16(Vt + row * D + sub * VEC);
      } else {
        kv[u] = make_uint4(0u, 0u, 0u, 0u);
        vv[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float s[kUD];
#pragma unroll
      for (int u = 0; u < kUD; ++u) {
        const float dot = group_allreduce<LPR>(slice_dot<T>(kv[u], qv[g]), OpAdd()) * inv;
        s[u] = ok[u] ? dot : -INFINITY;
      }
      online_update<T, kUD>(m[g], l[g], acc[g], s, vv);
    }
  }
  for (int g = 0; g < GT; ++g) {
    float* prow = (a.S > 1) ? part + ((head0 + g) * a.S + split) * (int64_t)(D + 2) : nullptr;
    combine_groups<T, D, RPB>(m[g], l[g], acc[g], grp, sub, s_m, s_l, s_acc, O + (head0 + g) * D,
                              prow);
    __syncthreads();
  }
}

// ===========================================================================
// Block path: many query heads against the same caches (a block of positions
// of one sequence).  Each chunk is selected by many heads there, so the work
// is turned around: (query head, tile) pairs are bucketed per tile of CT
// chunks, and a work item stages the selected chunks of one tile once for up
// to kBlkQ heads and runs both products on MFMA (a query block against a leaf
// tile is a dense contraction; unselected (head, chunk) cells are masked).
// Each pair leaves a softmax partial; a merge launch combines the partials of
// each head in tile order, so results do not depend on scheduling.
// ===========================================================================
// Query heads per work item: 4 waves x NB blocks of 16 MFMA rows.  Each item
// stages the selected chunks of its tile once, so a tile whose entries span
// several items is staged several times; two blocks per wave halve the items
// of a tile that holds more than 64 entries, and the K and V^T operands a wave
// reads from LDS serve both of its blocks, but the registers of the second
// block cost a wave per SIMD (3 -> 2).  Measured: causal prefill of 128K in
// calls of 4096 positions (~256 heads per tile) attention 19.05 -> 17.83 ms
// with two blocks; the 1M block (~16 heads per tile, 1,727 of 2,048 tiles in
// one item of 64) 0.331 -> 0.343 ms.  A call takes two blocks when its heads
// are at least kBlkNB2Heads per tile.
constexpr int kBlkGroup = 32;  // tokens per MFMA step
constexpr int kBlkNB2Heads = 64;
template <int NB>
struct BlkShape {
  static constexpr int kQ = 64 * NB;                // query heads per work item
  static constexpr int kWavesEU = NB > 1 ? 2 : 3;   // waves per SIMD the registers are held to
  static constexpr int kGrid = 256 * kWavesEU;      // persistent workgroups (one per wave slot)
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct BlkPtrs {
  int32_t* ctrl;   // [0] work items
  int32_t* qbase;  // per head: first slot
  int32_t* ntile;  // per head: tiles (>= 0), -1 attended per head, -2 failed route
  int64_t* wsum;   // per workgroup of the count launch (4 heads): slots wanted
  int32_t* tcnt;   // per tile: pairs
  int32_t* tcur;   // per tile: fill cursor
  int32_t* toff;   // per tile: first entry (exclusive scan of tcnt)
  int32_t* wpre;   // per tile: first work item
  int32_t* wbase;  // per (workgroup of the per-tile launches, tile): first entry in the tile
  int32_t* ent;    // entries, kBlkEntryInts ints each
  float* part;     // partials, d + 2 floats per slot
  __device__ __host__ BlkPtrs(char* scr, const BlkLayout& L)
      : ctrl(reinterpret_cast<int32_t*>(scr + L.off_ctrl)),
        qbase(reinterpret_cast<int32_t*>(scr + L.off_qbase)),
        ntile(reinterpret_cast<int32_t*>(scr + L.off_ntile)),
        wsum(reinterpret_cast<int64_t*>(scr + L.off_wsum)),
        tcnt(reinterpret_cast<int32_t*>(scr + L.off_tcnt)),
        tcur(reinterpret_cast<int32_t*>(scr + L.off_tcur)),
        toff(reinterpret_cast<int32_t*>(scr + L.off_toff)),
        wpre(reinterpret_cast<int32_t*>(scr + L.off_wpre)),
        wbase(reinterpret_cast<int32_t*>(scr + L.off_wbase)),
        ent(reinterpret_cast<int32_t*>(scr + L.off_ent)),
        part(reinterpret_cast<float*>(scr + L.off_part)) {}
};

__device__ __forceinline__ int64_t tree_of_head(int64_t head, const AttnArgs& a) {
  const int h = (int)(head % a.H_q);
  const int64_t b = head / ((int64_t)a.n_pos * a.H_q);
  return b * a.H_kv + h / a.G;
}

// The merge launch gives each query head a group of kGL lanes (four heads per
// wave): its work per head is short, and one wave per head took several
// rounds of resident waves.
constexpr int kGL = 16;
constexpr int kHPW = kWave / kGL;  // heads per wave

// The bookkeeping launches give each query head one lane.  A head of at most
// kWave chunk ids is walked by its lane with every id load issued at once (the
// loads are independent, so the lane waits once): each run of ids in one tile
// is handed to f(tile, mask of its chunks within the tile, run index).
// Returns the number of runs (tiles).  CT = 2^lct chunks per tile.
template <typename F>
__device__ __forceinline__ int short_runs(const int32_t* __restrict__ ids, int c, int lct, F f) {
  int v[kWave];
#pragma unroll
  for (int u = 0; u < kWave; ++u) v[u] = u < c ? ids[u] : -1;
  int n = 0, cur = -1;
  uint64_t mask = 0;
#pragma unroll
  for (int u = 0; u < kWave; ++u) {
    if (v[u] < 0) continue;
    const int t = v[u] >> lct;
    if (t != cur) {
      if (cur >= 0) {
        f(cur, mask, n);
        ++n;
      }
      cur = t;
      mask = 0;
    }
    mask |= 1ull << (v[u] - (t << lct));
  }
  if (cur >= 0) {
    f(cur, mask, n);
    ++n;
  }
  return n;
}

// The same walk by a whole wave for one head (c and ids uniform), for heads of
// more than kWave ids: lane i takes id j + i of each batch of 64; the lanes
// that start a tile's run are found by ballot, each lane ORs its chunk's bit
// into its run's mask in LDS (rm: kWave + 1 words of this wave; the last
// slot carries a run into the next batch), and the run's first lane calls
// emit(tile, mask, run index).  Returns the number of runs.
template <typename F>
__device__ __forceinline__ int wave_runs(const int32_t* __restrict__ ids, int c, int lct,
                                         unsigned long long* rm, F emit) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  if (lane == 0) rm[kWave] = 0ull;
  int k = 0, cur = -1;  // runs emitted; tile carried from the previous batch
  int pre[4];           // ids of the next four batches, loaded together
  for (int j = 0; j < c; j += kWave) {
    const int q = (j / kWave) & 3;
    if (q == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) pre[u] = j + u * kWave + lane < c ? ids[j + u * kWave + lane] : 0;
    }
    const bool valid = j + lane < c;
    const int id = q == 0 ? pre[0] : q == 1 ? pre[1] : q == 2 ? pre[2] : pre[3];
    const int t = valid ? id >> lct : -1;
    int tp = __shfl_up(t, 1, kWave);
    if (lane == 0) tp = cur;
    const bool first = valid && t != tp;
    const uint64_t fb = __ballot(first);
    // Run of this lane: starts at or below it, minus one (-1: the carried run).
    const int r = __popcll((unsigned long long)(fb & (lt | (1ull << lane)))) - 1;
    rm[lane] = 0ull;
    asm volatile("" ::: "memory");
    if (valid) atomicOr(&rm[r < 0 ? kWave : r], 1ull << (id - (t << lct)));
    asm volatile("" ::: "memory");
    if (fb != 0ull) {
      if (cur >= 0) {
        if (lane == 0) emit(cur, (uint64_t)rm[kWave], k);
        ++k;
      }
      const int last = 63 - __clzll((long long)fb);
      const int nrun = __popcll((unsigned long long)fb);
      if (first && lane != last) emit(t, (uint64_t)rm[r], k + r);
      k += nrun - 1;
      cur = __builtin_amdgcn_readlane(t, last);
      asm volatile("" ::: "memory");
      const unsigned long long lm = rm[nrun - 1];
      asm volatile("" ::: "memory");
      if (lane == 0) rm[kWave] = lm;
    }
  }
  if (cur >= 0) {
    if (lane == 0) emit(cur, (uint64_t)rm[kWave], k);
    ++k;
  }
  return k;
}

// Runs of every lane's head: heads of at most kWave ids by their own lane,
// longer ones by the whole wave, one after another.  Per lane: its head, the
// head's id count c (c < 0: no head) and one more value aux of the head;
// emit(head, aux, tile, mask, run index) is called in the head's own lane for
// the short heads and in a lane of the wave for the long ones.  All lanes of
// the wave must call it together.  Returns the lane's head's run count.
template <typename F>
__device__ __forceinline__ int head_runs(const int32_t* __restrict__ sel, int64_t head, int c,
                                         int aux, int cap, int lct, unsigned long long* rm,
                                         F emit) {
  const int lane = threadIdx.x & (kWave - 1);
  int n = 0;
  if (c > 0 && c <= kWave)
    n = short_runs(sel + head * cap, c, lct,
                   [&](int t, uint64_t m, int k) { emit(head, aux, t, m, k); });
  uint64_t longs = __ballot(c > kWave);
  while (longs != 0ull) {
    const int src = __ffsll((unsigned long long)longs) - 1;
    longs &= longs - 1;
    const int64_t hh = ((int64_t)__builtin_amdgcn_readlane((int)(head >> 32), src) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)head, src);
    const int hc = __builtin_amdgcn_readlane(c, src);
    const int ha = __builtin_amdgcn_readlane(aux, src);
    const int nn = wave_runs(sel + hh * cap, hc, lct, rm,
                             [&](int t, uint64_t m, int k) { emit(hh, ha, t, m, k); });
    if (lane == src) n = nn;
  }
  return n;
}

constexpr int kLaneHeads = 128;     // query heads per workgroup of the lane-per-head launches
constexpr int kHeadsPerWave = 8;    // of them per wave: lanes 0..7 (a wave walks long heads alone)
constexpr int kLaneWaves = kLaneHeads / kHeadsPerWave;
constexpr int kLaneThreads = kLaneWaves * kWave;
constexpr int kBlkLdsTiles = 4096;  // tiles of one cache that an LDS histogram covers

// Item i of cache tr, the caches' heads taken (position, query head of the
// group) in order: the launches that count and fill per tile give each
// workgroup heads of one cache, so its tiles aggregate in LDS.
__device__ __forceinline__ int64_t tree_item_head(int64_t tr, int64_t i, const AttnArgs& a) {
  const int64_t b = tr / a.H_kv;
  const int kvh = (int)(tr - b * a.H_kv);
  const int64_t pos = i / a.G;
  const int g = (int)(i - pos * a.G);
  return (b * a.n_pos + pos) * a.H_q + (int64_t)kvh * a.G + g;
}

// A head's pairs are the tiles of its selected chunks, ascending (its sink and
// partial-chunk tokens are the merge launch's).  One lane per head, heads in
// order: the head's tile count, and the slots each workgroup's heads want
// (tiles + 1 each) for the prefix sum.  Also clears the tile counters and
// cursors and the control words for the launches that follow.
__global__ __launch_bounds__(kLaneThreads) void blk_count_kernel(const int32_t* __restrict__ sel,
                                                                 const int32_t* __restrict__ cnt,
                                                                 AttnArgs a, BlkLayout L,
                                                                 char* scr) {
  __shared__ uint64_t s_w[kLaneWaves];
  __shared__ unsigned long long s_run[kLaneWaves][kWave + 1];
  BlkPtrs P(scr, L);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  for (int64_t i = (int64_t)blockIdx.x * kLaneThreads + tid; i < L.NTT;
       i += (int64_t)gridDim.x * kLaneThreads) {
    P.tcnt[i] = 0;
    P.tcur[i] = 0;
  }
  if (blockIdx.x == 0 && tid < 16) P.ctrl[tid] = 0;
  const int64_t head = (int64_t)blockIdx.x * kLaneHeads + wave * kHeadsPerWave + lane;
  const bool hv = lane < kHeadsPerWave && head < a.n_heads;
  int c = -1;
  if (hv) {
    c = visible_len(a, head) < 0 ? -1 : cnt[head];
    if (c > a.cap) c = -1;
  }
  int n = head_runs(sel, hv ? head : 0, c, 0, a.cap, L.lct, s_run[wave],
                    [](int64_t, int, int, uint64_t, int) {});
  if (c < 0) n = -2;
  if (hv) P.ntile[head] = n;
  const uint64_t w = wave_sum_u64_bcast(hv && n >= 0 ? (uint64_t)(n + 1) : 0ull);
  if (lane == 0) s_w[wave] = w;
  __syncthreads();
  if (tid == 0) {
    uint64_t t = 0;
#pragma unroll
    for (int x = 0; x < kLaneWaves; ++x) t += s_w[x];
    P.wsum[blockIdx.x] = (int64_t)t;
  }
}

// Slot bases, one launch of workgroups of 8192 heads: the slots of the heads
// before its range come from the count launch's per-workgroup sums; its own
// range goes through LDS in coalesced loads, each thread then sums 8
// consecutive heads, one block scan.  From the first head whose slots would
// pass the budget on, heads are marked for per-head attention (ntile = -1):
// they take no slots and no pairs.
constexpr int kScanPer = 8;
constexpr int kScanChunk = 1024 * kScanPer;  // heads per workgroup of the scan launch
__global__ __launch_bounds__(1024) void blk_scan_kernel(int64_t n_heads, BlkLayout L, char* scr) {
  BlkPtrs P(scr, L);
  __shared__ int64_t s_w[1024 / kWave];
  __shared__ int32_t s_c[kScanChunk];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kScanChunk;
  // This range's values, loaded first (coalesced, unconditional).
  int v[kScanPer];
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) v[k] = P.ntile[min(c0 + (int64_t)k * 1024 + tid, n_heads - 1)];
  // Slots of the heads before the range: the count launch's sums of kLaneHeads heads.
  const int64_t nw = c0 / kLaneHeads;
  int64_t before = 0;
  for (int64_t i0 = 0; i0 < nw; i0 += 8 * 1024) {  // 8 loads in flight per thread
    int64_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = P.wsum[min(i0 + u * 1024 + tid, nw - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) before += i0 + u * 1024 + tid < nw ? x[u] : 0;
  }
  before = (int64_t)wave_sum_u64_bcast((uint64_t)before);
  if (lane == 0) s_w[wave] = before;
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) s_c[k * 1024 + tid] = v[k];
  __syncthreads();
  int64_t run = 0;
#pragma unroll
  for (int x = 0; x < 1024 / kWave; ++x) run += s_w[x];
  int w[kScanPer];
  int64_t sum = 0;
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) {
    w[k] = c0 + tid * kScanPer + k < n_heads ? s_c[tid * kScanPer + k] : -3;
    sum += w[k] >= 0 ? w[k] + 1 : 0;
  }
  __syncthreads();  // s_w is reused
  const uint64_t incl = wave_incl_scan_u64((uint64_t)sum);
  if (lane == kWave - 1) s_w[wave] = (int64_t)incl;
  __syncthreads();
  int64_t off = 0;
#pragma unroll
  for (int x = 0; x < 1024 / kWave; ++x) off += x < wave ? s_w[x] : 0;
  int64_t start = run + off + (int64_t)incl - sum;
#pragma unroll
  for (int k = 0; k < kScanPer; ++k) {
    if (w[k] < 0) continue;
    const int64_t i = c0 + tid * kScanPer + k;
    if (start + w[k] + 1 > L.S) P.ntile[i] = -1;
    else P.qbase[i] = (int32_t)start;
    start += w[k] + 1;
  }
}

// Pairs per tile, over the heads that have slots.  Eight heads per wave, the
// workgroup's heads all of one cache: its pairs per tile are counted in LDS,
// then one global add per tile touched, whose old value is the workgroup's
// first place in the tile's entries (kept for the fill launch); caches of more
// than kBlkLdsTiles tiles add per pair.
__global__ __launch_bounds__(kLaneThreads) void blk_tcount_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, AttnArgs a, BlkLayout L,
    char* scr) {
  __shared__ int32_t s_h[kBlkLdsTiles];
  __shared__ unsigned long long s_run[kLaneWaves][kWave + 1];
  BlkPtrs P(scr, L);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int64_t per_tree = (int64_t)a.n_pos * a.G;
  const int64_t wpt = (per_tree + kLaneHeads - 1) / kLaneHeads;
  const int64_t tr = blockIdx.x / wpt;
  const int64_t i = (blockIdx.x - tr * wpt) * kLaneHeads + wave * kHeadsPerWave + lane;
  const bool hv = lane < kHeadsPerWave && i < per_tree;
  const bool lds = L.NT <= kBlkLdsTiles;
  int32_t* tc = P.tcnt + tr * L.NT;
  if (lds) {
    for (int t = tid; t < L.NT; t += kLaneThreads) s_h[t] = 0;
    __syncthreads();
  }
  const int64_t head = hv ? tree_item_head(tr, i, a) : 0;
  const int c = (hv && P.ntile[head] >= 0) ? cnt[head] : -1;
  head_runs(sel, head, c, 0, a.cap, L.lct, s_run[wave],
            [&](int64_t, int, int t, uint64_t, int) {
              if (lds) atomicAdd(&s_h[t], 1);
              else atomicAdd(&tc[t], 1);
            });
  if (lds) {
    __syncthreads();
    int32_t* wb = P.wbase + (int64_t)blockIdx.x * L.NT;
    for (int t = tid; t < L.NT; t += kLaneThreads)
      if (s_h[t] != 0) wb[t] = atomicAdd(&tc[t], s_h[t]);
  }
}

// Exclusive scans over the tiles: first entry and first work item of each
// (one workgroup), and the number of work items.
__global__ __launch_bounds__(1024) void blk_tscan_kernel(BlkLayout L, char* scr, int q) {
  BlkPtrs P(scr, L);
  __shared__ int64_t s_v[1024], s_w[1024];
  const int tid = threadIdx.x;
  const int64_t seg = (L.NTT + 1023) / 1024;
  const int64_t i0 = min(L.NTT, tid * seg), i1 = min(L.NTT, i0 + seg);
  int64_t sc = 0, sw = 0;
  for (int64_t i = i0; i < i1; ++i) {
    sc += P.tcnt[i];
    sw += (P.tcnt[i] + q - 1) / q;
  }
  s_v[tid] = sc;
  s_w[tid] = sw;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the 1024 run sums
    const int64_t vc = tid >= off ? s_v[tid - off] : 0;
    const int64_t vw = tid >= off ? s_w[tid - off] : 0;
    __syncthreads();
    s_v[tid] += vc;
    s_w[tid] += vw;
    __syncthreads();
  }
  int64_t rc = s_v[tid] - sc, rw = s_w[tid] - sw;
  for (int64_t i = i0; i < i1; ++i) {
    P.toff[i] = (int32_t)rc;
    P.wpre[i] = (int32_t)rw;
    rc += P.tcnt[i];
    rw += (P.tcnt[i] + q - 1) / q;
  }
  if (tid == 1023) {
    P.toff[L.NTT] = (int32_t)s_v[1023];
    P.wpre[L.NTT] = (int32_t)s_w[1023];
    P.ctrl[0] = (int32_t)s_w[1023];
  }
}

// One entry per (head with slots, tile): head, slot, 64-bit mask of the
// head's chunks in the tile.  The same heads per workgroup as the tile count
// launch: each pair takes the next place of the workgroup's range of its tile
// (first place from the tile count launch) from an LDS counter.  Caches of
// more than kBlkLdsTiles tiles take places one by one from a global cursor.
__global__ __launch_bounds__(kLaneThreads) void blk_fill_kernel(const int32_t* __restrict__ sel,
                                                                const int32_t* __restrict__ cnt,
                                                                AttnArgs a, BlkLayout L,
                                                                char* scr) {
  __shared__ int32_t s_h[kBlkLdsTiles];  // places taken per tile
  __shared__ int32_t s_b[kBlkLdsTiles];  // first place of the workgroup's range
  __shared__ unsigned long long s_run[kLaneWaves][kWave + 1];
  BlkPtrs P(scr, L);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int64_t per_tree = (int64_t)a.n_pos * a.G;
  const int64_t wpt = (per_tree + kLaneHeads - 1) / kLaneHeads;
  const int64_t tr = blockIdx.x / wpt;
  const int64_t i = (blockIdx.x - tr * wpt) * kLaneHeads + wave * kHeadsPerWave + lane;
  const bool hv = lane < kHeadsPerWave && i < per_tree;
  const bool lds = L.NT <= kBlkLdsTiles;
  const int64_t tb = tr * L.NT;
  const int64_t head = hv ? tree_item_head(tr, i, a) : 0;
  const bool live = hv && P.ntile[head] >= 0;
  const int c = live ? cnt[head] : -1;
  const int qb = live ? P.qbase[head] : 0;
  if (lds) {
    // Places of tiles this workgroup does not touch are never read.
    const int32_t* wb = P.wbase + (int64_t)blockIdx.x * L.NT;
    for (int t = tid; t < L.NT; t += kLaneThreads) {
      s_h[t] = 0;
      s_b[t] = P.toff[tb + t] + wb[t];
    }
    __syncthreads();
  }
  head_runs(sel, head, c, qb, a.cap, L.lct, s_run[wave],
            [&](int64_t h, int q, int t, uint64_t mask, int k) {
              const int pos = lds ? s_b[t] + atomicAdd(&s_h[t], 1)
                                  : P.toff[tb + t] + atomicAdd(&P.tcur[tb + t], 1);
              int32_t* e = P.ent + (int64_t)pos * kBlkEntryInts;
              e[0] = (int32_t)h;
              e[1] = q + k;
              e[2] = (int32_t)(uint32_t)mask;
              e[3] = (int32_t)(uint32_t)(mask >> 32);
            });
}

// Work items: (tile, block of up to kQ of its entries), persistent loop.
// Per 32-token step of the tile (skipped when no head of the block selected
// any of its chunks): the K and V rows go to LDS as they are; each
// wave (16 heads) computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (so a
// lane holds one head's scores for 8 tokens), masks the cells its heads did
// not select, updates the online softmax and accumulates P V with the same
// MFMA, the 8 tokens of a lane taken as the K dimension in the order the
// scores already sit in registers.  Operand layouts (gfx950, checked):
// A[i][k] in lane i + 16 (k / 8), element k % 8; B[k][j] in lane j + 16 (k / 8),
// element k % 8; D[i][j] in lane j + 16 (i / 4), element i % 4.
// First work item of workgroup b: blocks of kBlkXcdQ consecutive items (the
// items of one tile are consecutive) go to one XCD, so a tile staged by
// several items can be found in that XCD's L2 after its first read; the
// blocks are dealt round-robin over the XCDs, which keeps the load spread.
#ifndef ZHA_BLK_XCD_Q
#define ZHA_BLK_XCD_Q 8  // 1M block attention call: 1 -> 337, 2 -> 334, 4..32 -> 328-331 us
#endif
constexpr int kBlkXcdQ = ZHA_BLK_XCD_Q;
template <int D, bool BUF, int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BlkShape<NB>::kWavesEU, BlkShape<NB>::kWavesEU))) void blk_attn_kernel(const bf16_t* __restrict__ Q,
                                                       const bf16_t* __restrict__ K,
                                                       const bf16_t* __restrict__ V, AttnArgs a,
                                                       BlkLayout L, char* scr) {
  constexpr int kBlkNB = NB;
  constexpr int kBlkQ = BlkShape<NB>::kQ;
  constexpr int KS = D / 32;   // k-steps of S^T = K Q^T
  constexpr int NTD = D / 16;  // 16-column tiles of O
  constexpr int SEG = D / 8;   // 16-byte segments per row
  constexpr int KROW = D + 8;  // padded LDS row of K (bf16 elements)
  // LDS row of V (bf16 elements), padded so that the 16 rows one transposed
  // read touches start 8 banks apart.
  constexpr int VROW = D + 16;
  BlkPtrs P(scr, L);
  __shared__ int32_t s_head[kBlkQ], s_slot[kBlkQ];
  __shared__ unsigned long long s_mask[kBlkQ];
  __shared__ unsigned long long s_union;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kBlkGroup * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kBlkGroup * VROW];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const float inv = 1.0f / sqrtf((float)D);
  const int C = a.C;
  const int total = P.ctrl[0];
  // Work items of one tile are consecutive and stage the same chunks.  When
  // tiles average more than two items (causal prefill: ~8), consecutive
  // workgroup indices are placed on one XCD so those re-reads meet in its L2
  // (prefill attention 21.9 -> 21.1 ms); with about one item per tile (the 1M
  // block) the default round-robin spreads the load better (350 against 370 us).
  const int vb = total > 2 * L.NTT ? (int)xcd_major_index(blockIdx.x, gridDim.x)
                                    : xcd_blocked_index((int)blockIdx.x, (int)gridDim.x, kBlkXcdQ);
  for (int w = vb; w < total; w += gridDim.x) {
    // Tile of work item w: the last tile u with wpre[u] <= w.
    int64_t lo = 0, hi = L.NTT;
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) >> 1;
      if (P.wpre[mid] <= w) lo = mid;
      else hi = mid;
    }
    const int64_t u = lo;
    const int e0 = P.toff[u] + (w - P.wpre[u]) * kBlkQ;
    const int ne = min(kBlkQ, P.toff[u + 1] - e0);
    __syncthreads();  // the previous item is done with LDS
    if (tid == 0) s_union = 0ull;
    if (tid < kBlkQ) {
      if (tid < ne) {
        const int32_t* e = P.ent + (int64_t)(e0 + tid) * kBlkEntryInts;
        s_head[tid] = e[0];
        s_slot[tid] = e[1];
        s_mask[tid] = (unsigned long long)(uint32_t)e[2] | ((unsigned long long)(uint32_t)e[3] << 32);
      } else {
        s_head[tid] = -1;
        s_slot[tid] = -1;
        s_mask[tid] = 0ull;
      }
    }
    __syncthreads();
    if (tid < ne) atomicOr(&s_union, s_mask[tid]);
    __syncthreads();
    const uint64_t uni = s_union;
    const int64_t tr = u / L.NT;
    const int chunk0 = (int)(u - tr * L.NT) * L.CT;
    const int tok0 = chunk0 * C;
    const int tok_end = (int)min((int64_t)(chunk0 + L.CT) * C, a.T);
    const KvBlock<bf16_t, D, BUF> kvb(K, V, tr, a.Tc, C, a.chunked, tid % SEG);

    // This lane's heads (row li of each of the wave's kBlkNB blocks of 16):
    // their Q slices as the B operands.
    int qi[kBlkNB];
    bool qvalid[kBlkNB];
    uint64_t qmask[kBlkNB];
    bf16x8_t qb[kBlkNB][KS];
    f32x4_t o[kBlkNB][NTD];
#pragma unroll
    for (int nb = 0; nb < kBlkNB; ++nb) {
      qi[nb] = (wave * kBlkNB + nb) * 16 + li;
      qvalid[nb] = qi[nb] < ne && s_head[qi[nb]] >= 0;  // empty entries have head -1, mask 0
      qmask[nb] = s_mask[qi[nb]];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (qvalid[nb]) v = ld16c(Q + (int64_t)s_head[qi[nb]] * D + ks * 32 + lg * 8);
        qb[nb][ks] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int n = 0; n < NTD; ++n) o[nb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // 32-token steps that some head of the block selected.
    // Staging thread (row pair rp, 16-byte segment sg) holds rows 2 rp, 2 rp + 1,
    // so V^T is written as 32-bit words of two tokens.  C is a power of two here.
    constexpr int NRP = kBlkGroup / 2;
    const int sg = tid % SEG, rp = tid / SEG;
    const bool stager = rp < NRP;
    const int lc = a.log2C;
    auto next_step = [&](int g) {
      for (; g < tok_end; g += kBlkGroup) {
        const int cf = (g >> lc) - chunk0, cl = ((min(g + kBlkGroup, tok_end) - 1) >> lc) - chunk0;
        const uint64_t bits = (cl >= 63 ? ~0ull : ((1ull << (cl + 1)) - 1)) & ~((1ull << cf) - 1);
        if ((uni & bits) != 0ull) break;
      }
      return g;
    };
    // Two register sets of staged rows: the next two steps are in flight while
    // one computes.  A set past the last step loads nothing (out-of-range
    // buffer offsets), so the loads are unconditional and every wait counts
    // exactly the loads issued after the ones it needs.
    uint4 ka[2], va[2], kb[2], vb[2];
    auto fetch = [&](uint4 (&pk)[2], uint4 (&pv)[2], int g) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int tok = g + 2 * rp + p;
        kvb.load(kvb.key_row(tok >> lc, tok & (C - 1)), stager && tok < tok_end, pk[p], pv[p]);
      }
    };
    // Stage: K and V rows as they are (token-major); the P V product reads V
    // with LDS transposed loads.
    auto stage = [&](const uint4 (&pk)[2], const uint4 (&pv)[2]) {
      if (stager) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          *reinterpret_cast<uint4*>(&s_k[(2 * rp + p) * KROW + sg * 8]) = pk[p];
          *reinterpret_cast<uint4*>(&s_v[(2 * rp + p) * VROW + sg * 8]) = pv[p];
        }
      }
    };
    const float c2 = 1.4426950408889634f * inv;  // log2(e) / sqrt(d)
    float m_i[kBlkNB], l_i[kBlkNB];  // m in raw score units; l summed per lane
#pragma unroll
    for (int nb = 0; nb < kBlkNB; ++nb) {
      m_i[nb] = -INFINITY;
      l_i[nb] = 0.f;
    }
    auto compute = [&](int g0) {
      // S^T = K Q^T for the two 16-token halves of the step; each K operand
      // read from LDS serves every block of the wave.
      f32x4_t st[kBlkNB][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int nb = 0; nb < kBlkNB; ++nb) st[nb][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 kv = *reinterpret_cast<const uint4*>(&s_k[(nt * 16 + li) * KROW + ks * 32 + lg * 8]);
#pragma unroll
          for (int nb = 0; nb < kBlkNB; ++nb)
            st[nb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                                qb[nb][ks], st[nb][nt], 0, 0, 0);
        }
      }
      // Lane (li, lg) holds head li's scores (of each block) for tokens
      // nt * 16 + 4 lg + e.  A step starts on a chunk boundary (g0 is a
      // multiple of 32 and C <= 64 is a power of two >= 8), so the lane's 4
      // tokens of each half share a chunk: two mask bits per lane, from one
      // shift of the head's mask.
      const int nvalid = tok_end - g0;
      bf16x8_t pa[kBlkNB];
#pragma unroll
      for (int nb = 0; nb < kBlkNB; ++nb) {
        float x[8];
        float mloc = -INFINITY;
        const uint32_t smask = qvalid[nb] ? (uint32_t)(qmask[nb] >> ((g0 >> lc) - chunk0)) : 0u;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const bool on = ((smask >> ((nt * 16 + 4 * lg) >> lc)) & 1u) != 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = nt * 16 + 4 * lg + e;
            const float v = (on & (t < nvalid)) ? st[nb][nt][e] : -INFINITY;
            x[nt * 4 + e] = v;
            mloc = fmaxf(mloc, v);
          }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
        const float m_new = fmaxf(m_i[nb], mloc);
        if (__ballot(m_new != m_i[nb]) != 0ull) {  // some head's maximum moved: rescale
          const float sc = m_i[nb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_i[nb] - m_new) * c2);
          l_i[nb] *= sc;
          // O rows 4 lg + e belong to heads 4 lg + e: rescale by their factors.
          float sr[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) sr[e] = __shfl(sc, 4 * lg + e, kWave);
#pragma unroll
          for (int n = 0; n < NTD; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[nb][n][e] *= sr[e];
          m_i[nb] = m_new;
        }
        const float mc = m_i[nb] == -INFINITY ? 0.f : m_i[nb] * c2;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pj = __builtin_amdgcn_exp2f(fmaf(x[j], c2, -mc));
          l_i[nb] += pj;
          pa[nb][j] = (__bf16)pj;
        }
      }
      // B = V in the same token order: lane (li, lg) needs tokens 4 lg + (0..3)
      // and 16 + 4 lg + (0..3) of column n * 16 + li.  ds_read_b64_tr_b16
      // (gfx950, checked): each lane addresses 4 consecutive bf16 values, and
      // lane i of each 16-lane group receives as its element k (k = 0..3) value
      // i % 4 of those that lane 4 k + i / 4 of the group addresses.  So lane
      // (s, lg) addresses row 4 lg + s / 4 (+ 16 for the second half),
      // columns n * 16 + 4 (s % 4) .. + 3.  Each V^T operand serves every
      // block of the wave.
      const uint16_t* vsrc = &s_v[(4 * lg + (li >> 2)) * VROW + 4 * (li & 3)];
#pragma unroll
      for (int n = 0; n < NTD; ++n) {
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(vsrc + n * 16));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16_t*)(vsrc + 16 * VROW + n * 16));
        const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
        const uint4 w = make_uint4(a.x, a.y, b.x, b.y);
#pragma unroll
        for (int nb = 0; nb < kBlkNB; ++nb)
          o[nb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[nb], __builtin_bit_cast(bf16x8_t, w),
                                                             o[nb][n], 0, 0, 0);
      }
    };
    const bool wave_live = wave * kBlkNB * 16 < ne;
    int g0 = next_step(tok0);
    int g1 = next_step(g0 + kBlkGroup);
    fetch(ka, va, g0);
    fetch(kb, vb, g1);
    while (g0 < tok_end) {
      __syncthreads();
      stage(ka, va);
      __syncthreads();
      int g2 = next_step(g1 + kBlkGroup);
      fetch(ka, va, g2);
      if (wave_live) compute(g0);  // waves past the block's heads only stage
      g0 = g1;
      g1 = g2;
      if (g0 >= tok_end) break;
      __syncthreads();
      stage(kb, vb);
      __syncthreads();
      g2 = next_step(g1 + kBlkGroup);
      fetch(kb, vb, g2);
      if (wave_live) compute(g0);
      g0 = g1;
      g1 = g2;
    }
#pragma unroll
    for (int nb = 0; nb < kBlkNB; ++nb) {
      float l = l_i[nb];
      l += __shfl_xor(l, 16, kWave);
      l += __shfl_xor(l, 32, kWave);
      // Partials: O rows 4 lg + e (heads of the block), columns n * 16 + li;
      // m and l from the lanes of row group 0.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = (wave * kBlkNB + nb) * 16 + 4 * lg + e;
        if (r < ne && s_slot[r] >= 0) {
          float* pr = P.part + (int64_t)s_slot[r] * (D + 2);
#pragma unroll
          for (int n = 0; n < NTD; ++n) pr[n * 16 + li] = o[nb][n][e];
        }
      }
      if (lg == 0 && qvalid[nb]) {
        float* pr = P.part + (int64_t)s_slot[qi[nb]] * (D + 2);
        pr[D] = m_i[nb] * inv;
        pr[D + 1] = l;
      }
    }
  }
}

// kGL lanes per head (four heads per wave): the head's sink (when chunk 0 is
// not selected) and its partial-chunk tokens, then the merge with its pairs'
// partials (in tile order); a failed route gives a NaN row.  Loads that do not
// depend on each other are issued together, and the partials kSB at a time.
template <typename T, int D, bool POW2, bool BUF>
__global__ __launch_bounds__(kThreads) void blk_merge_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, T* __restrict__ O,
    AttnArgs a, BlkLayout L, char* scr) {
  constexpr int DPL = D / kGL;  // dimensions per lane
  BlkPtrs P(scr, L);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int gl = lane & (kGL - 1), gg = lane / kGL;
  const int64_t head = ((int64_t)blockIdx.x * kWaves + wave) * kHPW + gg;
  const bool hv = head < a.n_heads;
  const int64_t hh = hv ? head : 0;
  // Independent loads first: the head's counts, slot base, first chunk and query.
  const int n = hv ? P.ntile[hh] : -3;
  const int c = cnt[hh];
  const int qb = P.qbase[hh];  // meaningful only when n >= 0
  const int first = sel[hh * a.cap];
  float q[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) q[e] = load_elem(Q + hh * D, gl * DPL + e);
  // Every lane of the wave runs the same number of steps (shuffles below).
  const int64_t Th = visible_len(a, hh);  // valid when n >= 0
  const int64_t n1 = Th / a.C;
  const bool sink = n >= 0 && n1 > 0 && (c == 0 || first != 0);
  const int ne = n >= 0 ? (sink ? 1 : 0) + (int)(Th - n1 * a.C) : 0;
  const int ne_max = (int)wave_allreduce_u64((uint64_t)ne, OpMax());
  const int64_t nblk = kv_block_elems(a.Tc, a.C, D, a.chunked);
  const T* Kb = K + tree_of_head(hh, a) * nblk;
  const T* Vb = a.chunked ? Kb + (int64_t)a.C * D : V + tree_of_head(hh, a) * nblk;
  const int64_t row1 = n1 * (a.chunked ? 2 * a.C : a.C);  // first key row of chunk n_1
  const float inv = 1.0f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  // The sink and partial-chunk tokens, kXB at a time: every row load of a
  // batch issues before the first is used (causal prefill has up to C of them
  // per head); the online update still takes the tokens one by one, in order.
  constexpr int kXB = 4;
  for (int x0 = 0; x0 < ne_max; x0 += kXB) {
    float kr[kXB][DPL], vr[kXB][DPL];
#pragma unroll
    for (int u = 0; u < kXB; ++u) {
      const int x = x0 + u;
      const bool on = x < ne;
      const int64_t row = !on ? 0 : (sink && x == 0) ? 0 : row1 + (x - (sink ? 1 : 0));
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        kr[u][e] = load_elem(Kb + row * D, gl * DPL + e);
        vr[u][e] = load_elem(Vb + row * D, gl * DPL + e);
      }
    }
    float sc[kXB];
#pragma unroll
    for (int u = 0; u < kXB; ++u) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) part = fmaf(q[e], kr[u][e], part);
      sc[u] = x0 + u < ne_max ? group_allreduce<kGL>(part, OpAdd()) * inv : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kXB; ++u) {
      if (x0 + u < ne) {
        const float mn = fmaxf(m, sc[u]);
        const float r = __expf(m - mn), pw = __expf(sc[u] - mn);
        l = l * r + pw;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pw, vr[u][e], acc[e] * r);
        m = mn;
      }
    }
  }
  if (n == -2) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem(O + head * D, gl * DPL + e, __int_as_float(0x7fc00000));
  } else if (n >= 0) {
    // The pairs' partials, kSB at a time (indices clamped: every load issues).
    constexpr int kSB = 8;
    const float* slots = P.part + (int64_t)qb * (D + 2);
    float M = m, den = l, num[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) num[e] = acc[e];
    for (int s0 = 0; s0 < n; s0 += kSB) {
      float ms[kSB], ls[kSB], os[kSB][DPL];
#pragma unroll
      for (int j = 0; j < kSB; ++j) {
        const float* r = slots + (int64_t)min(s0 + j, n - 1) * (D + 2);
        ms[j] = r[D];
        ls[j] = r[D + 1];
#pragma unroll
        for (int e = 0; e < DPL; ++e) os[j][e] = r[gl * DPL + e];
        if (s0 + j >= n) ms[j] = -INFINITY;
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < kSB; ++j) Mn = fmaxf(Mn, ms[j]);
      if (Mn == -INFINITY) continue;
      const float rs = M == -INFINITY ? 0.f : __expf(M - Mn);
      den *= rs;
#pragma unroll
      for (int e = 0; e < DPL; ++e) num[e] *= rs;
#pragma unroll
      for (int j = 0; j < kSB; ++j) {
        const float w = ms[j] == -INFINITY ? 0.f : __expf(ms[j] - Mn);
        den = fmaf(w, ls[j], den);
#pragma unroll
        for (int e = 0; e < DPL; ++e) num[e] = fmaf(w, os[j][e], num[e]);
      }
      M = Mn;
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem(O + head * D, gl * DPL + e, num[e] / den);
  }
}

// Heads past the slot budget: a few persistent workgroups find them (each
// thread tests one head per pass, heads spread over the workgroups so that a
// run of marked heads is shared out) and attend them one per workgroup.
constexpr unsigned kBlkFallbackBlocks = 256;
template <typename T, int D, bool POW2, bool BUF>
__global__ __launch_bounds__(kThreads) void blk_fallback_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ cnt, T* __restrict__ O,
    AttnArgs a, BlkLayout L, char* scr) {
  BlkPtrs P(scr, L);
  __shared__ int64_t s_list[kThreads];
  __shared__ int s_n;
  AttnArgs a1 = a;
  a1.S = 1;
  const int tid = threadIdx.x;
  for (int64_t base = 0; base < a.n_heads; base += (int64_t)gridDim.x * kThreads) {
    const int64_t h = base + (int64_t)tid * gridDim.x + blockIdx.x;
    const bool f = h < a.n_heads && P.ntile[h] == -1;
    if (tid == 0) s_n = 0;
    __syncthreads();
    if (f) s_list[atomicAdd(&s_n, 1)] = h;
    __syncthreads();
    const int nl = s_n;
    for (int j = 0; j < nl; ++j) {
      attend_one_head<T, D, POW2, BUF>(Q, K, V, sel, cnt, O, nullptr, a1, s_list[j], 0);
      __syncthreads();  // the next head reuses the LDS areas
    }
  }
}

template <typename T, int D, bool POW2, bool BUF>
int launch_blk(const AttnArgs& a, const void* Q, const void* K, const void* V, const int32_t* sel,
               const int32_t* cnt, void* O, void* scratch, hipStream_t s) {
  const BlkLayout L =
      blk_layout(a.n_heads, a.n_heads / ((int64_t)a.n_pos * a.H_q) * a.H_kv, a.T, a.C, D);
  char* scr = reinterpret_cast<char*>(scratch);
  const unsigned lane_blocks = (unsigned)((a.n_heads + kLaneHeads - 1) / kLaneHeads);
  const int64_t n_trees = a.n_heads / ((int64_t)a.n_pos * a.H_q) * a.H_kv;
  const unsigned tree_blocks =
      (unsigned)(n_trees * (((int64_t)a.n_pos * a.G + kLaneHeads - 1) / kLaneHeads));
  const unsigned group_blocks = (unsigned)((a.n_heads + kWaves * kHPW - 1) / (kWaves * kHPW));
  blk_count_kernel<<<lane_blocks, kLaneThreads, 0, s>>>(sel, cnt, a, L, scr);
  blk_scan_kernel<<<(unsigned)((a.n_heads + kScanChunk - 1) / kScanChunk), 1024, 0, s>>>(
      a.n_heads, L, scr);
  blk_tcount_kernel<<<tree_blocks, kLaneThreads, 0, s>>>(sel, cnt, a, L, scr);
  const bool nb2 = a.n_heads >= (int64_t)kBlkNB2Heads * L.NTT;  // many heads per tile
  blk_tscan_kernel<<<1, 1024, 0, s>>>(L, scr, nb2 ? BlkShape<2>::kQ : BlkShape<1>::kQ);
  blk_fill_kernel<<<tree_blocks, kLaneThreads, 0, s>>>(sel, cnt, a, L, scr);
  if (nb2)
    blk_attn_kernel<D, BUF, 2><<<BlkShape<2>::kGrid, 256, 0, s>>>(
        reinterpret_cast<const bf16_t*>(Q), reinterpret_cast<const bf16_t*>(K),
        reinterpret_cast<const bf16_t*>(V), a, L, scr);
  else
    blk_attn_kernel<D, BUF, 1><<<BlkShape<1>::kGrid, 256, 0, s>>>(
        reinterpret_cast<const bf16_t*>(Q), reinterpret_cast<const bf16_t*>(K),
        reinterpret_cast<const bf16_t*>(V), a, L, scr);
  blk_merge_kernel<T, D, POW2, BUF><<<group_blocks, kThreads, 0, s>>>(
      reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K),
      reinterpret_cast<const T*>(V), sel, cnt, reinterpret_cast<T*>(O), a, L, scr);
  blk_fallback_kernel<T, D, POW2, BUF><<<kBlkFallbackBlocks, kThreads, 0, s>>>(
      reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K),
      reinterpret_cast<const T*>(V), sel, cnt, reinterpret_cast<T*>(O), a, L, scr);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

template <typename T, int D>
int launch_attn(const AttnArgs& a, const void* Q, const void* K, const void* V,
                const int32_t* sel, const int32_t* cnt, void* O, void* scratch, hipStream_t s) {
  if (a.n_heads <= kBalMaxHeads) {
    int64_t* plan = reinterpret_cast<int64_t*>(scratch);
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(scratch) +
                                           align256((a.n_heads + 2) * 8));
    const bool buf =
        kv_block_elems(a.Tc, a.C, D, a.chunked) * (int64_t)sizeof(T) < ((int64_t)1 << 31);
#define ZHA_BAL(P2, BF)                                                                    \
  attn_balanced_kernel<T, D, P2, BF><<<(unsigned)a.S, kThreads, 0, s>>>(                  \
      reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K),                       \
      reinterpret_cast<const T*>(V), sel, cnt, reinterpret_cast<T*>(O), part, plan, a)
    if (a.log2C >= 0) {
      if (buf) ZHA_BAL(true, true); else ZHA_BAL(true, false);
    } else {
      if (buf) ZHA_BAL(false, true); else ZHA_BAL(false, false);
    }
#undef ZHA_BAL
    if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
    merge_balanced_kernel<T, D><<<(unsigned)a.n_heads, kThreads, 0, s>>>(
        part, plan, cnt, a, reinterpret_cast<T*>(O));
    return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
  }
  const bool buf =
      kv_block_elems(a.Tc, a.C, D, a.chunked) * (int64_t)sizeof(T) < ((int64_t)1 << 31);
  if constexpr (sizeof(T) == 2 && (D == 64 || D == 128)) {
    if (blk_eligible(a.n_heads, a.C, D, a.dtype)) {
      if (buf) return launch_blk<T, D, true, true>(a, Q, K, V, sel, cnt, O, scratch, s);
      return launch_blk<T, D, true, false>(a, Q, K, V, sel, cnt, O, scratch, s);
    }
  }
  // Many heads: one workgroup per head, written directly.
  AttnArgs a1 = a;
  a1.S = 1;
  dim3 grid((unsigned)a.n_heads, 1u);
#define ZHA_PART(P2, BF)                                                                    \
  attn_partial_kernel<T, D, P2, BF><<<grid, kThreads, 0, s>>>(                              \
      reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K),                        \
      reinterpret_cast<const T*>(V), sel, cnt, reinterpret_cast<T*>(O), nullptr, a1)
  if (a.log2C >= 0) {
    if (buf) ZHA_PART(true, true); else ZHA_PART(true, false);
  } else {
    if (buf) ZHA_PART(false, true); else ZHA_PART(false, false);
  }
#undef ZHA_PART
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

// Dense decode on the matrix cores (bf16 caches, d in {64, 128}).  S waves
// per (KV cache, 16 query rows); wave s takes the 32-token steps s, s + S,
// s + 2S, ... (so the grid sweeps each cache nearly in address order, which
// measured faster than one contiguous range per wave).  The waves share
// nothing, so the token loop has no workgroup barrier.  Per step:
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16: K rows go from memory straight
//   into the A operand (lane i + 16 g holds dims 32 ks + 8 g .. + 7 of token
//   i), Q is the B operand, held for the whole range;
//   P V with the same instruction: a lane's 8 probabilities (one query row,
//   tokens 16 nt + 4 g + e) are its A operand, and V reaches the B operand
//   transposed through a wave-private LDS area, as 32-bit words holding one
//   dimension of two consecutive tokens.
// The next step's rows are loaded before the current step computes; their
// token indices are clamped into the cache, so every load is unconditional
// and each wait counts exactly the loads issued after it (rows past the range
// are masked).  The output rescale runs only when some row's maximum moved.
// LAY: 0 split caches, 1 chunked with C a power of two, 2 chunked otherwise.
#ifndef ZHA_DENSE_STRIDED
#define ZHA_DENSE_STRIDED 1
#endif
template <int D, int LAY>
__global__ __launch_bounds__(256) void dense_mfma_kernel(const bf16_t* __restrict__ Q,
                                                         const bf16_t* __restrict__ K,
                                                         const bf16_t* __restrict__ V,
                                                         bf16_t* __restrict__ O,
                                                         float* __restrict__ part, DenseArgs a) {
  constexpr int KS = D / 32;   // k-steps of S^T, and 16-byte V segments per lane and row
  constexpr int NTD = D / 16;  // 16-column tiles of O
  constexpr int VTW = 17;      // LDS row of V^T in 32-bit words (16 token pairs), padded
  __shared__ uint32_t s_vt[4][D * VTW];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int R = a.n_pos * a.G;  // query rows per KV cache
  const int RT = (R + 15) >> 4;
  const int64_t n_trees = a.n_heads / ((int64_t)a.n_pos * a.H_q) * a.H_kv;
  const int64_t item = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(wave);
  if (item >= n_trees * RT * a.S) return;  // the whole wave; no workgroup barrier follows
  const int split = (int)(item % a.S);
  const int64_t rest = item / a.S;
  const int rt = (int)(rest % RT);
  const int64_t tr = rest / RT;
  const int64_t b = tr / a.H_kv;
  const int kvh = (int)(tr - b * a.H_kv);
  auto head_of = [&](int r) {
    return (b * a.n_pos + r / a.G) * a.H_q + (int64_t)kvh * a.G + r % a.G;
  };
  const int64_t nblk = kv_block_elems(a.Tc, a.C, D, a.chunked);
  const char* Kc = reinterpret_cast<const char*>(K + tr * nblk);
  const char* Vc = reinterpret_cast<const char*>(LAY != 0 ? K + tr * nblk + (int64_t)a.C * D
                                                          : V + tr * nblk);
  // Steps of this wave: 32-token blocks at g = gbase + i gstride, i < ns, tokens
  // below lim.  Interleaved: the S waves of a (cache, 16 rows) take every S-th
  // step, so the whole grid sweeps the cache nearly in address order.
  const int T = (int)a.T;
#if ZHA_DENSE_STRIDED
  const int gbase = split * 32, gstride = a.S * 32, lim = T;
  const int ns = ((T + 31) / 32 - split + a.S - 1) / a.S;
#else
  const int gbase = (int)(split * a.tps), gstride = 32, lim = (int)min((int64_t)gbase + a.tps, a.T);
  const int ns = (lim - gbase + 31) / 32;
#endif
  // First row of the step (wave-uniform) and 32-bit byte offsets of its tokens.
  auto row0 = [&](int g) -> int64_t {
    if constexpr (LAY == 1) return (int64_t)g + ((g >> a.log2C) << a.log2C);
    if constexpr (LAY == 2) return (int64_t)g + (int64_t)(g / a.C) * a.C;
    return g;
  };
  auto off_of = [&](int g, int v) -> uint32_t {  // token g + v, clamped below lim
    v = min(v, lim - 1 - g);
    if constexpr (LAY == 1) v += (((g & (a.C - 1)) + v) >> a.log2C) << a.log2C;
    if constexpr (LAY == 2) v += ((g % a.C) + v) / a.C * a.C;
    return (uint32_t)v * (uint32_t)(D * 2);
  };

  // Q rows as the B operand: lane (li, lg) holds row li's dims 32 ks + 8 lg .. + 7.
  const int qr = rt * 16 + li;
  bf16x8_t qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (qr < R) v = ld16c(Q + head_of(qr) * D + ks * 32 + lg * 8);
    qb[ks] = __builtin_bit_cast(bf16x8_t, v);
  }

  // V staging: lane (li, lg) holds rows 2 li and 2 li + 1 of the step, 16-byte
  // segments lg + 4 s; K: lane (li, lg) holds row nt * 16 + li, segments lg + 4 ks.
  uint4 kb[2 * KS], vb[2 * KS];
  auto load_v = [&](int g) {
    const char* vbase = Vc + row0(g) * (D * 2);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const char* vr = vbase + (off_of(g, 2 * li + p) + lg * 16);
#pragma unroll
      for (int s = 0; s < KS; ++s) vb[p * KS + s] = ld16(vr + s * 64);
    }
  };
  auto load_k = [&](int g) {
    const char* kbase = Kc + row0(g) * (D * 2);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const char* kr = kbase + (off_of(g, nt * 16 + li) + lg * 16);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[nt * KS + ks] = ld16(kr + ks * 64);
    }
  };
  uint32_t* vt = s_vt[wave];
  auto stage_v = [&]() {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint32_t v0[4] = {vb[s].x, vb[s].y, vb[s].z, vb[s].w};
      const uint32_t v1[4] = {vb[KS + s].x, vb[KS + s].y, vb[KS + s].z, vb[KS + s].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dim = (lg + 4 * s) * 8 + 2 * e;
        vt[dim * VTW + li] = (v0[e] & 0xffffu) | (v1[e] << 16);
        vt[(dim + 1) * VTW + li] = (v0[e] >> 16) | (v1[e] & 0xffff0000u);
      }
    }
  };

  const float c2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
  float m_i = -INFINITY, l_i = 0.f;  // m in raw score units; l summed per lane
  f32x4_t o[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Step i: stage V(i); load V(i + 1); S^T from K(i); load K(i + 1) into the
  // same registers; softmax and P V.  Loads are issued V before K, so each
  // wait leaves the other tensor's loads in flight.  LDS accesses of one wave
  // complete in order; the empty asm statements keep the compiler from moving
  // them across steps.
  load_v(gbase);
  __builtin_amdgcn_sched_barrier(0);
  load_k(gbase);
  for (int i = 0; i < ns; ++i) {
    const int g = gbase + i * gstride;
    const int gn = i + 1 < ns ? g + gstride : g;  // past the last step: its rows again
    asm volatile("" ::: "memory");
    stage_v();
    asm volatile("" ::: "memory");
    load_v(gn);
    __builtin_amdgcn_sched_barrier(0);
    f32x4_t st[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      st[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb[nt * KS + ks]),
                                                        qb[ks], st[nt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_k(gn);
    __builtin_amdgcn_sched_barrier(0);
    const int nvalid = lim - g;
    float x[8], mloc = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = nt * 16 + 4 * lg + e < nvalid ? st[nt][e] : -INFINITY;
        x[nt * 4 + e] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    const float m_new = fmaxf(m_i, mloc);
    if (__ballot(m_new != m_i) != 0ull) {  // some row's maximum moved: rescale
      const float sc = m_i == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_i - m_new) * c2);
      l_i *= sc;
      float sr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sr[e] = __shfl(sc, 4 * lg + e, kWave);
#pragma unroll
      for (int n = 0; n < NTD; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[n][e] *= sr[e];
      m_i = m_new;
    }
    const float mc = m_i == -INFINITY ? 0.f : m_i * c2;
    bf16x8_t pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pj = __builtin_amdgcn_exp2f(fmaf(x[j], c2, -mc));
      l_i += pj;
      pa[j] = (__bf16)pj;
    }
#pragma unroll
    for (int n = 0; n < NTD; ++n) {
      const uint32_t* vr = &vt[(n * 16 + li) * VTW];
      const uint4 w = make_uint4(vr[2 * lg], vr[2 * lg + 1], vr[8 + 2 * lg], vr[9 + 2 * lg]);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8_t, w), o[n], 0,
                                                     0, 0);
    }
  }

  l_i += __shfl_xor(l_i, 16, kWave);
  l_i += __shfl_xor(l_i, 32, kWave);
  // O rows 4 lg + e, columns 16 n + li.
  float lr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) lr[e] = __shfl(l_i, 4 * lg + e, kWave);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = rt * 16 + 4 * lg + e;
    if (r >= R) continue;
    const int64_t h = head_of(r);
    if (a.S == 1) {
#pragma unroll
      for (int n = 0; n < NTD; ++n) store_elem(O + h * D, n * 16 + li, o[n][e] / lr[e]);
    } else {
      float* pr = part + (h * a.S + split) * (D + 2);
#pragma unroll
      for (int n = 0; n < NTD; ++n) pr[n * 16 + li] = o[n][e];
    }
  }
  if (a.S > 1 && lg == 0 && qr < R) {
    float* pr = part + (head_of(qr) * a.S + split) * (D + 2);
    pr[D] = m_i * (1.0f / sqrtf((float)D));
    pr[D + 1] = l_i;
  }
}

template <int D>
int launch_dense_mfma(const DenseArgs& a, const void* Q, const void* K, const void* V, void* O,
                      void* scratch, hipStream_t s) {
  const int64_t n_trees = a.n_heads / ((int64_t)a.n_pos * a.H_q) * a.H_kv;
  const int64_t items = n_trees * ((a.n_pos * a.G + 15) / 16) * a.S;
  float* part = reinterpret_cast<float*>(scratch);
#define ZHA_DM(LAY)                                                                   \
  dense_mfma_kernel<D, LAY><<<(unsigned)((items + 3) / 4), 256, 0, s>>>(                \
      reinterpret_cast<const bf16_t*>(Q), reinterpret_cast<const bf16_t*>(K),           \
      reinterpret_cast<const bf16_t*>(V), reinterpret_cast<bf16_t*>(O), part, a)
  if (!a.chunked) ZHA_DM(0);
  else if (a.log2C >= 0) ZHA_DM(1);
  else ZHA_DM(2);
#undef ZHA_DM
  if (a.S > 1) {
    if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
    merge_kernel<bf16_t, D><<<(unsigned)a.n_heads, kThreads, 0, s>>>(
        part, nullptr, 0, reinterpret_cast<bf16_t*>(O), a.S);
  }
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

template <typename T, int D, int GT>
int launch_dense_gt(const DenseArgs& a, const void* Q, const void* K, const void* V, void* O,
                    void* scratch, hipStream_t s) {
  const int64_t groups = (a.n_heads / a.H_q) * a.H_kv * (a.G / GT);
  dim3 grid((unsigned)groups, (unsigned)a.S);
  float* part = reinterpret_cast<float*>(scratch);
  dense_partial_kernel<T, D, GT><<<grid, kThreads, 0, s>>>(
      reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K),
      reinterpret_cast<const T*>(V), reinterpret_cast<T*>(O), part, a);
  if (a.S > 1) {
    if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
    merge_kernel<T, D><<<(unsigned)a.n_heads, kThreads, 0, s>>>(part, nullptr, 0,
                                                                reinterpret_cast<T*>(O), a.S);
  }
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

template <typename T, int D>
int launch_dense(const DenseArgs& a, const void* Q, const void* K, const void* V, void* O,
                 void* scratch, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && (D == 64 || D == 128))
    return launch_dense_mfma<D>(a, Q, K, V, O, scratch, s);
  const int gt = dense_head_tile(a.G);
  if (gt == 8) return launch_dense_gt<T, D, 8>(a, Q, K, V, O, scratch, s);
  if (gt == 4) return launch_dense_gt<T, D, 4>(a, Q, K, V, O, scratch, s);
  if (gt == 2) return launch_dense_gt<T, D, 2>(a, Q, K, V, O, scratch, s);
  return launch_dense_gt<T, D, 1>(a, Q, K, V, O, scratch, s);
}

}  // namespace

int attn_dispatch(const AttnArgs& a, int dtype, int d, const void* Q, const void* K,
                  const void* V, const int32_t* sel, const int32_t* cnt, void* O, void* scratch,
                  hipStream_t s) {
#define ZHA_ATTN_CASE(TT, DD) \
  if (d == DD) return launch_attn<TT, DD>(a, Q, K, V, sel, cnt, O, scratch, s);
  if (dtype == ZHA_BF16) {
    ZHA_ATTN_CASE(bf16_t, 64)
    ZHA_ATTN_CASE(bf16_t, 128)
    ZHA_ATTN_CASE(bf16_t, 256)
  } else {
    ZHA_ATTN_CASE(float, 64)
    ZHA_ATTN_CASE(float, 128)
    ZHA_ATTN_CASE(float, 256)
  }
#undef ZHA_ATTN_CASE
  return ZHA_ERR_DIM;
}

int dense_dispatch(const DenseArgs& a, int dtype, int d, const void* Q, const void* K,
                   const void* V, void* O, void* scratch, hipStream_t s) {
#define ZHA_DENSE_CASE(TT, DD) \
  if (d == DD) return launch_dense<TT, DD>(a, Q, K, V, O, scratch, s);
  if (dtype == ZHA_BF16) {
    ZHA_DENSE_CASE(bf16_t, 64)
    ZHA_DENSE_CASE(bf16_t, 128)
    ZHA_DENSE_CASE(bf16_t, 256)
  } else {
    ZHA_DENSE_CASE(float, 64)
    ZHA_DENSE_CASE(float, 128)
    ZHA_DENSE_CASE(float, 256)
  }
#undef ZHA_DENSE_CASE
  return ZHA_ERR_DIM;
}

}  // namespace zha
