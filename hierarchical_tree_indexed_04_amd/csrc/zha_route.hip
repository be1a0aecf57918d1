// Top-down top-p routing through the summary tree.
//
// "Subquadratic Attention with a Hierarchical Tree-Structured Indexer" §III-C
// and the summary page's "Routing" paragraph: at every level the candidates
// (the frontier) are scored with the max over tangents, ordered by score, and
// the shortest prefix whose share of the frontier's softmax mass reaches p is
// kept; the kept nodes' children (plus nodes with no complete parent, App.
// E-E) form the next frontier.  The order is score descending, ties to the
// lower node id.
//
// One workgroup (8 waves) per query head walks all levels in one launch.  The
// frontier, its scores and the cut's histograms stay in LDS; only the summary
// rows of the candidates are read from memory (cached loads: the upper levels
// are shared by every query head of the group).
//
// The cut never sorts the frontier.  Each candidate carries the 64-bit key
// (~ord(score) << 32 | id), whose ascending order is exactly the required
// order, and the fixed-point mass W = floor(exp(s - s_max) * 2^40).  Integer
// masses make every partial sum exact, hence independent of summation order:
// the result is deterministic and the prefix test W_m >= p Z is evaluated on
// the exact sums of the quantised weights.
//   * Frontiers of at most 64 candidates: every wave holds one candidate per
//     lane; candidate i is kept iff the mass of all smaller keys is < p Z, the
//     sum over smaller keys being split across the waves.
//   * Larger frontiers: a 256-bucket histogram over (s_max - s) (monotone in
//     the key) finds the bucket where the running mass crosses p Z; 8-bit
//     radix passes over the keys narrow a crowded bucket (ties in score fall
//     to the id bits) until at most 64 candidates remain, which wave 0 then
//     ranks.  kappa, the largest kept key, defines the cut: kept = {key <= kappa}.
// Compaction keeps ascending id order with per-wave ballots, and the next
// frontier is written as children of the kept nodes.
//
// Reductions and scans use DPP lane moves (zha_wave.hpp).

#include "zha_internal.hpp"
#include "zha_wave.hpp"

namespace zha {
namespace {

#ifndef ZHA_ROUTE_THREADS
#define ZHA_ROUTE_THREADS 512
#endif
constexpr int kThreads = ZHA_ROUTE_THREADS;  // 256 or 512
constexpr int kWaves = kThreads / kWave;
static_assert(kThreads >= 256, "histograms are cleared one bucket per thread");
#ifndef ZHA_ROUTE_ROWS
#define ZHA_ROUTE_ROWS 16
#endif
#ifndef ZHA_ROUTE_XCD
#define ZHA_ROUTE_XCD 1
#endif
constexpr int kU = ZHA_ROUTE_ROWS;  // summary rows in flight per lane while scoring
constexpr int kMaxChildren = 1024;  // C <= 1024

#ifndef ZHA_ROUTE_PROFILE
#define ZHA_ROUTE_PROFILE 0
#endif

__device__ __forceinline__ uint64_t make_key(float s, int32_t id) {
  return ((uint64_t)(~ord_f32(s)) << 32) | (uint32_t)id;
}
__device__ __forceinline__ float key_score(uint64_t k) { return unord_f32(~(uint32_t)(k >> 32)); }

// floor(exp(s - smax) * 2^40), exactly: w * 2^8 = hi + frac with frac in [0, 1).
__device__ __forceinline__ uint64_t fixed_mass(float s, float smax) {
  const float t = __expf(s - smax) * 256.0f;
  const uint32_t hi = (uint32_t)t;
  const uint32_t lo = (uint32_t)((t - (float)hi) * 4294967296.0f);
  return ((uint64_t)hi << 32) | lo;
}

template <int FMAX>
struct RouteSmem {
  int32_t fr[2][FMAX];               // frontier node ids, ascending (ping-pong)
  float sc[FMAX];                    // scores of the current frontier
  uint32_t hcnt[256];                // histogram: candidates per bucket
  unsigned long long hmass[256];     // histogram: fixed-point mass per bucket
  unsigned long long bkey[kWave];    // boundary candidates
  unsigned long long bw[kWave];
  unsigned long long part[kWaves][kWave];   // small cut: partial masses below each lane
  float pre[kMaxChildren];                  // scores of the top candidate's children
  uint32_t wcnt[FMAX / kThreads * kWaves];  // kept per (round, wave)
  float redf[2][kWaves];
  unsigned long long redu[2][kWaves];
  unsigned long long kappa, next, base, kmask;
  double target;
  int32_t bstar, bcount, bl_n;
};

// Where a batch item lives: its level's k_hat / b_hat and its node id.
struct Loc {
  const char* k;
  const float* b;
  int node;
};

// Scores items [0, NI) of a batch into out[] (LDS): s = max_r (q . k_hat_r +
// b_hat_r) over the R tangents of the item's node, q pre-scaled by 1/sqrt(d).
// LPR lanes read one 16-byte slice each of a summary row; kU rows per lane are
// in flight.  Ends with a barrier.
template <typename T, int D, bool R1, typename Locate>
__device__ __forceinline__ void score_items(float* out, int NI, int R, Locate locate,
                                            const float* q) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = kThreads / LPR;
  const int tid = threadIdx.x;
  const int sub = tid % LPR, grp = tid / LPR;
  uint32_t* outu = reinterpret_cast<uint32_t*>(out);
  if (!R1) {
    for (int i = tid; i < NI; i += kThreads) outu[i] = 0u;
    __syncthreads();
  }
  const int NR = R1 ? NI : NI * R;
  for (int base = 0; base < NR; base += RPB * kU) {
    // Slots beyond the last live row are skipped with uniform branches: a
    // wave64 VALU op costs the SIMD 4 cycles, so dead slots are not free.
    const int nu = min(kU, (NR - base + RPB - 1) / RPB);
    uint4 v[kU];
    float bias[kU];
    // Loads are straight-line (dead slots are masked lanes, no traffic) so
    // each slot's wait counts exactly the loads still in flight after it.
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int x = base + u * RPB + grp;
      if (x < NR) {
        const int item = R1 ? x : x / R;
        const int r = R1 ? 0 : x - item * R;
        const Loc lc = locate(item);
        const int64_t row = R1 ? (int64_t)lc.node : (int64_t)lc.node * R + r;
        v[u] = ld16c(lc.k + row * (int64_t)(D * sizeof(T)) + sub * 16);
        bias[u] = lc.b[row];
      } else {
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        bias[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u < nu) {
        const int x = base + u * RPB + grp;
        float k[VEC];
        Vec<T>::widen(v[u], k);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) dot = fmaf(q[e], k[e], dot);
        dot = group_allreduce<LPR>(dot, OpAdd());
        if (sub == 0 && x < NR) {
          const float s = dot + bias[u];
          if (R1)
            out[x] = s;
          else
            atomicMax(&outu[x / R], ord_f32(s));
        }
      }
    }
  }
  if (!R1) {
    __syncthreads();
    for (int i = tid; i < NI; i += kThreads) out[i] = unord_f32(outu[i]);
  }
  __syncthreads();
}

// Waves 1 .. kWaves-1, while wave 0 cuts a frontier of K <= 64 candidates:
// the top candidate (largest score, lowest id) is kept by every cut (nothing
// precedes it, so its preceding mass 0 is < p Z), so its C children are
// certainly in the next frontier.  Score them now (one tangent per node) into
// pre[]; when the cut keeps only that node and the next level has no
// orphans, the next frontier is exactly these children and its scoring costs
// no memory round trip.
template <typename T, int D, int FMAX>
__device__ __forceinline__ void score_top_children(RouteSmem<FMAX>& sm, const float* sc,
                                                   const int32_t* fr, int K, int C,
                                                   const char* khat, const float* bhat,
                                                   const float* q) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPW = kWave / LPR;  // rows per wave and pass
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const bool valid = lane < K;
  const uint64_t key = valid ? make_key(sc[lane], fr[lane]) : ~0ull;
  const int top = (int)(uint32_t)wave_allreduce_u64(key, OpMin());
  for (int c = (wave - 1) * RPW + lane / LPR; c - lane / LPR < C; c += (kWaves - 1) * RPW) {
    const int cc = min(c, C - 1);  // lanes past C recompute the last child, never stored
    const int64_t row = (int64_t)top * C + cc;
    float k[VEC];
    Vec<T>::widen(ld16c(khat + row * (int64_t)(D * sizeof(T)) + sub * 16), k);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = fmaf(q[e], k[e], dot);
    dot = group_allreduce<LPR>(dot, OpAdd());
    if (sub == 0 && c < C) sm.pre[c] = dot + bhat[row];
  }
}

// Cut of a frontier of 1 < K <= 64 candidates.  Lane i holds candidate i,
// which is kept iff the mass of the candidates with smaller keys is < p Z.
// The sum over smaller keys is split across nw = ceil(K / J) waves (wave w
// takes candidates [w J, (w + 1) J)); with nw = 1 wave 0 works alone and no
// partial goes through LDS.  Wave 0 decides and publishes the kept mask (and,
// for the gap, kappa and the smallest dropped key); the other waves only wait.
// Returns the kept mask (bit i = candidate i), the same in every wave.
template <int FMAX>
__device__ __forceinline__ uint64_t small_cut(RouteSmem<FMAX>& sm, const float* sc,
                                              const int32_t* fr, int K, float p, bool want_gap) {
  constexpr int J = kWave / kWaves;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int nw = (K + J - 1) / J;
  uint64_t key = ~0ull, w = 0, part = 0;
  if (wave < nw) {
    const bool valid = lane < K;
    const float s = valid ? sc[lane] : -INFINITY;
    const float smax = wave_max_f32_bcast(s);
    key = valid ? make_key(s, fr[lane]) : ~0ull;
    w = valid ? fixed_mass(s, smax) : 0ull;
    const int j0 = wave * J;
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int j = j0 + jj;
      if (j < K) {
        const uint64_t kj = readlane_u64(key, j);
        const uint64_t wj = readlane_u64(w, j);
        part += (kj < key) ? wj : 0ull;
      }
    }
    if (nw > 1) sm.part[wave][lane] = part;
  }
  if (nw > 1) __syncthreads();
  if (wave == 0) {
    const uint64_t Z = wave_sum_u64_bcast(w);
    uint64_t below = part;
    for (int v = 1; v < nw; ++v) below += sm.part[v][lane];
    const bool kept = lane < K && (double)below < (double)p * (double)Z;
    const uint64_t mask = __ballot(kept);
    if (lane == 0) sm.kmask = mask;
    if (want_gap) {
      const uint64_t kappa = wave_allreduce_u64(kept ? key : 0ull, OpMax());
      const uint64_t next = wave_allreduce_u64((lane < K && !kept) ? key : ~0ull, OpMin());
      if (lane == 0) {
        sm.kappa = kappa;
        sm.next = next;
      }
    }
  }
  __syncthreads();
  return sm.kmask;
}

// Wave 0: exact resolution of n <= 64 boundary candidates (one per lane).  A
// candidate is kept iff base + (mass of the candidates with smaller keys) < target.
// Writes kappa (largest kept key) to LDS.
template <int FMAX>
__device__ __forceinline__ void resolve_boundary(RouteSmem<FMAX>& sm, uint64_t key,
                                                 uint64_t w, int n, uint64_t base,
                                                 double target) {
  const int lane = threadIdx.x;
  uint64_t below = 0;
  for (int j = 0; j < n; ++j) {
    const uint64_t kj = readlane_u64(key, j);
    const uint64_t wj = readlane_u64(w, j);
    below += (kj < key) ? wj : 0ull;
  }
  const bool kept = lane < n && (double)(base + below) < target;
  const uint64_t kappa = wave_allreduce_u64(kept ? key : 0ull, OpMax());
  if (lane == 0) sm.kappa = kappa;
}

// Wave 0: scan the 256-bucket histogram from base0 and find the first bucket
// whose inclusive running mass reaches the target.  With `first`, the total
// mass Z is the histogram's sum and the target p Z is set.
template <int FMAX>
__device__ __forceinline__ void scan_find(RouteSmem<FMAX>& sm, uint64_t base0, bool first,
                                          float p) {
  const int lane = threadIdx.x;
  uint64_t c[4];
  uint64_t run = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    run += sm.hmass[4 * lane + k];
    c[k] = run;
  }
  const uint64_t incl = wave_incl_scan_u64(run);
  const uint64_t excl = incl - run;
  double target;
  if (first) {
    target = (double)p * (double)readlane_u64(incl, kWave - 1);
  } else {
    target = sm.target;
  }
  int kfound = 4;
#pragma unroll
  for (int k = 3; k >= 0; --k)
    if ((double)(base0 + excl + c[k]) >= target) kfound = k;
  const uint64_t bal = __ballot(kfound < 4);
  const int f = __ffsll((unsigned long long)bal) - 1;
  if (lane == f) {
    const int bk = 4 * lane + kfound;
    sm.bstar = bk;
    sm.bcount = (int32_t)sm.hcnt[bk];
    sm.base = base0 + excl + c[kfound] - sm.hmass[bk];
    if (first) sm.target = target;
  }
}

template <int FMAX, typename Op>
__device__ __forceinline__ uint64_t block_allreduce_u64(RouteSmem<FMAX>& sm, uint64_t v,
                                                        Op op, int slot) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  v = wave_allreduce_u64(v, op);
  if (lane == 0) sm.redu[slot][wave] = v;
  __syncthreads();
  uint64_t r = sm.redu[slot][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = op(r, (uint64_t)sm.redu[slot][w]);
  __syncthreads();
  return r;
}

// Cut of a frontier of K > 64 candidates (p < 1).  The histogram and bl_n are
// zero on entry.  Returns kappa.
template <int FMAX>
__device__ __forceinline__ uint64_t top_p_cut_large(RouteSmem<FMAX>& sm, const float* sc,
                                                    const int32_t* fr, int K, float p) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  float smax = -INFINITY, smin = INFINITY;
  for (int i = tid; i < K; i += kThreads) {
    const float s = sc[i];
    smax = fmaxf(smax, s);
    smin = fminf(smin, s);
  }
  smax = wave_allreduce_f32(smax, OpMax());
  smin = wave_allreduce_f32(smin, OpMin());
  if (lane == 0) {
    sm.redf[0][wave] = smax;
    sm.redf[1][wave] = smin;
  }
  __syncthreads();
  smax = sm.redf[0][0];
  smin = sm.redf[1][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    smax = fmaxf(smax, sm.redf[0][w]);
    smin = fminf(smin, sm.redf[1][w]);
  }

  // 1. Value-space histogram over (s_max - s).
  const float range = fminf(smax - smin, 32.f);
  const float bscale = range > 0.f ? 256.f / range : 0.f;
  auto bucket = [&](float s) { return min((int)((smax - s) * bscale), 255); };
  for (int i = tid; i < K; i += kThreads) {
    const float s = sc[i];
    const int bk = bucket(s);
    atomicAdd(&sm.hcnt[bk], 1u);
    atomicAdd(&sm.hmass[bk], (unsigned long long)fixed_mass(s, smax));
  }
  __syncthreads();
  if (wave == 0) scan_find(sm, 0ull, true, p);
  __syncthreads();
  const int bstar = sm.bstar;
  if (sm.bcount <= kWave) {
    for (int i = tid; i < K; i += kThreads) {
      const float s = sc[i];
      if (bucket(s) == bstar) {
        const int slot = atomicAdd(&sm.bl_n, 1);
        if (slot < kWave) {
          sm.bkey[slot] = make_key(s, fr[i]);
          sm.bw[slot] = fixed_mass(s, smax);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int n = min(sm.bl_n, kWave);
      resolve_boundary(sm, lane < n ? sm.bkey[lane] : ~0ull, lane < n ? sm.bw[lane] : 0ull, n,
                       sm.base, sm.target);
    }
    __syncthreads();
    return sm.kappa;
  }

  // 2. Radix refinement over the keys of the crowded bucket.  Keys are
  // distinct (ids are), so every pass fixes at least 8 more bits; the pass
  // bound is defensive.
  uint64_t lo = ~0ull, hi = 0ull;
  for (int i = tid; i < K; i += kThreads) {
    const float s = sc[i];
    if (bucket(s) == bstar) {
      const uint64_t k = make_key(s, fr[i]);
      lo = k < lo ? k : lo;
      hi = k > hi ? k : hi;
    }
  }
  lo = block_allreduce_u64(sm, lo, OpMin(), 0);
  hi = block_allreduce_u64(sm, hi, OpMax(), 1);
  for (int pass = 0;; ++pass) {
    const bool last_pass = pass >= 8 || lo == hi;
    const int hb = (lo == hi) ? 0 : 63 - __clzll((long long)(lo ^ hi));
    const int shift = hb > 7 ? hb - 7 : 0;
    if (tid < 256) {
      sm.hcnt[tid] = 0u;
      sm.hmass[tid] = 0ull;
    }
    if (tid == 0) sm.bl_n = 0;
    __syncthreads();
    for (int i = tid; i < K; i += kThreads) {
      const float s = sc[i];
      const uint64_t k = make_key(s, fr[i]);
      if (k >= lo && k <= hi) {
        const int dg = (int)((k >> shift) & 255u);
        atomicAdd(&sm.hcnt[dg], 1u);
        atomicAdd(&sm.hmass[dg], (unsigned long long)fixed_mass(s, smax));
      }
    }
    __syncthreads();
    if (wave == 0) scan_find(sm, sm.base, false, p);
    __syncthreads();
    const uint64_t top = (shift + 8 >= 64) ? 0ull : ((lo >> (shift + 8)) << (shift + 8));
    const uint64_t first = top | ((uint64_t)sm.bstar << shift);
    const uint64_t last = first | ((shift == 0) ? 0ull : ((1ull << shift) - 1));
    const uint64_t nlo = first > lo ? first : lo;
    const uint64_t nhi = last < hi ? last : hi;
    if (sm.bcount <= kWave || last_pass) {
      for (int i = tid; i < K; i += kThreads) {
        const float s = sc[i];
        const uint64_t k = make_key(s, fr[i]);
        if (k >= nlo && k <= nhi) {
          const int slot = atomicAdd(&sm.bl_n, 1);
          if (slot < kWave) {
            sm.bkey[slot] = k;
            sm.bw[slot] = fixed_mass(s, smax);
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        const int n = min(sm.bl_n, kWave);
        resolve_boundary(sm, lane < n ? sm.bkey[lane] : ~0ull, lane < n ? sm.bw[lane] : 0ull,
                         n, sm.base, sm.target);
      }
      __syncthreads();
      return sm.kappa;
    }
    lo = ~0ull;
    hi = 0ull;
    for (int i = tid; i < K; i += kThreads) {
      const uint64_t k = make_key(sc[i], fr[i]);
      if (k >= nlo && k <= nhi) {
        lo = k < lo ? k : lo;
        hi = k > hi ? k : hi;
      }
    }
    lo = block_allreduce_u64(sm, lo, OpMin(), 0);
    hi = block_allreduce_u64(sm, hi, OpMax(), 1);
  }
}

template <typename T, int D, int FMAX, bool R1>
__global__ __launch_bounds__(kThreads) void route_kernel(const char* __restrict__ tree,
                                                         const T* __restrict__ Q, RouteArgs a,
                                                         int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ stats,
                                                         float* __restrict__ gapo) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int kRounds = FMAX / kThreads;
  __shared__ RouteSmem<FMAX> sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous
  // range of heads so the heads sharing a tree share that XCD's L2.
  const int64_t head = ZHA_ROUTE_XCD ? xcd_major_index(blockIdx.x, a.n_heads) : blockIdx.x;
  const int h = (int)(head % a.H_q);
  const int64_t b = head / ((int64_t)a.n_pos * a.H_q);
  const int kvh = h / a.G;
  const char* tb = tree + (b * a.H_kv + kvh) * a.lay.stride;
  const int R = R1 ? 1 : a.lay.R;
  const int C = a.lay.C, L = a.lay.L;
  const bool want_gap = gapo != nullptr;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto khat = [&](int l) { return tb + a.lay.khat[l]; };
  auto bhat = [&](int l) { return reinterpret_cast<const float*>(tb + a.lay.bhat[l]); };

  float q[VEC];
  {
    const uint4 v = ld16c(Q + head * D + (tid % LPR) * VEC);
    Vec<T>::widen(v, q);
    const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
    for (int e = 0; e < VEC; ++e) q[e] *= inv;
  }

  int K = (int)a.lay.n[L];
  bool overflow = a.lay.n[L] > FMAX;
  if (!overflow)
    for (int i = tid; i < K; i += kThreads) sm.fr[0][i] = i;
  if (tid < 256) {
    sm.hcnt[tid] = 0u;
    sm.hmass[tid] = 0ull;
  }
  if (tid == 0) sm.bl_n = 0;
  __syncthreads();

  int cur = 0;
  int m1 = 0;
  bool ready = false;  // sm.sc already holds the frontier's scores
  for (int l = L; l >= 1 && !overflow; --l) {
    const int32_t* fr = sm.fr[cur];
    int32_t* nx = sm.fr[cur ^ 1];
#if ZHA_ROUTE_PROFILE
    const uint64_t t0 = wall_clock64();
    uint64_t t1 = t0, t2 = t0;
#endif
    const int n_orph = l > 1 ? (int)(a.lay.n[l - 1] - (int64_t)C * a.lay.n[l]) : 0;
    const int first_orphan = l > 1 ? (int)((int64_t)C * a.lay.n[l]) : 0;
    // 1. Scores of the frontier.
    const float* sc = sm.sc;
    if (K > 1 && !ready) {
      const char* k0 = khat(l);
      const float* b0 = bhat(l);
      score_items<T, D, R1>(sm.sc, K, R, [&](int x) { return Loc{k0, b0, fr[x]}; }, q);
    }
#if ZHA_ROUTE_PROFILE
    t1 = wall_clock64();
#endif
    // 2. The cut.
    const bool large = K > kWave;
    int m = 0;
    uint64_t next_key = ~0ull;
    uint64_t kappa = ~0ull;
    uint64_t kmask = 0;  // small frontier: bit i = candidate i kept
    // Small frontiers that one wave cuts alone leave the other waves free to
    // score the top candidate's children meanwhile.
    const bool pre = R1 && l > 1 && K > 1 && K <= kWave / kWaves;
    if (!large) {
      if (K > 1) {
        if (pre && wave != 0)
          score_top_children<T, D, FMAX>(sm, sc, fr, K, C, khat(l - 1), bhat(l - 1), q);
        kmask = small_cut(sm, sc, fr, K, a.p, want_gap);
        if (want_gap) {
          kappa = sm.kappa;
          next_key = sm.next;
        }
      } else {
        kmask = K == 1 ? 1ull : 0ull;
      }
      m = __popcll((unsigned long long)kmask);
    } else {
      kappa = top_p_cut_large(sm, sc, fr, K, a.p);
    }
#if ZHA_ROUTE_PROFILE
    t2 = wall_clock64();
#endif
    uint32_t mybits = 0;
    if (large) {
      // Kept flags per round of kThreads positions; ballots give ascending ranks.
      const int rounds = (K + kThreads - 1) / kThreads;
#pragma unroll
      for (int e = 0; e < kRounds; ++e) {
        if (e < rounds) {
          const int i = e * kThreads + tid;
          bool kept = false;
          if (i < K) {
            const uint64_t k = make_key(sc[i], fr[i]);
            kept = k <= kappa;
            if (!kept && k < next_key) next_key = k;
          }
          const uint64_t bal = __ballot(kept);
          if (lane == 0) sm.wcnt[e * kWaves + wave] = (uint32_t)__popcll((unsigned long long)bal);
          mybits |= (kept ? 1u : 0u) << e;
        }
      }
      if (want_gap) {
        next_key = wave_allreduce_u64(next_key, OpMin());
        if (lane == 0) sm.redu[0][wave] = next_key;
      }
      __syncthreads();
      for (int x = 0; x < rounds * kWaves; ++x) m += (int)sm.wcnt[x];
      if (want_gap) {
        next_key = sm.redu[0][0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
          next_key = sm.redu[0][w] < next_key ? (uint64_t)sm.redu[0][w] : next_key;
      }
      // The histogram is free again: clear it for the next large cut (the
      // barrier that ends this level orders the clearing before that cut).
      if (tid < 256) {
        sm.hcnt[tid] = 0u;
        sm.hmass[tid] = 0ull;
      }
      if (tid == 0) sm.bl_n = 0;
    }
    if (tid == 0) {
      const int64_t o = head * L + (l - 1);
      if (stats != nullptr) {
        stats[2 * o] = K;
        stats[2 * o + 1] = m;
      }
      if (want_gap)
        gapo[o] = (next_key == ~0ull || kappa == ~0ull) ? INFINITY
                                                        : key_score(kappa) - key_score(next_key);
    }
    // 3. Next frontier: children of the kept nodes in ascending order, then the
    // orphans.
    if (l > 1) {
      const int64_t knext = (int64_t)m * C + n_orph;
      if (knext > FMAX) {
        overflow = true;
        break;
      }
      if (!large) {
        // Every wave knows the kept set; wave w writes children c = w, w + kWaves, ...
        const bool kept_small = (kmask >> lane) & 1ull;
        const int j = __popcll((unsigned long long)(kmask & lt));
        if (kept_small) {
          const int id = fr[lane];
          for (int c = wave; c < C; c += kWaves) nx[j * C + c] = id * C + c;
        }
      } else {
        uint32_t run = 0;
        const int rounds = (K + kThreads - 1) / kThreads;
#pragma unroll
        for (int e = 0; e < kRounds; ++e) {
          if (e < rounds) {
            const bool kept = (mybits >> e) & 1u;
            const uint64_t bal = __ballot(kept);
            uint32_t off = run;
            for (int w = 0; w < wave; ++w) off += sm.wcnt[e * kWaves + w];
            for (int w = 0; w < kWaves; ++w) run += sm.wcnt[e * kWaves + w];
            if (kept) {
              const int j = (int)off + __popcll((unsigned long long)(bal & lt));
              const int id = fr[e * kThreads + tid];
              for (int c = 0; c < C; ++c) nx[j * C + c] = id * C + c;
            }
          }
        }
      }
      for (int x = tid; x < n_orph; x += kThreads) nx[m * C + x] = first_orphan + x;
      // Exactly the top candidate's children: their scores are already known.
      ready = pre && m == 1 && n_orph == 0;
      if (ready)
        for (int c = tid; c < C; c += kThreads) sm.sc[c] = sm.pre[c];
      __syncthreads();
      K = (int)knext;
      cur ^= 1;
    } else {
      int32_t* out = sel + head * a.cap;
      if (!large) {
        const int j = __popcll((unsigned long long)(kmask & lt));
        if (wave == 0 && ((kmask >> lane) & 1ull) && j < a.cap) out[j] = fr[lane];
      } else {
        uint32_t run = 0;
        const int rounds = (K + kThreads - 1) / kThreads;
#pragma unroll
        for (int e = 0; e < kRounds; ++e) {
          if (e < rounds) {
            const bool kept = (mybits >> e) & 1u;
            const uint64_t bal = __ballot(kept);
            uint32_t off = run;
            for (int w = 0; w < wave; ++w) off += sm.wcnt[e * kWaves + w];
            for (int w = 0; w < kWaves; ++w) run += sm.wcnt[e * kWaves + w];
            if (kept) {
              const int j = (int)off + __popcll((unsigned long long)(bal & lt));
              if (j < a.cap) out[j] = fr[e * kThreads + tid];
            }
          }
        }
      }
      m1 = m;
    }
#if ZHA_ROUTE_PROFILE
    // Profiling build: (score, cut) ticks in level_stats, compaction ticks in gap.
    __syncthreads();
    if (tid == 0) {
      const uint64_t t3 = wall_clock64();
      const int64_t o = head * L + (l - 1);
      stats[2 * o] = (int32_t)(t1 - t0);
      stats[2 * o + 1] = (int32_t)(t2 - t1);
      gapo[o] = (float)(t3 - t2);
    }
#endif
  }
  if (tid == 0) cnt[head] = overflow ? -1 : m1;
}

// p >= 1 keeps every candidate at every level, so S_l is all of level l and
// S_1 is every leaf chunk 0 .. n_1 - 1 (orphans included).
__global__ __launch_bounds__(kThreads) void route_keep_all_kernel(RouteArgs a,
                                                                  int32_t* __restrict__ sel,
                                                                  int32_t* __restrict__ cnt,
                                                                  int32_t* __restrict__ stats,
                                                                  float* __restrict__ gapo) {
  const int64_t head = blockIdx.x;
  const int64_t n1 = a.lay.n[1];
  const int64_t lim = n1 < a.cap ? n1 : a.cap;
  for (int64_t j = threadIdx.x; j < lim; j += kThreads) sel[head * a.cap + j] = (int32_t)j;
  if (threadIdx.x < a.lay.L) {
    const int l = threadIdx.x + 1;
    const int64_t o = head * a.lay.L + (l - 1);
    if (stats != nullptr) {
      stats[2 * o] = (int32_t)a.lay.n[l];
      stats[2 * o + 1] = (int32_t)a.lay.n[l];
    }
    if (gapo != nullptr) gapo[o] = INFINITY;
  }
  if (threadIdx.x == 0) cnt[head] = (int32_t)n1;
}

template <typename T, int D>
int launch_route(const RouteArgs& a, const void* tree, const void* Q, int32_t* sel, int32_t* cnt,
                 int32_t* stats, float* gap, hipStream_t s) {
  const unsigned blocks = (unsigned)a.n_heads;
  const char* tr = reinterpret_cast<const char*>(tree);
  const T* q = reinterpret_cast<const T*>(Q);
  if (!(a.p < 1.0f)) {
    route_keep_all_kernel<<<blocks, kThreads, 0, s>>>(a, sel, cnt, stats, gap);
  } else if (a.lay.R == 1) {
    route_kernel<T, D, kRouteFrontierMax, true>
        <<<blocks, kThreads, 0, s>>>(tr, q, a, sel, cnt, stats, gap);
  } else {
    route_kernel<T, D, kRouteFrontierMax, false>
        <<<blocks, kThreads, 0, s>>>(tr, q, a, sel, cnt, stats, gap);
  }
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

}  // namespace

int route_dispatch(const RouteArgs& a, int dtype, int d, const void* tree, const void* Q,
                   int32_t* sel, int32_t* cnt, int32_t* stats, float* gap, hipStream_t s) {
#define ZHA_ROUTE_CASE(TT, DD) \
  if (d == DD) return launch_route<TT, DD>(a, tree, Q, sel, cnt, stats, gap, s);
  if (dtype == ZHA_BF16) {
    ZHA_ROUTE_CASE(bf16_t, 64)
    ZHA_ROUTE_CASE(bf16_t, 128)
    ZHA_ROUTE_CASE(bf16_t, 256)
  } else {
    ZHA_ROUTE_CASE(float, 64)
    ZHA_ROUTE_CASE(float, 128)
    ZHA_ROUTE_CASE(float, 256)
  }
#undef ZHA_ROUTE_CASE
  return ZHA_ERR_DIM;
}

}  // namespace zha
