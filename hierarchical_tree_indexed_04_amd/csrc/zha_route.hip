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
// One workgroup (4 waves) per query head walks all levels in one launch.  The
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
//   1. A 256-bucket histogram over (s_max - s) (monotone in the key) finds the
//      bucket where the running mass crosses p Z.
//   2. If that bucket holds more than 64 candidates, 8-bit radix passes over
//      the keys inside it narrow it further (ties in score fall to the id
//      bits).
//   3. One wave ranks the <= 64 boundary candidates: a candidate is kept iff
//      the mass of all keys below it is < p Z.  The largest kept key, kappa,
//      defines the cut: kept = {key <= kappa}.
// Compaction keeps ascending id order with per-wave ballots, and the next
// frontier is written as children of the kept nodes.

#include "zha_internal.hpp"

namespace zha {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = 8;  // summary rows in flight per lane while scoring
constexpr float kFix = 1099511627776.0f;  // 2^40

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const int lo = __shfl((int)(uint32_t)v, src, kWave);
  const int hi = __shfl((int)(uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m, kWave);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), m, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const int lo = __shfl_up((int)(uint32_t)v, d, kWave);
  const int hi = __shfl_up((int)(uint32_t)(v >> 32), d, kWave);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, j);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t t = shfl_xor_u64(v, o);
    v = t > v ? t : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t t = shfl_xor_u64(v, o);
    v = t < v ? t : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor_u64(v, o);
  return v;
}

__device__ __forceinline__ uint64_t make_key(float s, int32_t id) {
  return ((uint64_t)(~ord_f32(s)) << 32) | (uint32_t)id;
}
__device__ __forceinline__ float key_score(uint64_t k) {
  return unord_f32(~(uint32_t)(k >> 32));
}
__device__ __forceinline__ uint64_t fixed_mass(float s, float smax) {
  return (uint64_t)(expf(s - smax) * kFix);
}

template <int FMAX>
struct RouteSmem {
  int32_t fr[2][FMAX];         // frontier node ids, ascending (ping-pong)
  float sc[FMAX];              // scores of the current frontier
  int32_t comp[FMAX / 2];      // kept ids of a level > 1 (m * C <= FMAX, C >= 2)
  uint32_t hcnt[256];          // histogram: candidates per bucket
  unsigned long long hmass[256];  // histogram: fixed-point mass per bucket
  unsigned long long bkey[64];    // boundary candidates
  unsigned long long bw[64];
  uint32_t wcnt[FMAX / kThreads][kWaves];  // kept per (round, wave), then offsets
  unsigned long long redu[kWaves];
  float redf[2][kWaves];
  unsigned long long kappa, base, lo, hi;
  double target;
  int32_t bstar, bcount, bl_n, m;
};

// Block-wide reductions (all threads participate; result broadcast).
template <int FMAX>
__device__ __forceinline__ void block_minmax_f(RouteSmem<FMAX>& sm, float& mx, float& mn) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  mx = group_max<kWave>(mx);
  mn = -group_max<kWave>(-mn);
  if (lane == 0) {
    sm.redf[0][wave] = mx;
    sm.redf[1][wave] = mn;
  }
  __syncthreads();
  mx = fmaxf(fmaxf(sm.redf[0][0], sm.redf[0][1]), fmaxf(sm.redf[0][2], sm.redf[0][3]));
  mn = fminf(fminf(sm.redf[1][0], sm.redf[1][1]), fminf(sm.redf[1][2], sm.redf[1][3]));
  __syncthreads();
}

template <int FMAX, bool kMin>
__device__ __forceinline__ uint64_t block_ext_u64(RouteSmem<FMAX>& sm, uint64_t v) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  v = kMin ? wave_min_u64(v) : wave_max_u64(v);
  if (lane == 0) sm.redu[wave] = v;
  __syncthreads();
  uint64_t r = sm.redu[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    const uint64_t t = sm.redu[w];
    r = kMin ? (t < r ? t : r) : (t > r ? t : r);
  }
  __syncthreads();
  return r;
}

// Wave 0: scan the 256-bucket histogram from `base0`, find the first bucket
// whose inclusive running mass reaches the target.  With `first`, the total
// mass Z is the histogram's sum and the target p Z is set.
template <int FMAX>
__device__ __forceinline__ void scan_find(RouteSmem<FMAX>& sm, uint64_t base0, bool first,
                                          float p) {
  const int lane = threadIdx.x;  // wave 0 only
  uint64_t c[4];
  uint64_t run = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    run += sm.hmass[4 * lane + k];
    c[k] = run;
  }
  uint64_t incl = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint64_t t = shfl_up_u64(incl, o);
    if (lane >= o) incl += t;
  }
  const uint64_t excl = incl - run;
  double target;
  if (first) {
    const uint64_t Z = readlane_u64(incl, kWave - 1);
    target = (double)p * (double)Z;
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

// Wave 0: exact resolution of n <= 64 boundary candidates (one per lane).  A
// candidate is kept iff base + (mass of the candidates with smaller keys) < target.
template <int FMAX>
__device__ __forceinline__ void resolve_boundary(RouteSmem<FMAX>& sm, uint64_t key, uint64_t w,
                                                 int n, uint64_t base, double target) {
  const int lane = threadIdx.x;
  const bool valid = lane < n;
  uint64_t below = 0;
  for (int j = 0; j < n; ++j) {
    const uint64_t kj = readlane_u64(key, j);
    const uint64_t wj = readlane_u64(w, j);
    below += (kj < key) ? wj : 0ull;
  }
  const bool kept = valid && (double)(base + below) < target;
  const uint64_t kappa = wave_max_u64(kept ? key : 0ull);
  if (lane == 0) sm.kappa = kappa;
}

// Wave 0: resolve the candidates collected in bkey/bw (after a barrier).
template <int FMAX>
__device__ __forceinline__ void resolve_collected(RouteSmem<FMAX>& sm) {
  const int lane = threadIdx.x;
  const int n = min(sm.bl_n, kWave);
  const uint64_t key = lane < n ? sm.bkey[lane] : ~0ull;
  const uint64_t w = lane < n ? sm.bw[lane] : 0ull;
  resolve_boundary(sm, key, w, n, sm.base, sm.target);
}

// Scores of the frontier: s_i = max_r (q . k_hat_{r,i} + b_hat_{r,i}), q pre-scaled by 1/sqrt(d).
template <typename T, int D, int FMAX>
__device__ __forceinline__ void score_frontier(RouteSmem<FMAX>& sm, const int32_t* fr, int K,
                                               int R, const char* __restrict__ khat,
                                               const float* __restrict__ bhat, const float* q) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = kThreads / LPR;
  const int tid = threadIdx.x;
  const int sub = tid % LPR, grp = tid / LPR;
  uint32_t* sco = reinterpret_cast<uint32_t*>(sm.sc);
  if (R > 1) {
    for (int i = tid; i < K; i += kThreads) sco[i] = 0u;
    __syncthreads();
  }
  const int NR = K * R;
  for (int base = 0; base < NR; base += RPB * kU) {
    uint4 v[kU];
    float bias[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int x = base + u * RPB + grp;
      if (x < NR) {
        const int node = fr[R == 1 ? x : x / R];
        const int r = R == 1 ? 0 : x % R;
        const int64_t row = (int64_t)node * R + r;
        v[u] = ld16c(khat + row * (int64_t)(D * sizeof(T)) + sub * 16);
        bias[u] = bhat[row];
      } else {
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        bias[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int x = base + u * RPB + grp;
      float k[VEC];
      Vec<T>::widen(v[u], k);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dot = fmaf(q[e], k[e], dot);
      dot = group_sum<LPR>(dot);
      if (sub == 0 && x < NR) {
        const float s = dot + bias[u];
        if (R == 1)
          sm.sc[x] = s;
        else
          atomicMax(&sco[x / R], ord_f32(s));
      }
    }
  }
  if (R > 1) {
    __syncthreads();
    for (int i = tid; i < K; i += kThreads) sm.sc[i] = unord_f32(sco[i]);
  }
  __syncthreads();
}

// Finds kappa, the largest kept key, for a frontier of K > 1 candidates (p < 1).
template <int FMAX>
__device__ __forceinline__ uint64_t top_p_cut(RouteSmem<FMAX>& sm, const int32_t* fr, int K,
                                              float p) {
  const int tid = threadIdx.x, wave = tid >> 6;
  float smax = -INFINITY, smin = INFINITY;
  for (int i = tid; i < K; i += kThreads) {
    const float s = sm.sc[i];
    smax = fmaxf(smax, s);
    smin = fminf(smin, s);
  }
  block_minmax_f(sm, smax, smin);

  if (K <= kWave) {
    if (wave == 0) {
      const int lane = tid;
      const bool valid = lane < K;
      const float s = valid ? sm.sc[lane] : 0.f;
      const uint64_t key = valid ? make_key(s, fr[lane]) : ~0ull;
      const uint64_t w = valid ? fixed_mass(s, smax) : 0ull;
      const uint64_t Z = wave_sum_u64(w);
      resolve_boundary(sm, key, w, K, 0ull, (double)p * (double)Z);
    }
    __syncthreads();
    return sm.kappa;
  }

  // 1. Value-space histogram over (s_max - s).
  const float range = fminf(smax - smin, 32.f);
  const float bscale = range > 0.f ? 256.f / range : 0.f;
  auto bucket = [&](float s) { return min((int)((smax - s) * bscale), 255); };
  sm.hcnt[tid] = 0u;
  sm.hmass[tid] = 0ull;
  __syncthreads();
  for (int i = tid; i < K; i += kThreads) {
    const float s = sm.sc[i];
    const int bk = bucket(s);
    atomicAdd(&sm.hcnt[bk], 1u);
    atomicAdd(&sm.hmass[bk], (unsigned long long)fixed_mass(s, smax));
  }
  __syncthreads();
  if (wave == 0) scan_find(sm, 0ull, true, p);
  __syncthreads();
  const int bstar = sm.bstar;
  if (sm.bcount <= kWave) {
    if (tid == 0) sm.bl_n = 0;
    __syncthreads();
    for (int i = tid; i < K; i += kThreads) {
      const float s = sm.sc[i];
      if (bucket(s) == bstar) {
        const int slot = atomicAdd(&sm.bl_n, 1);
        if (slot < kWave) {
          sm.bkey[slot] = make_key(s, fr[i]);
          sm.bw[slot] = fixed_mass(s, smax);
        }
      }
    }
    __syncthreads();
    if (wave == 0) resolve_collected(sm);
    __syncthreads();
    return sm.kappa;
  }

  // 2. Radix refinement over the keys of the crowded bucket.
  uint64_t lo = ~0ull, hi = 0ull;
  for (int i = tid; i < K; i += kThreads) {
    const float s = sm.sc[i];
    if (bucket(s) == bstar) {
      const uint64_t k = make_key(s, fr[i]);
      lo = k < lo ? k : lo;
      hi = k > hi ? k : hi;
    }
  }
  lo = block_ext_u64<FMAX, true>(sm, lo);
  hi = block_ext_u64<FMAX, false>(sm, hi);
  // Keys are distinct (ids are), so every pass fixes at least 8 more bits and
  // at most 8 passes reach a single key; the bound below is defensive.
  for (int pass = 0;; ++pass) {
    const bool last_pass = pass >= 8 || lo == hi;
    const int hb = (lo == hi) ? 0 : 63 - __clzll((long long)(lo ^ hi));
    const int shift = hb > 7 ? hb - 7 : 0;
    sm.hcnt[tid] = 0u;
    sm.hmass[tid] = 0ull;
    __syncthreads();
    for (int i = tid; i < K; i += kThreads) {
      const float s = sm.sc[i];
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
      if (tid == 0) sm.bl_n = 0;
      __syncthreads();
      for (int i = tid; i < K; i += kThreads) {
        const float s = sm.sc[i];
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
      if (wave == 0) resolve_collected(sm);
      __syncthreads();
      return sm.kappa;
    }
    lo = ~0ull;
    hi = 0ull;
    for (int i = tid; i < K; i += kThreads) {
      const uint64_t k = make_key(sm.sc[i], fr[i]);
      if (k >= nlo && k <= nhi) {
        lo = k < lo ? k : lo;
        hi = k > hi ? k : hi;
      }
    }
    lo = block_ext_u64<FMAX, true>(sm, lo);
    hi = block_ext_u64<FMAX, false>(sm, hi);
  }
}

template <typename T, int D, int FMAX>
__global__ __launch_bounds__(kThreads) void route_kernel(const char* __restrict__ tree,
                                                         const T* __restrict__ Q, RouteArgs a,
                                                         int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ stats,
                                                         float* __restrict__ gapo) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  __shared__ RouteSmem<FMAX> sm;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int64_t head = blockIdx.x;
  const int h = (int)(head % a.H_q);
  const int64_t b = head / ((int64_t)a.n_pos * a.H_q);
  const int kvh = h / a.G;
  const char* tb = tree + (b * a.H_kv + kvh) * a.lay.stride;
  const int R = a.lay.R, C = a.lay.C, L = a.lay.L;

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
  __syncthreads();
  int cur = 0;
  int m1 = 0;
  for (int l = L; l >= 1 && !overflow; --l) {
    const int32_t* fr = sm.fr[cur];
    int32_t* nx = sm.fr[cur ^ 1];
    uint64_t kappa = ~0ull;
    if (K > 1) {
      score_frontier<T, D, FMAX>(sm, fr, K, R, tb + a.lay.khat[l],
                                 reinterpret_cast<const float*>(tb + a.lay.bhat[l]), q);
      kappa = top_p_cut<FMAX>(sm, fr, K, a.p);
    }
    const bool all = kappa == ~0ull;

    // Compaction: kept flags per round of 256 positions, ballots give ascending ranks.
    const int rounds = (K + kThreads - 1) / kThreads;
    uint64_t next_key = ~0ull;
    for (int e = 0; e < rounds; ++e) {
      const int i = e * kThreads + tid;
      bool kept = false;
      if (i < K) {
        const uint64_t k = all ? 0ull : make_key(sm.sc[i], fr[i]);
        kept = all || k <= kappa;
        if (!kept) next_key = k < next_key ? k : next_key;
      }
      const uint64_t bal = __ballot(kept);
      if (lane == 0) sm.wcnt[e][wave] = (uint32_t)__popcll((unsigned long long)bal);
    }
    if (!all) next_key = block_ext_u64<FMAX, true>(sm, next_key);
    else __syncthreads();
    if (tid == 0) {
      uint32_t run = 0;
      for (int e = 0; e < rounds; ++e)
        for (int w = 0; w < kWaves; ++w) {
          const uint32_t c = sm.wcnt[e][w];
          sm.wcnt[e][w] = run;
          run += c;
        }
      sm.m = (int32_t)run;
    }
    __syncthreads();
    const int m = sm.m;
    if (tid == 0) {
      const int64_t o = head * L + (l - 1);
      if (stats != nullptr) {
        stats[2 * o] = K;
        stats[2 * o + 1] = m;
      }
      if (gapo != nullptr)
        gapo[o] = (all || next_key == ~0ull) ? INFINITY : key_score(kappa) - key_score(next_key);
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (l > 1) {
      const int n_orph = (int)(a.lay.n[l - 1] - (int64_t)C * a.lay.n[l]);
      const int64_t knext = (int64_t)m * C + n_orph;
      if (knext > FMAX) {
        overflow = true;
        break;
      }
      for (int e = 0; e < rounds; ++e) {
        const int i = e * kThreads + tid;
        const bool kept = i < K && (all || make_key(sm.sc[i], fr[i]) <= kappa);
        const uint64_t bal = __ballot(kept);
        if (kept) sm.comp[sm.wcnt[e][wave] + __popcll((unsigned long long)(bal & lt))] = fr[i];
      }
      __syncthreads();
      for (int x = tid; x < m * C; x += kThreads) nx[x] = sm.comp[x / C] * C + x % C;
      const int first_orphan = (int)((int64_t)C * a.lay.n[l]);
      for (int x = tid; x < n_orph; x += kThreads) nx[m * C + x] = first_orphan + x;
      __syncthreads();
      K = (int)knext;
      cur ^= 1;
    } else {
      int32_t* out = sel + head * a.cap;
      for (int e = 0; e < rounds; ++e) {
        const int i = e * kThreads + tid;
        const bool kept = i < K && (all || make_key(sm.sc[i], fr[i]) <= kappa);
        const uint64_t bal = __ballot(kept);
        if (kept) {
          const int j = (int)sm.wcnt[e][wave] + __popcll((unsigned long long)(bal & lt));
          if (j < a.cap) out[j] = fr[i];
        }
      }
      m1 = m;
    }
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
  if (!(a.p < 1.0f)) {
    route_keep_all_kernel<<<blocks, kThreads, 0, s>>>(a, sel, cnt, stats, gap);
  } else {
    route_kernel<T, D, kRouteFrontierMax><<<blocks, kThreads, 0, s>>>(
        reinterpret_cast<const char*>(tree), reinterpret_cast<const T*>(Q), a, sel, cnt, stats,
        gap);
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
