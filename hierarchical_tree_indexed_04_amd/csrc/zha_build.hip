// Tree construction: leaf summaries and parent merges.
//
// Follows "Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer" §III-A (chunk log-mass F_C, tangent summaries k_hat_r, b_hat_r) and
// App. D-B2 (leaf: reference/key scores and weighted key sums, two key reads;
// parent: per reference, rescale and sum the children's weighted sums, keeping
// a maximum, a weight sum and a d-vector).
//
// Accumulation is fp64.  With a zero reference every weight is exactly 1 and
// every sum of stored keys is exact, so each stored k_hat is the correctly
// rounded mean of its span; with other references the fp64 result is within
// a few ulps of the exact summary before the single rounding to storage.
//
// Layout of the work: a node is summarised by one lane group of LPR lanes,
// lane `sub` owning the VEC dims of one 16-byte slice of every row (LPR = d /
// VEC, VEC = 8 bf16 or 4 fp32 values), so each key or child row is read with
// one 16-byte load per lane.  Sums over a node's rows run row by row in order,
// per dim; the dot products of a row are summed over the group by a fixed
// butterfly.  References are processed one at a time.
//
// A zero reference (the plain mean of the span; tested per node) takes a
// shorter path with the same result bits: every score is +0, every weight
// exp(0) = 1, Z = C, F = log C and b_hat = F, so the leaf skips the score
// pass, the dot products and the exponentials and only sums the keys.
//
// A full build summarises each complete level-2 subtree in one workgroup
// (fused_kernel): the leaves' fp64 summaries stay in LDS for the level-2
// merge, so only nodes a later merge reads get an fp64 copy in the scratch
// (level-2 nodes, and leaves and nodes past the last complete parent, which
// decode-time maintenance merges later).  The other leaves and parents, and
// every node of a decode-time update, are done by leaf_kernel and
// merge_kernel, one lane group per node, with the same per-node arithmetic,
// so an updated tree equals a fresh build bit for bit.
//
// With RoPE (§III-B, reference queries) every node is summarised at its
// references rotated to the last position of its span, and a merge first
// moves each child to the parent's reference: the child's log-mass there is
// its tangent, b_hat_c + q_P . k_hat_c / sqrt(d) (equal to the pages' F_c +
// <k_hat_c, q_P - q_c> / sqrt(d)), so the scratch keeps b_hat_c in place of F_c.
//
// Each launch summarises the nodes [lo_l, n_l) of a level: lo_l = 0 for a
// full build; during decode (§III-A, App. D-B2: a summary is written once,
// when the last token of its span arrives) lo_l = n_l at the previous length,
// so only the spans completed since are visited.  Rows are strided by the
// level's capacity nc_l, so the tree and the fp64 scratch stay in place as the
// cache grows.

#include "zha_internal.hpp"
#include "zha_wave.hpp"

namespace zha {
namespace {

// Sum over aligned groups of W lanes (W = 8 .. 64), every lane of a group
// receiving the same bits: the xor butterfly, steps W/2, ..., 2, 1.  Steps
// inside a 16-lane DPP row are lane moves instead of LDS permutes: after the
// steps above a step of o lanes, lane i's value depends only on i mod 2o, so
// rotating the row by o (o = 8, 4) or the quad permutes (o = 2, 1) bring lane i
// the value of lane i ^ o, and every addition has the butterfly's operands.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return __longlong_as_double((long long)dpp_u64<CTRL>(u, u));
}
template <int W>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
  for (int o = W / 2; o >= (W < 16 ? 1 : 16); o >>= 1) v += __shfl_xor(v, o, kWave);
  if constexpr (W >= 16) {
    v += dpp_f64<kDppRowRor8>(v);
    v += dpp_f64<kDppRowRor4>(v);
    v += dpp_f64<kDppQpXor2>(v);
    v += dpp_f64<kDppQpXor1>(v);
  }
  return v;
}

constexpr int kBuildThreads = 256;
constexpr int kRowBatch = 4;              // key rows loaded before the first is used
constexpr int kChildBatch = 4;            // fp64 child rows loaded before the first is used
constexpr int kStageBatch = 8;            // 16-byte loads in flight per thread while staging children
#ifndef ZHA_ZERO_BATCH
#define ZHA_ZERO_BATCH 4
#endif
constexpr int kZeroBatch = ZHA_ZERO_BATCH;  // key rows per batch of a zero-reference stream (two in flight)
constexpr int64_t kFusedLds = 64 * 1024;  // LDS of a fused workgroup's leaf summaries
constexpr int64_t kFusedGrid = 1024;      // persistent workgroups of fused_kernel
constexpr int kStreamMaxC = 16;           // zero references: one lane group per level-2 node up to this C

template <typename T, int D>
struct LG {
  static constexpr int VEC = Vec<T>::N;             // dims per lane
  static constexpr int LPR = D / VEC;               // lanes per node
  static constexpr int NG = kBuildThreads / LPR;    // lane groups per workgroup
};

// This lane's dims of reference row qr for a node whose span ends at position
// pos: rotated by pos * theta_j in the pairs (j, j + dims/2), or as given.
// Reference r of KV head kvh ([H_kv, R, d] rows), or null when the caller
// passed no references: every reference is then zero.
__device__ __forceinline__ const float* ref_row(const float* __restrict__ qref, int kvh, int R,
                                                int r, int D) {
  return qref != nullptr ? qref + ((int64_t)kvh * R + r) * D : nullptr;
}

template <typename T, int D, bool ROPE>
__device__ __forceinline__ void node_reference(const float* __restrict__ qr, int sub,
                                               const BuildArgs& a, double pos,
                                               double (&q)[LG<T, D>::VEC]) {
  constexpr int VEC = LG<T, D>::VEC;
  const int dims = a.rope_dims, h = dims >> 1;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int k = sub * VEC + e;
    double x = qr != nullptr ? (double)qr[k] : 0.0;
    if (ROPE && k < dims) {
      const int j = k < h ? k : k - h;
      const double y = qr != nullptr ? (double)qr[k < h ? k + h : k - h] : 0.0;
      double sn, cs;
      sincos(pos * a.theta[j], &sn, &cs);
      x = k < h ? x * cs - y * sn : y * sn + x * cs;
    }
    q[e] = x;
  }
}

// True when the reference slice of some lane of this lane group is nonzero
// (uniform over the group).
template <int LPR, int VEC>
__device__ __forceinline__ bool group_nonzero(const double (&q)[VEC]) {
  bool nz = false;
#pragma unroll
  for (int e = 0; e < VEC; ++e) nz |= q[e] != 0.0;
  const uint64_t bal = __ballot(nz);
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t gm = (LPR == kWave) ? ~0ull : (((1ull << LPR) - 1) << (lane & ~(LPR - 1)));
  return (bal & gm) != 0;
}

template <typename T, int VEC>
__device__ __forceinline__ void widen_f64(const uint4& raw, double (&k)[VEC]) {
  float f[VEC];
  Vec<T>::widen(raw, f);
#pragma unroll
  for (int e = 0; e < VEC; ++e) k[e] = (double)f[e];
}

// Summary of one leaf chunk (C key rows from `keys`, consecutive rows of d
// elements) at one reference q (this lane's slice).  Returns F (or the fp64
// b_hat with ROPE, what a merge reads), writes this lane's slice of the fp64
// k_hat to acc and b_hat to b.
template <typename T, int D>
__device__ __forceinline__ double leaf_node(const T* __restrict__ keys, int C, int sub,
                                            const double (&q)[LG<T, D>::VEC], bool qnz,
                                            double (&acc)[LG<T, D>::VEC], double& b) {
  constexpr int VEC = LG<T, D>::VEC, LPR = LG<T, D>::LPR;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  const T* base = keys + sub * VEC;
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  if (!qnz) {
    // Zero reference: weights are exactly 1; only the key sums remain.
    for (int j0 = 0; j0 < C; j0 += kRowBatch) {
      uint4 raw[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u)
        raw[u] = ld16(base + (int64_t)min(j0 + u, C - 1) * D);
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        if (j0 + u >= C) break;
        double k[VEC];
        widen_f64<T, VEC>(raw[u], k);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += k[e];
      }
    }
    const double Z = (double)C;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = acc[e] / Z;
    const double F = 0.0 + log(Z);
    b = F;
    return F;
  }
  // First key read: the maximum score of the chunk.
  double m = -INFINITY;
  for (int j0 = 0; j0 < C; j0 += kRowBatch) {
    uint4 raw[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) raw[u] = ld16c(base + (int64_t)min(j0 + u, C - 1) * D);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      if (j0 + u >= C) break;
      double k[VEC];
      widen_f64<T, VEC>(raw[u], k);
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) part = fma(q[e], k[e], part);
      m = fmax(m, group_sum_f64<LPR>(part) * inv_sqrt_d);
    }
  }
  // Second key read: weights exp(s - m), their sum and the weighted key sum.
  double Z = 0.0;
  for (int j0 = 0; j0 < C; j0 += kRowBatch) {
    uint4 raw[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) raw[u] = ld16(base + (int64_t)min(j0 + u, C - 1) * D);
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      if (j0 + u >= C) break;
      double k[VEC];
      widen_f64<T, VEC>(raw[u], k);
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) part = fma(q[e], k[e], part);
      const double w = exp(group_sum_f64<LPR>(part) * inv_sqrt_d - m);
      Z += w;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fma(w, k[e], acc[e]);
    }
  }
  const double F = m + log(Z);
  double part = 0.0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc[e] = acc[e] / Z;
    part = fma(q[e], acc[e], part);
  }
  b = F - group_sum_f64<LPR>(part) * inv_sqrt_d;
  return F;
}

// Parent summary from C children at the parent's reference qp (this lane's
// slice).  childF(c) is child c's F (its fp64 b_hat with ROPE), childK(c, k)
// loads this lane's slice of its fp64 k_hat.  Returns F (b_hat with ROPE) and
// writes acc and b as leaf_node.  Children are taken in order.
template <typename T, int D, bool ROPE, typename ChildF, typename ChildK>
__device__ __forceinline__ double merge_node(int C, const double (&qp)[LG<T, D>::VEC],
                                             ChildF childF, ChildK childK,
                                             double (&acc)[LG<T, D>::VEC], double& b) {
  constexpr int VEC = LG<T, D>::VEC, LPR = LG<T, D>::LPR;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  // A child's log-mass at the parent's reference.
  auto f_of = [&](int c, const double (&kc)[VEC]) {
    double f = childF(c);
    if constexpr (ROPE) {
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) part = fma(qp[e], kc[e], part);
      f += group_sum_f64<LPR>(part) * inv_sqrt_d;
    }
    return f;
  };
  double m = -INFINITY;
  for (int c = 0; c < C; ++c) {
    double kc[VEC];
    if constexpr (ROPE) childK(c, kc);
    m = fmax(m, f_of(c, kc));
  }
  double Z = 0.0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  for (int c0 = 0; c0 < C; c0 += kChildBatch) {
    double kc[kChildBatch][VEC];
#pragma unroll
    for (int u = 0; u < kChildBatch; ++u) childK(min(c0 + u, C - 1), kc[u]);
#pragma unroll
    for (int u = 0; u < kChildBatch; ++u) {
      if (c0 + u >= C) break;
      const double w = exp(f_of(c0 + u, kc[u]) - m);
      Z += w;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = fma(w, kc[u][e], acc[e]);
    }
  }
  const double F = m + log(Z);
  double part = 0.0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc[e] = acc[e] / Z;
    part = fma(qp[e], acc[e], part);
  }
  b = F - group_sum_f64<LPR>(part) * inv_sqrt_d;
  return ROPE ? b : F;
}

// Stored copy of this lane's slice: k_hat rounded once to the storage dtype.
template <typename T, int VEC>
__device__ __forceinline__ void store_khat(T* row, int sub, const double (&acc)[VEC]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[VEC / 2];
#pragma unroll
    for (int e = 0; e < VEC / 2; ++e)
      w[e] = (uint32_t)f64_to_bf16(acc[2 * e]) | ((uint32_t)f64_to_bf16(acc[2 * e + 1]) << 16);
    *reinterpret_cast<uint4*>(row + sub * VEC) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<float4*>(row + sub * VEC) =
        make_float4((float)acc[0], (float)acc[1], (float)acc[2], (float)acc[3]);
  }
}

template <int VEC>
__device__ __forceinline__ void load_f64_slice(const double* p, double (&k)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC; e += 2) {
    const double2 v = *reinterpret_cast<const double2*>(p + e);
    k[e] = v.x;
    k[e + 1] = v.y;
  }
}
template <int VEC>
__device__ __forceinline__ void store_f64_slice(double* p, const double (&k)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC; e += 2) *reinterpret_cast<double2*>(p + e) = make_double2(k[e], k[e + 1]);
}

// The first key row of leaf chunk i of tree tr (chunks are C consecutive rows
// in both layouts; chunked pages hold C key rows, then C value rows).
template <typename T, int D>
__device__ __forceinline__ const T* chunk_keys(const T* K, const BuildArgs& a, int64_t tr,
                                               int64_t i) {
  return K + tr * kv_block_elems(a.Tc, a.lay.C, D, a.chunked) +
         i * (int64_t)a.lay.C * (a.chunked ? 2 : 1) * D;
}

// Leaves [lo, hi) of every tree, one lane group per (leaf, reference): the R
// references of a leaf are independent summaries, so they run side by side in
// adjacent lane groups (sharing the leaf's keys in cache).  sF/sK: fp64 copies
// for later merges (NULL when the tree has one level).
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kBuildThreads) void leaf_kernel(const T* __restrict__ K,
                                                             const float* __restrict__ qref,
                                                             char* __restrict__ tree,
                                                             double* __restrict__ sF,
                                                             double* __restrict__ sK, BuildArgs a,
                                                             int64_t lo, int64_t hi) {
  using G = LG<T, D>;
  const int sub = threadIdx.x % G::LPR;
  const int C = a.lay.C, R = a.lay.R;
  const int64_t item = (int64_t)blockIdx.x * G::NG + threadIdx.x / G::LPR;
  const int64_t nn = hi - lo;
  // Lane groups past the end still take part in the group reductions' lanes
  // of their own group only, so they can simply leave.
  if (item >= (int64_t)a.n_trees * nn * R) return;
  const int64_t node = item / R;
  const int r = (int)(item - node * R);
  const int64_t tr = node / nn;
  const int64_t i = lo + (node - tr * nn);
  const int kvh = (int)(tr % a.H_kv);
  const T* keys = chunk_keys<T, D>(K, a, tr, i);
  T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[1]);
  float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[1]);
  const double pos = (double)((i + 1) * C - 1);  // the chunk's last position
  {
    double q[G::VEC], acc[G::VEC], b;
    node_reference<T, D, ROPE>(ref_row(qref, kvh, R, r, D), sub, a, pos, q);
    const bool qnz = group_nonzero<G::LPR, G::VEC>(q);
    const double f = leaf_node<T, D>(keys, C, sub, q, qnz, acc, b);
    const int64_t row = i * R + r;
    store_khat<T, G::VEC>(khat + row * D, sub, acc);
    if (sub == 0) bhat[row] = (float)b;
    if (sF != nullptr) {
      const int64_t srow = tr * a.lay.ncap[1] * R + row;
      store_f64_slice<G::VEC>(sK + srow * D + sub * G::VEC, acc);
      if (sub == 0) sF[srow] = ROPE ? b : f;
    }
  }
}

// Parents [lo_level, n_level) of every tree from their children's fp64
// copies, one lane group per (parent, reference), as leaf_kernel.
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kBuildThreads) void merge_kernel(const float* __restrict__ qref,
                                                              char* __restrict__ tree,
                                                              const double* __restrict__ cF,
                                                              const double* __restrict__ cK,
                                                              double* __restrict__ pF,
                                                              double* __restrict__ pK,
                                                              BuildArgs a, int level) {
  using G = LG<T, D>;
  const int sub = threadIdx.x % G::LPR;
  const int C = a.lay.C, R = a.lay.R;
  const int64_t lo = a.lo[level];
  const int64_t nn = a.lay.n[level] - lo;  // nodes to merge per tree
  const int64_t item = (int64_t)blockIdx.x * G::NG + threadIdx.x / G::LPR;
  if (item >= (int64_t)a.n_trees * nn * R) return;
  const int64_t node = item / R;
  const int r = (int)(item - node * R);
  const int64_t tr = node / nn;
  const int64_t i = lo + (node - tr * nn);
  const int kvh = (int)(tr % a.H_kv);
  T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[level]);
  float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[level]);
  const int64_t child0 = tr * a.lay.ncap[level - 1] + i * C;  // first child's scratch row
  double span = 1.0;
  for (int l = 0; l < level; ++l) span *= C;
  const double pos = (double)(i + 1) * span - 1.0;  // the node's last position
  {
    double qp[G::VEC], acc[G::VEC], b;
    node_reference<T, D, ROPE>(ref_row(qref, kvh, R, r, D), sub, a, pos, qp);
    const double f = merge_node<T, D, ROPE>(
        C, qp, [&](int c) { return cF[(child0 + c) * R + r]; },
        [&](int c, double (&k)[G::VEC]) {
          load_f64_slice<G::VEC>(cK + ((child0 + c) * R + r) * D + sub * G::VEC, k);
        },
        acc, b);
    const int64_t row = i * R + r;
    store_khat<T, G::VEC>(khat + row * D, sub, acc);
    if (sub == 0) bhat[row] = (float)b;
    if (pF != nullptr) {
      const int64_t prow = (tr * a.lay.ncap[level] + i) * R + r;
      store_f64_slice<G::VEC>(pK + prow * D + sub * G::VEC, acc);
      if (sub == 0) pF[prow] = f;
    }
  }
}

__host__ __device__ inline int fused_f_slots(int n) { return (n + 1) & ~1; }

// Workgroup-uniform: does any of KV head kvh's R references have a nonzero
// entry?  (A rotation keeps a zero reference zero.)
__device__ __forceinline__ bool kv_head_has_nonzero_reference(const float* __restrict__ qref,
                                                              const BuildArgs& a, int kvh) {
  if (qref == nullptr) return false;  // no references given: all zero (uniform)
  const int n = a.lay.R * a.d;
  const float* q = qref + (int64_t)kvh * n;
  bool nz = false;
  for (int x = threadIdx.x; x < n; x += kBuildThreads) nz |= q[x] != 0.0f;
  return __syncthreads_or(nz) != 0;
}

// Parents [lo_level, n_level) of every tree, one workgroup each, when a
// parent's children fit the LDS (C R fp64 F, C R d fp64 k_hat): the children's
// rows are contiguous in the scratch and are staged into LDS with every load
// in flight at once, then one lane group per reference merges them with
// merge_node (children in order, the bits of merge_kernel).  One memory round
// trip per parent instead of one per kChildBatch children: the small top
// levels of a tree are latency chains otherwise.
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kBuildThreads) void merge_staged_kernel(
    const float* __restrict__ qref, char* __restrict__ tree, const double* __restrict__ cF,
    const double* __restrict__ cK, double* __restrict__ pF, double* __restrict__ pK,
    BuildArgs a, int level, bool skip_zero) {
  using G = LG<T, D>;
  extern __shared__ double lds[];  // [C R] F (padded to even), then [C R, D] k_hat
  const int sub = threadIdx.x % G::LPR, grp = threadIdx.x / G::LPR;
  const int C = a.lay.C, R = a.lay.R;
  const int64_t lo = a.lo[level];
  const int64_t nn = a.lay.n[level] - lo;
  const int64_t tr = blockIdx.x / nn;
  const int64_t i = lo + (blockIdx.x - tr * nn);
  const int kvh = (int)(tr % a.H_kv);
  // skip_zero: zero_stream3_kernel has written this level for zero references.
  if (skip_zero && !kv_head_has_nonzero_reference(qref, a, kvh)) return;
  const int64_t child0 = tr * a.lay.ncap[level - 1] + i * C;
  const int nf = C * R;
  double* lF = lds;
  double* lK = lds + fused_f_slots(nf);
  {
    // Loads first, then the LDS writes: a loop that stored each load before
    // the next would wait one memory round trip per iteration.
    const double2* src = reinterpret_cast<const double2*>(cK + child0 * R * D);
    double2* dst = reinterpret_cast<double2*>(lK);
    const int n2 = nf * D / 2;
    const int tid = threadIdx.x;
    const double f0 = cF[child0 * R + min(tid, nf - 1)];
    for (int x0 = tid; x0 < n2; x0 += kStageBatch * kBuildThreads) {
      double2 v[kStageBatch];
      // No branch: indexes past the end are clamped to the last element (its
      // own value rewritten), so no load is moved down into a conditional store.
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) v[u] = src[min(x0 + u * kBuildThreads, n2 - 1)];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) dst[min(x0 + u * kBuildThreads, n2 - 1)] = v[u];
    }
    if (tid < nf) lF[tid] = f0;
    for (int x = tid + kBuildThreads; x < nf; x += kBuildThreads) lF[x] = cF[child0 * R + x];
  }
  __syncthreads();
  T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[level]);
  float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[level]);
  double span = 1.0;
  for (int l = 0; l < level; ++l) span *= C;
  const double pos = (double)(i + 1) * span - 1.0;
  for (int r = grp; r < R; r += G::NG) {
    double qp[G::VEC], acc[G::VEC], b;
    node_reference<T, D, ROPE>(ref_row(qref, kvh, R, r, D), sub, a, pos, qp);
    const double f = merge_node<T, D, ROPE>(
        C, qp, [&](int c) { return lF[c * R + r]; },
        [&](int c, double (&k)[G::VEC]) {
          load_f64_slice<G::VEC>(lK + ((int64_t)c * R + r) * D + sub * G::VEC, k);
        },
        acc, b);
    const int64_t row = i * R + r;
    store_khat<T, G::VEC>(khat + row * D, sub, acc);
    if (sub == 0) bhat[row] = (float)b;
    if (pF != nullptr) {
      const int64_t prow = (tr * a.lay.ncap[level] + i) * R + r;
      store_f64_slice<G::VEC>(pK + prow * D + sub * G::VEC, acc);
      if (sub == 0) pF[prow] = f;
    }
  }
}

// Complete level-2 subtrees, PW parents per workgroup: the PW C leaves below
// them are summarised into LDS (fp64, all R references), then each parent is
// merged from LDS by one lane group.  Level-2 nodes get their fp64 copy in the
// scratch (pF/pK, NULL when level 2 is the top); the leaves get none.
template <typename T, int D, bool ROPE>
__device__ __forceinline__ void fused_body(const T* __restrict__ K, const float* __restrict__ qref,
                                           char* __restrict__ tree, double* __restrict__ pF,
                                           double* __restrict__ pK, const BuildArgs& a, int PW,
                                           int RB, double* lds, int64_t item) {
  using G = LG<T, D>;
  // lds: [LW * RB] fp64 F (padded to an even count, so the k_hat rows stay
  // 16-byte aligned), then [LW * RB, D] fp64 k_hat; LW = PW C leaves.  The R
  // references go through in blocks of RB (all of them when they fit); within
  // a block the lane groups take (leaf, reference) pairs, then (parent,
  // reference) pairs: independent summaries, the same per-node arithmetic.
  const int sub = threadIdx.x % G::LPR, grp = threadIdx.x / G::LPR;
  const int C = a.lay.C, R = a.lay.R;
  const int64_t n2 = a.lay.n[2];
  const int64_t wpt = (n2 + PW - 1) / PW;  // workgroups per tree
  const int64_t tr = item / wpt;
  const int64_t p0 = (item - tr * wpt) * PW;
  const int np = (int)min((int64_t)PW, n2 - p0);  // parents of this workgroup
  const int nl = np * C;                          // leaves of this workgroup
  const int kvh = (int)(tr % a.H_kv);
  double* lF = lds;
  double* lK = lds + fused_f_slots(PW * C * RB);
  T* khat1 = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[1]);
  float* bhat1 = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[1]);
  T* khat2 = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[2]);
  float* bhat2 = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[2]);
  const double span = (double)C * (double)C;
  for (int r0 = 0; r0 < R; r0 += RB) {
    const int nr = min(RB, R - r0);
    for (int w = grp; w < nl * nr; w += G::NG) {
      const int x = w / nr, rr = w - x * nr, r = r0 + rr;
      const int64_t i = p0 * C + x;
      const T* keys = chunk_keys<T, D>(K, a, tr, i);
      const double pos = (double)((i + 1) * C - 1);
      double q[G::VEC], acc[G::VEC], b;
      node_reference<T, D, ROPE>(ref_row(qref, kvh, R, r, D), sub, a, pos, q);
      const bool qnz = group_nonzero<G::LPR, G::VEC>(q);
      const double f = leaf_node<T, D>(keys, C, sub, q, qnz, acc, b);
      const int64_t row = i * R + r;
      store_khat<T, G::VEC>(khat1 + row * D, sub, acc);
      if (sub == 0) {
        bhat1[row] = (float)b;
        lF[x * RB + rr] = ROPE ? b : f;
      }
      store_f64_slice<G::VEC>(lK + ((int64_t)x * RB + rr) * D + sub * G::VEC, acc);
    }
    __syncthreads();
    for (int w = grp; w < np * nr; w += G::NG) {
      const int y = w / nr, rr = w - y * nr, r = r0 + rr;
      const int64_t i = p0 + y;
      const double pos = (double)(i + 1) * span - 1.0;
      double qp[G::VEC], acc[G::VEC], b;
      node_reference<T, D, ROPE>(ref_row(qref, kvh, R, r, D), sub, a, pos, qp);
      const double f = merge_node<T, D, ROPE>(
          C, qp, [&](int c) { return lF[(y * C + c) * RB + rr]; },
          [&](int c, double (&k)[G::VEC]) {
            load_f64_slice<G::VEC>(lK + ((int64_t)(y * C + c) * RB + rr) * D + sub * G::VEC, k);
          },
          acc, b);
      const int64_t row = i * R + r;
      store_khat<T, G::VEC>(khat2 + row * D, sub, acc);
      if (sub == 0) bhat2[row] = (float)b;
      if (pF != nullptr) {
        const int64_t prow = (tr * a.lay.ncap[2] + i) * R + r;
        store_f64_slice<G::VEC>(pK + prow * D + sub * G::VEC, acc);
        if (sub == 0) pF[prow] = f;
      }
    }
    if (r0 + RB < R) __syncthreads();  // lds is reused by the next block of references
  }
}

// Parents per fused workgroup: at least C leaves, about 32 where C is
// smaller, within the LDS budget; 0 when one parent's leaves do not fit.
// Zero references, complete level-2 subtrees (the common case: R = 1, a zero
// reference, every node the mean of its span).  As fused_body, for KV heads
// whose R references are all zero: every leaf
// then has F = log C and b_hat = F, and all references give the same summary,
// which is computed once and stored for each.  Each lane group streams its
// leaves' key rows kZeroBatch at a time with the next batch's loads issued
// before the current batch is summed; a finished leaf's fp64 k_hat goes to
// LDS (one row) for the level-2 merge.  The arithmetic is leaf_node's and
// merge_node's with a zero reference, so the bits are theirs.
template <typename T, int D>
__device__ __forceinline__ void zero_fused_body(const T* __restrict__ K, char* __restrict__ tree,
                                                double* __restrict__ pF, double* __restrict__ pK,
                                                const BuildArgs& a, int PW, double* lds,
                                                int64_t item) {
  using G = LG<T, D>;
  constexpr int VEC = G::VEC, NG = G::NG;
  // lds: [PW C, D] fp64 k_hat of the leaves
  const int sub = threadIdx.x % G::LPR, grp = threadIdx.x / G::LPR;
  const int C = a.lay.C, R = a.lay.R;
  const int64_t n2 = a.lay.n[2];
  const int64_t wpt = (n2 + PW - 1) / PW;
  const int64_t tr = item / wpt;
  const int64_t p0 = (item - tr * wpt) * PW;
  const int np = (int)min((int64_t)PW, n2 - p0);
  const int nl = np * C;
  const double Fleaf = 0.0 + log((double)C);  // leaf_node's F with a zero reference
  {
    T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[1]);
    float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[1]);
    const int mine = grp < nl ? (nl - grp + NG - 1) / NG : 0;  // leaves grp, grp + NG, ...
    int lt = 0, lj = 0;  // load cursor: leaf (of this group) and row
    int ct = 0, cj = 0;  // sum cursor
    double acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
    // Row lj of this group's leaf lt: kbase + (grp + NG lt) cstride + lj D.
    const T* kbase = chunk_keys<T, D>(K, a, tr, p0 * C) + sub * VEC;
    const int64_t cstride = (int64_t)C * (a.chunked ? 2 : 1) * D;
    auto load_batch = [&](uint4 (&buf)[kZeroBatch]) {
#pragma unroll
      for (int u = 0; u < kZeroBatch; ++u) {
        if (lt < mine)
          buf[u] = ld16(kbase + (grp + (int64_t)NG * lt) * cstride + (int64_t)lj * D);
        if (++lj == C) {
          lj = 0;
          ++lt;
        }
      }
    };
    auto sum_batch = [&](const uint4 (&buf)[kZeroBatch]) {
#pragma unroll
      for (int u = 0; u < kZeroBatch; ++u) {
        if (ct < mine) {
          double k[VEC];
          widen_f64<T, VEC>(buf[u], k);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] += k[e];
          if (++cj == C) {  // leaf done
            const int x = grp + NG * ct;
            const int64_t i = p0 * C + x;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = acc[e] / (double)C;
            for (int r = 0; r < R; ++r) {
              store_khat<T, VEC>(khat + (i * R + r) * D, sub, acc);
              if (sub == 0) bhat[i * R + r] = (float)Fleaf;
            }
            store_f64_slice<VEC>(lds + (int64_t)x * D + sub * VEC, acc);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
            cj = 0;
            ++ct;
          }
        }
      }
    };
    uint4 bufA[kZeroBatch], bufB[kZeroBatch];
    load_batch(bufA);
    while (ct < mine) {
      load_batch(bufB);
      sum_batch(bufA);
      if (ct >= mine) break;
      load_batch(bufA);
      sum_batch(bufB);
    }
  }
  __syncthreads();
  T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[2]);
  float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[2]);
  double qz[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) qz[e] = 0.0;
  for (int y = grp; y < np; y += NG) {
    const int64_t i = p0 + y;
    double acc[VEC], b;
    const double f = merge_node<T, D, false>(
        C, qz, [&](int) { return Fleaf; },
        [&](int c, double (&k)[VEC]) {
          load_f64_slice<VEC>(lds + (int64_t)(y * C + c) * D + sub * VEC, k);
        },
        acc, b);
    for (int r = 0; r < R; ++r) {
      const int64_t row = i * R + r;
      store_khat<T, VEC>(khat + row * D, sub, acc);
      if (sub == 0) bhat[row] = (float)b;
      if (pF != nullptr) {
        const int64_t prow = (tr * a.lay.ncap[2] + i) * R + r;
        store_f64_slice<VEC>(pK + prow * D + sub * VEC, acc);
        if (sub == 0) pF[prow] = f;
      }
    }
  }
}

// Complete level-2 subtrees with zero references, PW parents per workgroup
// (one workgroup per item); a workgroup whose KV head has a nonzero reference
// leaves it to fused_kernel.
template <typename T, int D>
__global__ __launch_bounds__(kBuildThreads) __attribute__((amdgpu_waves_per_eu(4)))
void zero_fused_kernel(const T* __restrict__ K,
                                                                   const float* __restrict__ qref,
                                                                   char* __restrict__ tree,
                                                                   double* __restrict__ pF,
                                                                   double* __restrict__ pK,
                                                                   BuildArgs a, int PW) {
  extern __shared__ double lds[];
  const int64_t wpt = (a.lay.n[2] + PW - 1) / PW;
  const int kvh = (int)((blockIdx.x / wpt) % a.H_kv);
  if (kv_head_has_nonzero_reference(qref, a, kvh)) return;
  zero_fused_body<T, D>(K, tree, pF, pK, a, PW, lds, blockIdx.x);
}

// True when some lane of this lane group sees a nonzero value among the R
// references of KV head kvh (uniform over the group; no barrier).
template <typename T, int D>
__device__ __forceinline__ bool group_has_nonzero_reference(const float* __restrict__ qref,
                                                            int R, int kvh, int sub) {
  using G = LG<T, D>;
  if (qref == nullptr) return false;  // no references given: all zero
  bool nz = false;
  const float* q = qref + (int64_t)kvh * R * D;
  for (int x = sub; x < R * D; x += G::LPR) nz |= q[x] != 0.0f;
  const uint64_t bal = __ballot(nz);
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t gm = (G::LPR == kWave) ? ~0ull
                                        : (((1ull << G::LPR) - 1) << (lane & ~(G::LPR - 1)));
  return (bal & gm) != 0;
}

// Zero references and small chunks (C <= kStreamMaxC): one lane group streams
// the C C key rows below level-2 node p of tree tr (kZeroBatch rows at a time,
// the next batch in flight while one is summed), writes each leaf when its C
// rows are in, and adds the leaf's fp64 k_hat into the parent's sum in child
// order, which is merge_node's sum with every weight 1; then writes the
// level-2 node.  Returns its F, its fp64 k_hat slice in pacc.
template <typename T, int D>
__device__ __forceinline__ double zero_stream_node(const T* __restrict__ K, char* __restrict__ tree,
                                                   const BuildArgs& a, int64_t tr, int64_t p,
                                                   int sub, double (&pacc)[LG<T, D>::VEC]) {
  constexpr int VEC = LG<T, D>::VEC;
  const int C = a.lay.C, R = a.lay.R;
  const double Fleaf = 0.0 + log((double)C);
  T* khat1 = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[1]);
  float* bhat1 = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[1]);
  const T* kbase = chunk_keys<T, D>(K, a, tr, p * C) + sub * VEC;
  const int64_t cstride = (int64_t)C * (a.chunked ? 2 : 1) * D;
  // Load cursor: leaf lc, row lj (pointer lp); sum cursor: leaf cc, row cj.
  int lc = 0, lj = 0, cc = 0, cj = 0;
  const T* lp = kbase;
  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = pacc[e] = 0.0;
  auto load_batch = [&](uint4 (&buf)[kZeroBatch]) {
#pragma unroll
    for (int u = 0; u < kZeroBatch; ++u) {
      if (lc < C) buf[u] = ld16(lp);
      lp += D;
      if (++lj == C) {
        lj = 0;
        ++lc;
        lp = kbase + lc * cstride;
      }
    }
  };
  auto sum_batch = [&](const uint4 (&buf)[kZeroBatch]) {
#pragma unroll
    for (int u = 0; u < kZeroBatch; ++u) {
      if (cc < C) {
        double k[VEC];
        widen_f64<T, VEC>(buf[u], k);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += k[e];
        if (++cj == C) {  // leaf cc done
          cj = 0;
          const int64_t i = p * C + cc;
          ++cc;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            acc[e] = acc[e] / (double)C;
            pacc[e] = fma(1.0, acc[e], pacc[e]);
          }
          for (int r = 0; r < R; ++r) {
            store_khat<T, VEC>(khat1 + (i * R + r) * D, sub, acc);
            if (sub == 0) bhat1[i * R + r] = (float)Fleaf;
          }
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
        }
      }
    }
  };
  uint4 bufA[kZeroBatch], bufB[kZeroBatch];
  load_batch(bufA);
  while (cc < C) {
    load_batch(bufB);
    sum_batch(bufA);
    if (cc >= C) break;
    load_batch(bufA);
    sum_batch(bufB);
  }
  // The parent: merge_node with C children of equal F: m = Fleaf, every
  // weight exp(0) = 1, Z = C.
  double Z = 0.0;
  for (int c = 0; c < C; ++c) Z += exp(Fleaf - Fleaf);
  const double F = Fleaf + log(Z);
#pragma unroll
  for (int e = 0; e < VEC; ++e) pacc[e] = pacc[e] / Z;
  T* khat2 = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[2]);
  float* bhat2 = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[2]);
  for (int r = 0; r < R; ++r) {
    const int64_t row = p * R + r;
    store_khat<T, VEC>(khat2 + row * D, sub, pacc);
    if (sub == 0) bhat2[row] = (float)F;
  }
  return F;
}

// Level-2 nodes [p_lo, n_2) of every tree with zero references, one lane group
// each (zero_stream_node), each with its fp64 copy for a later merge: no LDS,
// no barrier, every lane group busy.  A lane group whose KV head has a nonzero
// reference leaves it to fused_kernel.
#ifndef ZHA_STREAM_WAVES
#define ZHA_STREAM_WAVES 1
#endif
template <typename T, int D>
__global__ __launch_bounds__(kBuildThreads) __attribute__((amdgpu_waves_per_eu(ZHA_STREAM_WAVES)))
void zero_stream_kernel(const T* __restrict__ K, const float* __restrict__ qref,
                        char* __restrict__ tree, double* __restrict__ pF,
                        double* __restrict__ pK, BuildArgs a, int64_t p_lo) {
  using G = LG<T, D>;
  constexpr int VEC = G::VEC;
  const int sub = threadIdx.x % G::LPR;
  const int R = a.lay.R;
  const int64_t np = a.lay.n[2] - p_lo;
  const int64_t node = (int64_t)blockIdx.x * G::NG + threadIdx.x / G::LPR;
  if (node >= (int64_t)a.n_trees * np) return;
  const int64_t tr = node / np;
  const int64_t p = p_lo + (node - tr * np);
  const int kvh = (int)(tr % a.H_kv);
  if (group_has_nonzero_reference<T, D>(qref, R, kvh, sub)) return;
  double pacc[VEC];
  const double F = zero_stream_node<T, D>(K, tree, a, tr, p, sub, pacc);
  if (pF != nullptr) {
    for (int r = 0; r < R; ++r) {
      const int64_t prow = (tr * a.lay.ncap[2] + p) * R + r;
      store_f64_slice<VEC>(pK + prow * D + sub * VEC, pacc);
      if (sub == 0) pF[prow] = F;
    }
  }
}

// Complete level-3 subtrees with zero references, NG / C per workgroup: lane
// group g streams child g % C of subtree g / C (zero_stream_node); the C
// level-2 k_hat meet in LDS and the subtree's first lane group merges them,
// children in order, with every weight exp(0) = 1 (merge_node's arithmetic,
// so the bits of merge_staged_kernel), writing the level-3 node and its fp64
// copy (pF3/pK3, NULL when level 3 is the top).  Level-2 nodes get no fp64
// copy: no later merge reads them.  Lane groups of a KV head with a nonzero
// reference only take part in the barrier.
template <typename T, int D>
__global__ __launch_bounds__(kBuildThreads) __attribute__((amdgpu_waves_per_eu(ZHA_STREAM_WAVES)))
void zero_stream3_kernel(const T* __restrict__ K, const float* __restrict__ qref,
                         char* __restrict__ tree, double* __restrict__ pF3,
                         double* __restrict__ pK3, BuildArgs a) {
  using G = LG<T, D>;
  constexpr int VEC = G::VEC;
  __shared__ __align__(16) double s_k2[G::NG][D];
  const int sub = threadIdx.x % G::LPR, grp = threadIdx.x / G::LPR;
  const int C = a.lay.C, R = a.lay.R;
  const int P3 = G::NG / C;  // subtrees per workgroup (the host keeps C <= NG)
  const int64_t n3 = a.lay.n[3];
  const int64_t s3 = (int64_t)blockIdx.x * P3 + grp / C;
  bool mine = grp < P3 * C && s3 < (int64_t)a.n_trees * n3;
  const int64_t tr = mine ? s3 / n3 : 0;
  const int64_t i3 = s3 - tr * n3;
  if (mine) mine = !group_has_nonzero_reference<T, D>(qref, R, (int)(tr % a.H_kv), sub);
  double F2 = 0.0;
  if (mine) {
    double pacc[VEC];
    F2 = zero_stream_node<T, D>(K, tree, a, tr, i3 * C + grp % C, sub, pacc);
    store_f64_slice<VEC>(&s_k2[grp][sub * VEC], pacc);
  }
  __syncthreads();
  if (!mine || grp % C != 0) return;
  // merge_node at a zero reference: children of equal F2, m = F2, w = 1.
  double m = -INFINITY;
  for (int c = 0; c < C; ++c) m = fmax(m, F2);
  double Z = 0.0, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
  for (int c = 0; c < C; ++c) {
    double kc[VEC];
    load_f64_slice<VEC>(&s_k2[grp + c][sub * VEC], kc);
    const double w = exp(F2 - m);
    Z += w;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = fma(w, kc[e], acc[e]);
  }
  const double F = m + log(Z);
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = acc[e] / Z;
  T* khat3 = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[3]);
  float* bhat3 = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[3]);
  for (int r = 0; r < R; ++r) {
    const int64_t row = i3 * R + r;
    store_khat<T, VEC>(khat3 + row * D, sub, acc);
    if (sub == 0) bhat3[row] = (float)F;
    if (pF3 != nullptr) {
      const int64_t prow = (tr * a.lay.ncap[3] + i3) * R + r;
      store_f64_slice<VEC>(pK3 + prow * D + sub * VEC, acc);
      if (sub == 0) pF3[prow] = F;
    }
  }
}

// The same items for KV heads with a nonzero reference, on a persistent grid:
// each workgroup first marks which KV heads have one (a 64-bit mask when H_kv
// <= 64, else a check per item), then takes items blockIdx.x, + gridDim.x, ...
// and skips the others, so a build with zero references costs one short launch.
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kBuildThreads) void fused_kernel(const T* __restrict__ K,
                                                              const float* __restrict__ qref,
                                                              char* __restrict__ tree,
                                                              double* __restrict__ pF,
                                                              double* __restrict__ pK,
                                                              BuildArgs a, int PW, int RB) {
  extern __shared__ double lds[];
  const int64_t wpt = (a.lay.n[2] + PW - 1) / PW;
  const int64_t items = (int64_t)a.n_trees * wpt;
  uint64_t mask = 0;
  const bool small = a.H_kv <= 64;
  if (small)
    for (int h = 0; h < a.H_kv; ++h)
      if (kv_head_has_nonzero_reference(qref, a, h)) mask |= 1ull << h;
  if (small && mask == 0) return;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int kvh = (int)((it / wpt) % a.H_kv);
    const bool nz = small ? ((mask >> kvh) & 1ull) != 0 : kv_head_has_nonzero_reference(qref, a, kvh);
    if (!nz) continue;
    fused_body<T, D, ROPE>(K, qref, tree, pF, pK, a, PW, RB, lds, it);
    __syncthreads();  // lds is reused by the next item
  }
}

inline int64_t fused_lds_bytes(int pw, int C, int R, int D) {
  return ((int64_t)fused_f_slots(pw * C * R) + (int64_t)pw * C * R * D) * 8;
}
template <int D>
int fused_parents(int C, int R) {
  int pw = C >= 32 ? 1 : 32 / C;
  while (pw > 1 && fused_lds_bytes(pw, C, R, D) > kFusedLds) pw >>= 1;
  return fused_lds_bytes(pw, C, R, D) <= kFusedLds ? pw : 0;
}


template <typename T, int D, bool ROPE>
int launch_build_impl(const BuildArgs& a, const void* K, const float* qref, void* tree,
                      void* scratch, hipStream_t s) {
  using G = LG<T, D>;
  const BuildScratch sc = build_scratch_layout(a);
  char* base = reinterpret_cast<char*>(scratch);
  auto F = [&](int l) { return reinterpret_cast<double*>(base + sc.F[l]); };
  auto Kp = [&](int l) { return reinterpret_cast<double*>(base + sc.K[l]); };
  const int L = a.lay.L, C = a.lay.C, R = a.lay.R;
  const T* kp = reinterpret_cast<const T*>(K);
  char* tp = reinterpret_cast<char*>(tree);
  auto leaves = [&](int64_t lo, int64_t hi) {
    if (hi <= lo) return;
    const int64_t items = (int64_t)a.n_trees * (hi - lo) * R;  // (leaf, reference) pairs
    const unsigned blocks = (unsigned)((items + G::NG - 1) / G::NG);
    leaf_kernel<T, D, ROPE><<<blocks, kBuildThreads, 0, s>>>(
        kp, qref, tp, L > 1 ? F(1) : nullptr, L > 1 ? Kp(1) : nullptr, a, lo, hi);
  };
  // A full build takes every complete level-2 subtree in the fused kernel; the
  // leaves past them (no complete parent yet) go through leaf_kernel with
  // their fp64 copies kept for the merge that will complete them.
  // Parents per workgroup of the complete level-2 subtree launches; 0 when
  // one parent's leaves at all R references do not fit the LDS.  (Taking the
  // references in blocks instead measured slower at R = 16, 21.4 -> 28.4 ms
  // at 256K, than leaf_kernel and merge_kernel over (node, reference) pairs.)
  const bool full = L >= 2 && a.lo[1] == 0 && a.lo[2] == 0 && a.lay.n[2] > 0;
  const int PW = full ? fused_parents<D>(C, R) : 0;
  const int RB = R;
  int first_merge = 2;
  const int64_t staged_lds = ((int64_t)fused_f_slots(C * R) + (int64_t)C * R * D) * 8;
  // Zero references with small C: complete level-3 subtrees in one pass when
  // the level-3 merge of the other KV heads can stage (it skips these heads).
  const bool fold3 = PW > 0 && C <= kStreamMaxC && C <= G::NG && L >= 3 && a.lo[3] == 0 &&
                     a.lay.n[3] > 0 && staged_lds <= kFusedLds;
  if (PW > 0) {
    const int64_t wpt = (a.lay.n[2] + PW - 1) / PW;
    const size_t lds = (size_t)fused_lds_bytes(PW, C, RB, D);
    const int64_t items = a.n_trees * wpt;
    if (C <= kStreamMaxC) {
      int64_t p_lo = 0;
      if (fold3) {
        const int P3 = G::NG / C;
        const int64_t subtrees = a.n_trees * a.lay.n[3];
        zero_stream3_kernel<T, D><<<(unsigned)((subtrees + P3 - 1) / P3), kBuildThreads, 0, s>>>(
            kp, qref, tp, L > 3 ? F(3) : nullptr, L > 3 ? Kp(3) : nullptr, a);
        p_lo = a.lay.n[3] * C;  // level-2 nodes below no complete level-3 node
      }
      const int64_t groups = a.n_trees * (a.lay.n[2] - p_lo);
      if (groups > 0)
        zero_stream_kernel<T, D><<<(unsigned)((groups + G::NG - 1) / G::NG), kBuildThreads, 0, s>>>(
            kp, qref, tp, L > 2 ? F(2) : nullptr, L > 2 ? Kp(2) : nullptr, a, p_lo);
    } else {
      zero_fused_kernel<T, D><<<(unsigned)items, kBuildThreads,
                                (size_t)PW * C * D * sizeof(double), s>>>(
          kp, qref, tp, L > 2 ? F(2) : nullptr, L > 2 ? Kp(2) : nullptr, a, PW);
    }
    if (qref != nullptr)  // without references every KV head took the zero-reference kernels
      fused_kernel<T, D, ROPE><<<(unsigned)min(items, (int64_t)kFusedGrid), kBuildThreads, lds, s>>>(
          kp, qref, tp, L > 2 ? F(2) : nullptr, L > 2 ? Kp(2) : nullptr, a, PW, RB);
    leaves(a.lay.n[2] * C, a.lay.n[1]);
    first_merge = 3;
  } else {
    leaves(a.lo[1], a.lay.n[1]);
  }
  if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
  for (int l = first_merge; l <= L; ++l) {
    if (a.lay.n[l] == a.lo[l]) continue;  // no span of this level completed
    const int64_t nodes = (int64_t)a.n_trees * (a.lay.n[l] - a.lo[l]);
    if (staged_lds <= kFusedLds) {
      merge_staged_kernel<T, D, ROPE><<<(unsigned)nodes, kBuildThreads, (size_t)staged_lds, s>>>(
          qref, tp, F(l - 1), Kp(l - 1), l < L ? F(l) : nullptr, l < L ? Kp(l) : nullptr, a, l,
          fold3 && l == 3);
    } else {
      const unsigned blocks = (unsigned)((nodes * R + G::NG - 1) / G::NG);  // (parent, reference)
      merge_kernel<T, D, ROPE><<<blocks, kBuildThreads, 0, s>>>(
          qref, tp, F(l - 1), Kp(l - 1), l < L ? F(l) : nullptr, l < L ? Kp(l) : nullptr, a, l);
    }
    if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
  }
  return ZHA_OK;
}

template <typename T, int D>
int launch_build(const BuildArgs& a, const void* K, const float* qref, void* tree,
                 void* scratch, hipStream_t s) {
  if (a.rope_dims) return launch_build_impl<T, D, true>(a, K, qref, tree, scratch, s);
  return launch_build_impl<T, D, false>(a, K, qref, tree, scratch, s);
}

}  // namespace

int build_dispatch(const BuildArgs& a, int dtype, int d, const void* K, const float* qref,
                   void* tree, void* scratch, hipStream_t s) {
#define ZHA_BUILD_CASE(TT, DD)                                                      \
  if (d == DD) return launch_build<TT, DD>(a, K, qref, tree, scratch, s);
  if (dtype == ZHA_BF16) {
    ZHA_BUILD_CASE(bf16_t, 64)
    ZHA_BUILD_CASE(bf16_t, 128)
    ZHA_BUILD_CASE(bf16_t, 256)
  } else {
    ZHA_BUILD_CASE(float, 64)
    ZHA_BUILD_CASE(float, 128)
    ZHA_BUILD_CASE(float, 256)
  }
#undef ZHA_BUILD_CASE
  return ZHA_ERR_DIM;
}

}  // namespace zha
