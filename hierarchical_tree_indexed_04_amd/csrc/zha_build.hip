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
// One wave per node; lane l owns dims [l*DPL, l*DPL + DPL).  References are
// processed one at a time (the chunk's keys are re-read from cache).
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

namespace zha {

template <typename T, int D>
__device__ __forceinline__ void load_row_f64(const T* row, int lane, double* out) {
  constexpr int DPL = D / kWave;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[e] = (double)load_elem(row, lane * DPL + e);
}

// This lane's dims of reference row qr for a node whose span ends at position
// pos: rotated by pos * theta_j in the pairs (j, j + dims/2), or as given.
template <int D, bool ROPE>
__device__ __forceinline__ void node_reference(const float* __restrict__ qr, int lane,
                                               const BuildArgs& a, double pos, double* q) {
  constexpr int DPL = D / kWave;
  const int dims = a.rope_dims, h = dims >> 1;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const int k = lane * DPL + e;
    double x = (double)qr[k];
    if (ROPE && k < dims) {
      const int j = k < h ? k : k - h;
      const double y = (double)qr[k < h ? k + h : k - h];
      double sn, cs;
      sincos(pos * a.theta[j], &sn, &cs);
      x = k < h ? x * cs - y * sn : y * sn + x * cs;
    }
    q[e] = x;
  }
}

template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(256) void leaf_kernel(const T* __restrict__ K,
                                                   const float* __restrict__ qref,
                                                   char* __restrict__ tree,
                                                   double* __restrict__ sF,
                                                   double* __restrict__ sK, BuildArgs a) {
  constexpr int DPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t node = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t lo = a.lo[1];
  const int64_t nn = a.lay.n[1] - lo;  // nodes to summarise per tree
  if (node >= (int64_t)a.n_trees * nn) return;
  const int64_t tr = node / nn;
  const int64_t i = lo + (node - tr * nn);
  const int kvh = (int)(tr % a.H_kv);
  const int C = a.lay.C;
  const int R = a.lay.R;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  // Chunk i's C keys are consecutive rows in both layouts; only the chunk's
  // first row differs (chunked: each page holds C key rows, then C value rows).
  const T* keys = K + tr * kv_block_elems(a.Tc, C, D, a.chunked) +
                  i * (int64_t)C * (a.chunked ? 2 : 1) * D;
  T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[1]);
  float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[1]);

  const double pos = (double)((i + 1) * C - 1);  // the chunk's last position
  for (int r = 0; r < R; ++r) {
    double q[DPL];
    node_reference<D, ROPE>(qref + ((int64_t)kvh * R + r) * D, lane, a, pos, q);
    // Rows are read kB at a time, every load of a batch issued before the
    // first is used (one memory latency per batch, not per row); the
    // arithmetic runs row by row in order.
    constexpr int kB = 8;
    // First key read: the maximum score of the chunk.
    double m = -INFINITY;
    for (int j0 = 0; j0 < C; j0 += kB) {
      double k[kB][DPL];
#pragma unroll
      for (int u = 0; u < kB; ++u) load_row_f64<T, D>(keys + (int64_t)min(j0 + u, C - 1) * D, lane, k[u]);
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (j0 + u >= C) break;
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) part = fma(q[e], k[u][e], part);
        m = fmax(m, group_sum64<kWave>(part) * inv_sqrt_d);
      }
    }
    // Second key read: weights exp(s - m), their sum and the weighted key sum.
    double Z = 0.0;
    double acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
    for (int j0 = 0; j0 < C; j0 += kB) {
      double k[kB][DPL];
#pragma unroll
      for (int u = 0; u < kB; ++u) load_row_f64<T, D>(keys + (int64_t)min(j0 + u, C - 1) * D, lane, k[u]);
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (j0 + u >= C) break;
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) part = fma(q[e], k[u][e], part);
        const double w = exp(group_sum64<kWave>(part) * inv_sqrt_d - m);
        Z += w;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fma(w, k[u][e], acc[e]);
      }
    }
    const double F = m + log(Z);
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      acc[e] = acc[e] / Z;
      part = fma(q[e], acc[e], part);
    }
    const double b = F - group_sum64<kWave>(part) * inv_sqrt_d;
    const int64_t row = i * R + r;
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem64(khat, row * D + lane * DPL + e, acc[e]);
    if (lane == 0) bhat[row] = (float)b;
    if (sF != nullptr) {
      const int64_t srow = tr * a.lay.ncap[1] * R + row;
#pragma unroll
      for (int e = 0; e < DPL; ++e) sK[srow * D + lane * DPL + e] = acc[e];
      if (lane == 0) sF[srow] = ROPE ? b : F;
    }
  }
}

template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ qref,
                                                    char* __restrict__ tree,
                                                    const double* __restrict__ cF,
                                                    const double* __restrict__ cK,
                                                    double* __restrict__ pF,
                                                    double* __restrict__ pK, BuildArgs a,
                                                    int level) {
  constexpr int DPL = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t lo = a.lo[level];
  const int64_t nn = a.lay.n[level] - lo;  // nodes to merge per tree
  const int64_t node = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (node >= (int64_t)a.n_trees * nn) return;
  const int64_t tr = node / nn;
  const int64_t i = lo + (node - tr * nn);
  const int kvh = (int)(tr % a.H_kv);
  const int C = a.lay.C;
  const int R = a.lay.R;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  T* khat = reinterpret_cast<T*>(tree + tr * a.lay.stride + a.lay.khat[level]);
  float* bhat = reinterpret_cast<float*>(tree + tr * a.lay.stride + a.lay.bhat[level]);
  // First child's scratch row (per reference block).
  const int64_t child0 = tr * a.lay.ncap[level - 1] + i * C;
  // Children's log-masses at the parent's rotated reference (one wave's row).
  __shared__ double s_f[ROPE ? 4 : 1][ROPE ? 1024 : 1];
  double* fw = s_f[ROPE ? (threadIdx.x >> 6) : 0];
  double span = 1.0;
  for (int l = 0; l < level; ++l) span *= C;
  const double pos = (double)(i + 1) * span - 1.0;  // the node's last position

  for (int r = 0; r < R; ++r) {
    double qp[DPL];
    node_reference<D, ROPE>(qref + ((int64_t)kvh * R + r) * D, lane, a, pos, qp);
    // Maximum child log-mass.
    double m = -INFINITY;
    if constexpr (ROPE) {
      for (int c = 0; c < C; ++c) {
        const double* krow = cK + ((child0 + c) * R + r) * D + lane * DPL;
        double part = 0.0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) part = fma(qp[e], krow[e], part);
        const double f = cF[(child0 + c) * R + r] + group_sum64<kWave>(part) * inv_sqrt_d;
        fw[c] = f;  // every lane holds f; the row is read back by this wave only
        m = fmax(m, f);
      }
    } else {
      for (int c = lane; c < C; c += kWave) m = fmax(m, cF[(child0 + c) * R + r]);
      m = group_max64<kWave>(m);
    }
    // Weight sum and rescaled sum of the children's summaries, children in order.
    double Z = 0.0;
    double acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0;
    for (int c0 = 0; c0 < C; c0 += kWave) {
      const double f_mine =
          c0 + lane < C ? (ROPE ? fw[c0 + lane] : cF[(child0 + c0 + lane) * R + r]) : 0.0;
      const double e_mine = (c0 + lane < C) ? exp(f_mine - m) : 0.0;
      const int cn = min(kWave, C - c0);
      // Children's rows kB at a time, all loads of a batch issued first; the
      // sums run child by child in order.
      constexpr int kB = 8;
      for (int cb = 0; cb < cn; cb += kB) {
        double kr[kB][DPL];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const double* krow = cK + ((child0 + c0 + min(cb + u, cn - 1)) * R + r) * D + lane * DPL;
#pragma unroll
          for (int e = 0; e < DPL; ++e) kr[u][e] = krow[e];
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          if (cb + u >= cn) break;
          const double w = __shfl(e_mine, cb + u, kWave);
          Z += w;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fma(w, kr[u][e], acc[e]);
        }
      }
    }
    const double F = m + log(Z);
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      acc[e] = acc[e] / Z;
      part = fma(qp[e], acc[e], part);
    }
    const double b = F - group_sum64<kWave>(part) * inv_sqrt_d;
    const int64_t row = i * R + r;
#pragma unroll
    for (int e = 0; e < DPL; ++e) store_elem64(khat, row * D + lane * DPL + e, acc[e]);
    if (lane == 0) bhat[row] = (float)b;
    if (pF != nullptr) {
      const int64_t prow = (tr * a.lay.ncap[level] + i) * R + r;
#pragma unroll
      for (int e = 0; e < DPL; ++e) pK[prow * D + lane * DPL + e] = acc[e];
      if (lane == 0) pF[prow] = ROPE ? b : F;
    }
  }
}

template <typename T, int D>
static int launch_build(const BuildArgs& a, const void* K, const float* qref, void* tree,
                        void* scratch, hipStream_t s) {
  const BuildScratch sc = build_scratch_layout(a);
  char* base = reinterpret_cast<char*>(scratch);
  auto F = [&](int l) { return reinterpret_cast<double*>(base + sc.F[l]); };
  auto Kp = [&](int l) { return reinterpret_cast<double*>(base + sc.K[l]); };
  const int L = a.lay.L;
  if (a.lay.n[1] > a.lo[1]) {
    const int64_t nodes = (int64_t)a.n_trees * (a.lay.n[1] - a.lo[1]);
    const unsigned blocks = (unsigned)((nodes + 3) / 4);
    if (a.rope_dims)
      leaf_kernel<T, D, true><<<blocks, 256, 0, s>>>(
          reinterpret_cast<const T*>(K), qref, reinterpret_cast<char*>(tree),
          L > 1 ? F(1) : nullptr, L > 1 ? Kp(1) : nullptr, a);
    else
      leaf_kernel<T, D, false><<<blocks, 256, 0, s>>>(
          reinterpret_cast<const T*>(K), qref, reinterpret_cast<char*>(tree),
          L > 1 ? F(1) : nullptr, L > 1 ? Kp(1) : nullptr, a);
    if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
  }
  for (int l = 2; l <= L; ++l) {
    if (a.lay.n[l] == a.lo[l]) continue;  // no span of this level completed
    const int64_t nodes = (int64_t)a.n_trees * (a.lay.n[l] - a.lo[l]);
    const unsigned blocks = (unsigned)((nodes + 3) / 4);
    if (a.rope_dims)
      merge_kernel<T, D, true><<<blocks, 256, 0, s>>>(qref, reinterpret_cast<char*>(tree),
                                                      F(l - 1), Kp(l - 1),
                                                      l < L ? F(l) : nullptr,
                                                      l < L ? Kp(l) : nullptr, a, l);
    else
      merge_kernel<T, D, false><<<blocks, 256, 0, s>>>(qref, reinterpret_cast<char*>(tree),
                                                       F(l - 1), Kp(l - 1),
                                                       l < L ? F(l) : nullptr,
                                                       l < L ? Kp(l) : nullptr, a, l);
    if (hipGetLastError() != hipSuccess) return ZHA_ERR_LAUNCH;
  }
  return ZHA_OK;
}

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
