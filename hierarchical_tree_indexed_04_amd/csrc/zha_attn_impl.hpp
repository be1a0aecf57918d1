// Building blocks of the sparse attention kernels, shared by zha_attn and the
// fused route + attention entry: the K/V rows of one cache in either layout,
// q . k over 16-byte row slices, the online softmax of a row group, the
// combine of a workgroup's row groups into an output row or a split partial,
// the merge of a head's partials, and the attention of one head over a range
// of its token list (attend_segment).
//
// Attended tokens of a query head (the summary page of the paper, "Routing":
// I(q) = {0} U selected leaf chunks U C_cur): its list is the tokens of its
// selected chunks in chunk order, then the sink (token 0, unless chunk 0 is
// selected) and the tail after the last full chunk.
//
// COH (the fused entry): the chunk ids are read, and partials written and read
// back, with device-coherent (agent-scope) accesses, for data that workgroups
// on other XCDs produce or consume within the same launch.
#pragma once

#include "zha_internal.hpp"
#include "zha_wave.hpp"

namespace zha {
namespace {

constexpr int kThreads = 256;
#ifndef ZHA_ATTN_ROWS
#define ZHA_ATTN_ROWS 4
#endif
#ifndef ZHA_DENSE_ROWS
#define ZHA_DENSE_ROWS 4
#endif
#ifndef ZHA_ATTN_WAVES
#define ZHA_ATTN_WAVES 2
#endif
constexpr int kUA = ZHA_ATTN_ROWS;   // K/V rows in flight per lane (sparse)
constexpr int kUD = ZHA_DENSE_ROWS;  // K/V rows in flight per lane (dense)
constexpr int kIds = 1024;  // chunk ids staged in LDS per round (sparse)
constexpr int kWaves = kThreads / kWave;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// q . k over one 16-byte slice of a row.  bf16: packed bf16 dot products
// (exact products, fp32 sums); fp32: fused multiply-adds.
template <typename T>
__device__ __forceinline__ float slice_dot(const uint4& k, const uint4& q) {
  if constexpr (sizeof(T) == 2) {
    float d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.x), as_bf16x2(q.x), 0.0f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.y), as_bf16x2(q.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.z), as_bf16x2(q.z), d, false);
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(k.w), as_bf16x2(q.w), d, false);
  } else {
    float d = __uint_as_float(k.x) * __uint_as_float(q.x);
    d = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), d);
    d = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), d);
    return fmaf(__uint_as_float(k.w), __uint_as_float(q.w), d);
  }
}

// Inclusive prefix sum over the 64 lanes of a 32-bit value.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u32<kDppRowShr1>(0u, v);
  v += dpp_u32<kDppRowShr2>(0u, v);
  v += dpp_u32<kDppRowShr4>(0u, v);
  v += dpp_u32<kDppRowShr8>(0u, v);
  v += dpp_u32<kDppRowBcast15, 0xA>(0u, v);
  v += dpp_u32<kDppRowBcast31, 0xC>(0u, v);
  return v;
}



// The K/V rows of one (b, kvh) pair in either cache layout.  Rows are
// addressed by key row: token j of chunk c is key row c * CS + j, with CS = C
// (split: K and V are [T, d] arrays, the value row has the same index in V)
// or 2 C (chunked: pages of C key rows then C value rows, the value row is C
// rows further in the same buffer).  Each lane reads its 16-byte slice `sub`.
// BUF: buffer loads (block < 2^31 bytes), a slot without a row reads nothing.
template <typename T, int D, bool BUF>
struct KvBlock {
  static constexpr uint32_t kRow = D * sizeof(T);
  const char* k;
  const char* v;
  buf_t rk, rv;
  int cs;
  __device__ __forceinline__ KvBlock(const T* K, const T* V, int64_t tr, int64_t T_, int C,
                                     int chunked, int sub) {
    const int64_t n = kv_block_elems(T_, C, D, chunked);
    const T* kb = K + tr * n;
    const T* vb = chunked ? kb + (int64_t)C * D : V + tr * n;
    k = reinterpret_cast<const char*>(kb) + sub * 16;
    v = reinterpret_cast<const char*>(vb) + sub * 16;
    const int64_t bytes = BUF ? n * (int64_t)sizeof(T) : 0;
    rk = make_buf(kb, bytes);
    rv = chunked ? rk : make_buf(vb, bytes);
    cs = chunked ? 2 * C : C;
    vdelta = chunked ? (uint32_t)C * kRow : 0u;
    sub16 = (uint32_t)sub * 16u;
  }
  uint32_t vdelta, sub16;
  __device__ __forceinline__ int key_row(int chunk, int j) const { return chunk * cs + j; }
  // K or V row alone (the same rules as load).
  __device__ __forceinline__ uint4 load_k(int row, bool live) const {
    if (BUF) return bld16(rk, live ? (uint32_t)row * kRow + sub16 : kBufNone);
    return live ? ld16(k + (size_t)(uint32_t)row * kRow) : make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ uint4 load_v(int row, bool live) const {
    if (BUF) return bld16(rv, live ? (uint32_t)row * kRow + sub16 + vdelta : kBufNone);
    return live ? ld16(v + (size_t)(uint32_t)row * kRow) : make_uint4(0u, 0u, 0u, 0u);
  }
  __device__ __forceinline__ void load(int row, bool live, uint4& kv, uint4& vv) const {
    if (BUF) {
      // Straight-line: a slot without a row reads nothing and gets zeros.
      const uint32_t off = live ? (uint32_t)row * kRow + sub16 : kBufNone;
      kv = bld16(rk, off);
      vv = bld16(rv, live ? off + vdelta : kBufNone);
    } else if (live) {
      const size_t off = (size_t)(uint32_t)row * kRow;
      kv = ld16(k + off);
      vv = ld16(v + off);
    } else {
      kv = make_uint4(0u, 0u, 0u, 0u);
      vv = make_uint4(0u, 0u, 0u, 0u);
    }
  }
};

// Device-coherent (agent-scope) accesses for data exchanged between the
// workgroups of one launch, or plain ones.
template <bool COH>
__device__ __forceinline__ void st_f32(float* p, float v) {
  if constexpr (COH)
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COH>
__device__ __forceinline__ float2 ld_f32x2(const float* p) {
  if constexpr (COH) {
    const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}
template <bool COH>
__device__ __forceinline__ int32_t ld_i32(const int32_t* p) {
  if constexpr (COH)
    return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// Combines the online-softmax states of the RPB row groups of a workgroup and
// writes either the final output row(s) or a split partial.
template <typename T, int D, int RPB, bool COH = false, int NT = kThreads>
__device__ __forceinline__ void combine_groups(float m, float l, const float* acc, int grp, int sub,
                                               float* s_m, float* s_l, float* s_acc,
                                               T* out_row, float* part_row) {
  constexpr int VEC = Vec<T>::N;
  if (sub == 0) {
    s_m[grp] = m;
    s_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) s_acc[grp * D + sub * VEC + e] = acc[e];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int g = 0; g < RPB; ++g) M = fmaxf(M, s_m[g]);
  for (int t = threadIdx.x; t < D; t += NT) {
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int g = 0; g < RPB; ++g) {
      const float w = (s_m[g] == -INFINITY) ? 0.f : __expf(s_m[g] - M);
      num = fmaf(w, s_acc[g * D + t], num);
      den = fmaf(w, s_l[g], den);
    }
    if (part_row != nullptr) {
      st_f32<COH>(part_row + t, num);
      if (t == 0) {
        st_f32<COH>(part_row + D, M);
        st_f32<COH>(part_row + D + 1, den);
      }
    } else {
      store_elem(out_row, t, num / den);
    }
  }
}

// Online-softmax update of one row group with U scores and value slices.
template <typename T, int U>
__device__ __forceinline__ void online_update(float& m, float& l, float* acc, const float* s,
                                              const uint4* vv) {
  constexpr int VEC = Vec<T>::N;
  float mloc = m;
#pragma unroll
  for (int u = 0; u < U; ++u) mloc = fmaxf(mloc, s[u]);
  // Branch-free (a branch here lets the compiler sink the V loads into it,
  // after the waits for K): with no finite score yet, the reference point is
  // 0 and every weight below is exp(-inf) = 0, leaving the state unchanged.
  const float mref = (mloc == -INFINITY) ? 0.f : mloc;
  const float scale = __expf(m - mref);  // m = -inf gives 0
  l *= scale;
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] *= scale;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float p = __expf(s[u] - mref);  // -inf scores give 0
    l += p;
    float v[VEC];
    Vec<T>::widen(vv[u], v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = fmaf(p, v[e], acc[e]);
  }
  m = mloc;
}

// Merge of S split partials (o unnormalised, m, l) of one head by the whole
// workgroup: thread (column pair c, group g) folds partials g, g + NG, ... with
// a running maximum (loads issued kSB at a time), then group 0 combines the NG
// group results from LDS, in group order.  Block-uniform call (one barrier).
template <typename T, int D, bool COH = false, int NT = kThreads>
__device__ __forceinline__ void merge_partials(const float* part_head, int S, T* out_row) {
  constexpr int NC = D / 2;           // column pairs (rows of D + 2 floats are 8-byte aligned)
  constexpr int NG = NT / NC;         // partial groups
  constexpr int kSB = 8;
  __shared__ float s_M[NG], s_den[NG];
  __shared__ float2 s_num[NG][NC];
  const int c = threadIdx.x % NC, g = threadIdx.x / NC;
  float M = -INFINITY, den = 0.f;
  float2 num = make_float2(0.f, 0.f);
  for (int s0 = g; s0 < S; s0 += NG * kSB) {
    float2 ml[kSB], av[kSB];
#pragma unroll
    for (int j = 0; j < kSB; ++j) {
      const int s = s0 + j * NG;
      const float* r = part_head + (int64_t)min(s, S - 1) * (D + 2);
      ml[j] = ld_f32x2<COH>(r + D);
      av[j] = ld_f32x2<COH>(r + 2 * c);
      if (s >= S) ml[j].x = -INFINITY;
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kSB; ++j) Mn = fmaxf(Mn, ml[j].x);
    if (Mn == -INFINITY) continue;
    const float rs = M == -INFINITY ? 0.f : __expf(M - Mn);
    num.x *= rs;
    num.y *= rs;
    den *= rs;
#pragma unroll
    for (int j = 0; j < kSB; ++j) {
      const float w = ml[j].x == -INFINITY ? 0.f : __expf(ml[j].x - Mn);
      num.x = fmaf(w, av[j].x, num.x);
      num.y = fmaf(w, av[j].y, num.y);
      den = fmaf(w, ml[j].y, den);
    }
    M = Mn;
  }
  if (c == 0) {
    s_M[g] = M;
    s_den[g] = den;
  }
  s_num[g][c] = num;
  __syncthreads();
  if (g == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int k = 0; k < NG; ++k) Mt = fmaxf(Mt, s_M[k]);
    float nx = 0.f, ny = 0.f, dt = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const float w = s_M[k] == -INFINITY ? 0.f : __expf(s_M[k] - Mt);
      nx = fmaf(w, s_num[k][c].x, nx);
      ny = fmaf(w, s_num[k][c].y, ny);
      dt = fmaf(w, s_den[k], dt);
    }
    store_elem(out_row, 2 * c, nx / dt);
    store_elem(out_row, 2 * c + 1, ny / dt);
  }
}

// LDS of attend_segment (NT threads per workgroup).
template <typename T, int D, int NT = kThreads>
struct SegSmem {
  static constexpr int RPB = NT / (D / Vec<T>::N);
  int32_t ids[kIds];
  float m[RPB], l[RPB];
  float acc[RPB * D];
};

// Attention of query head h over positions [x0, x1) of its token list, by the
// whole workgroup (block-uniform call, ends with a barrier).  c: its selected
// chunk count, listed ascending at ids; Th: the tokens it sees.  Writes the
// output row when prow is NULL, else a partial (o unnormalised, m, l) at prow.
// A workgroup streams the K and V rows of its positions (one 16-byte slice
// per lane, LPR lanes per row, kUA rows in flight per lane, q . k with packed
// bf16 dot products), keeps an online softmax per row group and combines the
// row groups in LDS in a fixed order.
template <typename T, int D, bool POW2, bool BUF, bool COH = false, int NT = kThreads>
__device__ __forceinline__ void attend_segment(const T* __restrict__ Q, const T* __restrict__ K,
                                               const T* __restrict__ V,
                                               const int32_t* __restrict__ ids, int c, int64_t Th,
                                               const AttnArgs& a, int64_t h, int x0, int x1,
                                               T* __restrict__ out_row, float* prow,
                                               SegSmem<T, D, NT>& sm) {
  constexpr int VEC = Vec<T>::N;
  constexpr int LPR = D / VEC;
  constexpr int RPB = NT / LPR;
  const int tid = threadIdx.x;
  const int sub = tid % LPR, grp = tid / LPR;
  const int n1 = (int)(Th / a.C);
  const bool sink = n1 > 0 && ((c == 0) || (ld_i32<COH>(ids) != 0));
  const int hq = (int)(h % a.H_q);
  const int64_t b = h / ((int64_t)a.n_pos * a.H_q);
  const int64_t tr = b * a.H_kv + hq / a.G;
  const KvBlock<T, D, BUF> kvb(K, V, tr, a.Tc, a.C, a.chunked, sub);
  const uint4 qv = ld16c(Q + (int64_t)h * D + sub * VEC);
  const float inv = 1.0f / sqrtf((float)D);
  const int Cc = a.C, log2C = a.log2C;
  const int ct = c * Cc;  // chunk tokens come first, then the extras
  float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int xr = x0; xr < x1;) {
    // Stage the chunk ids this round needs (positions [xr, xe) of the list).
    const int fc = xr < ct ? (log2C >= 0 ? (xr >> log2C) : xr / Cc) : 0;
    const int xe = xr < ct ? (int)min((int64_t)x1, (int64_t)(fc + kIds) * Cc) : x1;
    if (xr < ct) {
      const int lc = (min(xe, ct) - 1) / Cc;  // last chunk touched
      __syncthreads();
      for (int i = tid; i <= lc - fc; i += NT) sm.ids[i] = ld_i32<COH>(ids + fc + i);
      __syncthreads();
    }
    // Each tensor's rows of the next batch are loaded as soon as its rows of
    // the current batch have been read: K(i + 1) right after the scores of
    // batch i, V(i + 1) right after its softmax update.  Past the round's
    // end a batch loads nothing (slots without a row use out-of-range buffer
    // offsets), so the loads stay unconditional and each wait counts exactly
    // the loads issued after it.  The next batch's key rows (which need
    // branches) are computed first, so the loads and the arithmetic form one
    // straight-line block; the empty asm statements keep them in order.
    auto rows_of = [&](int base, int (&row)[kUA]) {
      // Chunk ids from LDS for every slot first (clamped in bounds, one wait).
#pragma unroll
      for (int u = 0; u < kUA; ++u) {
        const int x = base + u * RPB + grp;
        const int ci = POW2 ? (x >> log2C) : x / Cc;
        row[u] = sm.ids[min(max(ci - fc, 0), kIds - 1)];
      }
#pragma unroll
      for (int u = 0; u < kUA; ++u) {
        // Position x is token j of chunk `row` (a selected chunk), or an
        // extra: the sink (chunk 0, token 0) or token e - sink of the
        // partial chunk n1.
        const int x = base + u * RPB + grp;
        const int ci = POW2 ? (x >> log2C) : x / Cc;
        const int e = x - ct;
        const bool is_sink = sink && e == 0;
        const int chunk = x < ct ? row[u] : (is_sink ? 0 : n1);
        const int j = x < ct ? x - ci * Cc : (is_sink ? 0 : e - (sink ? 1 : 0));
        row[u] = kvb.key_row(chunk, j);
      }
    };
    constexpr int kStep = RPB * kUA;
    int row[kUA];
    uint4 kv[kUA], vv[kUA];
    rows_of(xr, row);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUA; ++u) kv[u] = kvb.load_k(row[u], xr + u * RPB + grp < xe);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUA; ++u) vv[u] = kvb.load_v(row[u], xr + u * RPB + grp < xe);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    for (int base = xr; base < xe; base += kStep) {
      const int nb = base + kStep;
      rows_of(nb, row);
      asm volatile("" ::: "memory");
      float sc[kUA];
#pragma unroll
      for (int u = 0; u < kUA; ++u) {
        const float dot = group_allreduce<LPR>(slice_dot<T>(kv[u], qv), OpAdd()) * inv;
        sc[u] = (base + u * RPB + grp < xe) ? dot : -INFINITY;
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kUA; ++u) kv[u] = kvb.load_k(row[u], nb + u * RPB + grp < xe);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      online_update<T, kUA>(m, l, acc, sc, vv);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kUA; ++u) vv[u] = kvb.load_v(row[u], nb + u * RPB + grp < xe);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
    }
    xr = xe;
  }
  combine_groups<T, D, RPB, COH, NT>(m, l, acc, grp, sub, sm.m, sm.l, sm.acc, out_row, prow);
  __syncthreads();
}

}  // namespace
}  // namespace zha
