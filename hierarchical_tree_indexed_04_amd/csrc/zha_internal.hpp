// Host/device argument blocks, buffer layouts and launch entry points shared
// by the kernel translation units and the C ABI.
#pragma once

#include "zha_common.hpp"

namespace zha {

constexpr int kRouteFrontierMax = 4096;  // candidates per level held in LDS by the router
constexpr int kBalMaxHeads = 2048;       // balanced split-KV: per-head prefix held in LDS

#ifndef ZHA_ATTN_BLOCKS
#define ZHA_ATTN_BLOCKS 512
#endif

// zha_attn scratch: with n_heads <= kBalMaxHeads, a plan (n_heads + 2 int32)
// and (workgroups + n_heads) partials of d + 2 floats; otherwise none.
inline int64_t attn_scratch_layout_bytes(int64_t n_heads, int d) {
  if (n_heads > kBalMaxHeads) return 0;
  return ((n_heads + 2) * 4 + 255) / 256 * 256 + (ZHA_ATTN_BLOCKS + n_heads) * (int64_t)(d + 2) * 4;
}

struct BuildArgs {
  TreeLayout lay;
  int32_t n_trees;  // B * H_kv
  int32_t H_kv;
  int32_t d;
  int32_t chunked;  // ZHA_KV_CHUNKED layout
  int64_t T;
};

// fp64 F [n_trees, n_l, R] and k_hat [n_trees, n_l, R, d] for levels 1..L-1.
struct BuildScratch {
  int64_t F[kMaxLevels + 1];
  int64_t K[kMaxLevels + 1];
  int64_t total;
};

struct RouteArgs {
  TreeLayout lay;
  int64_t n_heads;  // B * n_pos * H_q
  int32_t n_pos;
  int32_t H_q;
  int32_t H_kv;
  int32_t G;
  int32_t cap;
  float p;
};

struct AttnArgs {
  int64_t T;
  int64_t n_heads;  // B * n_pos * H_q
  int64_t n1;       // full leaf chunks
  int32_t n_pos;
  int32_t H_q;
  int32_t H_kv;
  int32_t G;
  int32_t C;
  int32_t log2C;  // log2(C) when C is a power of two, else -1
  int32_t cap;
  int32_t S;      // workgroups of the balanced split (or splits per head)
  int32_t chunked;  // ZHA_KV_CHUNKED layout
};

struct DenseArgs {
  int64_t T;
  int64_t n_heads;
  int32_t n_pos;
  int32_t H_q;
  int32_t H_kv;
  int32_t G;
  int32_t S;
  int32_t C;
  int32_t log2C;    // log2(C) when C is a power of two, else -1
  int32_t chunked;  // ZHA_KV_CHUNKED layout
};

// Elements of one (b, kvh) block of the KV cache: [T, d] per tensor (split)
// or [ceil(T / C), 2, C, d] holding both (chunked).
__host__ __device__ inline int64_t kv_block_elems(int64_t T, int C, int d, bool chunked) {
  return chunked ? (T + C - 1) / C * 2 * C * (int64_t)d : T * (int64_t)d;
}

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Query heads per dense-decode workgroup: the largest of 8, 4, 2, 1 dividing G.
#ifndef ZHA_DENSE_MAX_TILE
#define ZHA_DENSE_MAX_TILE 8
#endif
inline int dense_head_tile(int G) {
  for (int t = ZHA_DENSE_MAX_TILE; t > 1; t >>= 1)
    if (G % t == 0) return t;
  return 1;
}

inline BuildScratch build_scratch_layout(const BuildArgs& a) {
  BuildScratch s{};
  int64_t off = 0;
  for (int l = 1; l < a.lay.L; ++l) {
    s.F[l] = off;
    off += align256((int64_t)a.n_trees * a.lay.n[l] * a.lay.R * 8);
    s.K[l] = off;
    off += align256((int64_t)a.n_trees * a.lay.n[l] * a.lay.R * a.d * 8);
  }
  s.total = off;
  return s;
}

// Launch entry points (defined in the .hip files).
int build_dispatch(const BuildArgs& a, int dtype, int d, const void* K, const float* qref,
                   void* tree, void* scratch, hipStream_t s);
int route_dispatch(const RouteArgs& a, int dtype, int d, const void* tree, const void* Q,
                   int32_t* sel, int32_t* cnt, int32_t* stats, float* gap, hipStream_t s);
int attn_dispatch(const AttnArgs& a, int dtype, int d, const void* Q, const void* K,
                  const void* V, const int32_t* sel, const int32_t* cnt, void* O, void* scratch,
                  hipStream_t s);
int dense_dispatch(const DenseArgs& a, int dtype, int d, const void* Q, const void* K,
                   const void* V, void* O, void* scratch, hipStream_t s);

// Split-KV scratch: fp32 partials [n_heads, S, d + 2] (S == 1 needs none).
inline int64_t splitkv_scratch_bytes(int64_t n_heads, int S, int d) {
  return S > 1 ? n_heads * S * (int64_t)(d + 2) * 4 : 0;
}

}  // namespace zha
