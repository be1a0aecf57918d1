// Host/device argument blocks, buffer layouts and launch entry points shared
// by the kernel translation units and the C ABI.
#pragma once

#include "zha_common.hpp"
#include "zha_plan.hpp"

namespace zha {

constexpr int kRouteFrontierMax = 4096;  // candidates per level held in LDS by the router
constexpr int64_t kTputMinHeads = 4096;  // query heads per call for the router's throughput shape
constexpr int kRouteSpillBlocks = 8;     // device-memory frontier slots for heads that outgrow the LDS
// A head waiting for a device-memory frontier slot retries all slots this many
// rounds (a ~1 us sleep each) before it gives up with cnt = ZHA_ROUTE_SLOT_BUSY.
constexpr int32_t kRouteSpillWaitRounds = 1 << 20;
// Fractional bits of the fixed-point candidate masses of the top-p cut: the
// top candidate's mass is exactly 2^kMassBits.
constexpr int kMassBits = 40;

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// zha_route scratch (byte offsets, -1 where absent).
//   list1  throughput shape (n_heads >= kTputMinHeads): a count and the heads
//          whose frontier outgrew its LDS, routed again by the latency shape.
//   ws     trees whose level 1 can hold more than kRouteFrontierMax nodes (n1c,
//          at capacity): kRouteSpillBlocks slots, each a frontier of n1c
//          candidates in device memory (two id arrays and the scores, 12 bytes
//          per candidate), for the heads that outgrow the latency shape's LDS.
struct RouteScratch {
  int64_t list1 = -1, ws = -1, ws_stride = 0, bytes = 0;
};
inline RouteScratch route_scratch_layout(int64_t n_heads, int64_t n1c) {
  RouteScratch s;
  int64_t off = 0;
  if (n_heads >= kTputMinHeads) {
    s.list1 = off;
    off += align256((n_heads + 1) * 4);
  }
  if (n1c > kRouteFrontierMax) {
    s.ws_stride = align256(n1c * 12);
    s.ws = off;
    off += s.ws_stride * kRouteSpillBlocks;
  }
  s.bytes = off;
  return s;
}

#ifndef ZHA_ATTN_BLOCKS
#define ZHA_ATTN_BLOCKS 512
#endif

// Block path of zha_attn (calls with more than kBalMaxHeads query heads):
// (query head, tile) pairs, a tile being CT consecutive chunks of one (b, kvh)
// cache.  A head takes one partial slot per tile of its selected chunks plus
// one for its sink and partial-chunk tokens; slots are handed out by a prefix
// sum over the heads, within a budget of kBlkSlots per head on average (heads
// past the budget are attended one head per workgroup instead and take no
// pairs, so the entries never outnumber the slots).  Scratch:
// counters, per-head slot bases and tile counts, per-tile counts and offsets,
// the pair entries and the fp32 partials (d + 2 each).
constexpr int kBlkSlots = 9;
constexpr int kBlkEntryInts = 4;  // head, slot, mask lo, mask hi

struct BlkLayout {
  int32_t CT;  // chunks per tile (<= 64: one bit each in a 64-bit mask)
  int32_t lct;  // log2(CT)
  int32_t NT;  // tiles per (b, kvh) cache
  int64_t NTT;  // tiles in all
  int64_t S;    // slot budget
  int64_t off_ctrl, off_qbase, off_ntile, off_wsum, off_tcnt, off_tcur, off_toff, off_wpre,
      off_wbase, off_ent, off_part, total;
};

// The block path serves bf16 caches with d in {64, 128} and C in {8, 16, 32, 64}.
inline bool blk_eligible(int64_t n_heads, int C, int d, int dtype) {
  return n_heads > kBalMaxHeads && dtype == ZHA_BF16 && (d == 64 || d == 128) &&
         (C == 8 || C == 16 || C == 32 || C == 64);
}

inline BlkLayout blk_layout(int64_t n_heads, int64_t n_trees, int64_t T, int C, int d) {
  BlkLayout L{};
  const int64_t nchunks = (T + C - 1) / C;
  L.CT = C >= 16 ? 1024 / C : 64;
  L.lct = __builtin_ctz((unsigned)L.CT);
  L.NT = (int32_t)((nchunks + L.CT - 1) / L.CT);
  L.NTT = n_trees * L.NT;
  L.S = n_heads * kBlkSlots;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  L.off_ctrl = take(64);
  L.off_qbase = take(n_heads * 4);
  L.off_ntile = take(n_heads * 4);
  L.off_wsum = take((n_heads + 127) / 128 * 8);  // slots per workgroup of the count launch
  L.off_tcnt = take(L.NTT * 4);
  L.off_tcur = take(L.NTT * 4);
  L.off_toff = take((L.NTT + 1) * 4);
  L.off_wpre = take((L.NTT + 1) * 4);
  // Per workgroup of the per-tile launches (128 heads of one cache), its first
  // entry within each tile's range.
  const int64_t per_tree = n_heads / n_trees;
  L.off_wbase = take(n_trees * ((per_tree + 127) / 128) * L.NT * 4);
  L.off_ent = take(L.S * kBlkEntryInts * 4);
  L.off_part = take(L.S * (int64_t)(d + 2) * 4);
  L.total = off;
  return L;
}

// zha_attn scratch: with n_heads <= kBalMaxHeads, a plan (n_heads + 2 int64)
// and (workgroups + n_heads) partials of d + 2 floats; with more heads, the
// block path's layout when it applies, else none.
inline int64_t attn_scratch_layout_bytes(int64_t n_heads, int64_t n_trees, int64_t T, int C, int d,
                                         int dtype) {
  if (n_heads > kBalMaxHeads)
    return blk_eligible(n_heads, C, d, dtype) ? blk_layout(n_heads, n_trees, T, C, d).total : 0;
  return align256((n_heads + 2) * 8) + (ZHA_ATTN_BLOCKS + n_heads) * (int64_t)(d + 2) * 4;
}

struct BuildArgs {
  TreeLayout lay;
  int32_t n_trees;  // B * H_kv
  int32_t H_kv;
  int32_t d;
  int32_t chunked;  // ZHA_KV_CHUNKED layout
  int64_t T;
  int64_t Tc;                    // token capacity (strides)
  int64_t lo[kMaxLevels + 1];    // first node of each level to summarise (0 for a build)
  int32_t rope_dims;             // rotated dims of the references (0: none)
  double theta[128];             // their angular frequencies (rope_dims / 2 used)
};

// fp64 F [n_trees, nc_l, R] and k_hat [n_trees, nc_l, R, d] for levels 1..L-1
// (nc_l: rows of capacity).  With rotated references the F slot holds the fp64
// bias b_hat instead: a child's log-mass at its parent's reference is then its
// tangent there, b_hat_c + q_P . k_hat_c / sqrt(d).
struct BuildScratch {
  int64_t F[kMaxLevels + 1];
  int64_t K[kMaxLevels + 1];
  int64_t total;
};

struct RouteArgs {
  TreeLayout lay;
  int64_t T;
  int64_t span[kMaxLevels + 1];  // C^l: tokens under a level-l node
  const int32_t* ctx;  // visible length per position [B, n_pos] (device), or null: all T
  int64_t n_heads;  // B * n_pos * H_q
  int32_t n_pos;
  int32_t H_q;
  int32_t H_kv;
  int32_t G;
  int32_t cap;
  float p;
  uint32_t cdiv;  // ceil(2^32 / C): floor(x / C) = umulhi(x, cdiv) for 0 <= x < 2^16
  int32_t spill_wait;  // rounds of waiting for a frontier slot (negative: none)
};

// Tokens visible to query head h (of B * n_pos * H_q): its position's entry
// of ctx, or T; -1 when the entry is outside [1, T] (the head then fails).
template <typename A>
__device__ __forceinline__ int64_t visible_len(const A& a, int64_t h) {
  if (a.ctx == nullptr) return a.T;
  const int64_t v = a.ctx[h / a.H_q];
  return (v >= 1 && v <= a.T) ? v : -1;
}

struct AttnArgs {
  int64_t T;
  int64_t Tc;       // token capacity (KV strides)
  const int32_t* ctx;  // visible length per position [B, n_pos] (device), or null: all T
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
  int32_t dtype;
};

struct DenseArgs {
  int64_t T;
  int64_t Tc;   // token capacity (KV strides)
  int64_t tps;  // tokens per split (matrix-core path; a multiple of 32)
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
    off += align256((int64_t)a.n_trees * a.lay.ncap[l] * a.lay.R * 8);
    s.K[l] = off;
    off += align256((int64_t)a.n_trees * a.lay.ncap[l] * a.lay.R * a.d * 8);
  }
  s.total = off;
  return s;
}

// Fused route + attention (zha_route_attn): calls of up to kFzMaxHeads query
// heads with R = 1, a power-of-two C, p < 1 and K/V blocks under 2^31 bytes
// run as one persistent launch of kFzGrid workgroups; a head's attended
// tokens are cut into at most kFzMaxPieces pieces of at least kFzPieceTokens.
// Scratch: zha_route's (device-memory frontier slots), then fp32 partials
// (d + 2 each) for kFzMaxPieces pieces per head.
constexpr int kFzMaxHeads = kBalMaxHeads;
constexpr int kFzMaxPieces = 64;
constexpr int kFzPieceTokens = 1024;
constexpr unsigned kFzGrid = 256;
inline bool fused_eligible(int64_t n_heads, int R, int C, float p, int64_t kv_block_bytes) {
  return n_heads <= kFzMaxHeads && R == 1 && (C & (C - 1)) == 0 && p < 1.0f &&
         kv_block_bytes < ((int64_t)1 << 31);
}

// Launch entry points (defined in the .hip files).
int build_dispatch(const BuildArgs& a, int dtype, int d, const void* K, const float* qref,
                   void* tree, void* scratch, hipStream_t s);
int route_dispatch(const RouteArgs& a, int dtype, int d, const void* tree, const void* Q,
                   int32_t* sel, int32_t* cnt, int32_t* stats, float* gap, void* scratch,
                   hipStream_t s);
int attn_dispatch(const AttnArgs& a, int dtype, int d, const void* Q, const void* K,
                  const void* V, const int32_t* sel, const int32_t* cnt, void* O, void* scratch,
                  hipStream_t s);
int dense_dispatch(const DenseArgs& a, int dtype, int d, const void* Q, const void* K,
                   const void* V, void* O, void* scratch, hipStream_t s);
int fused_dispatch(const RouteArgs& ra, const AttnArgs& aa, int dtype, int d, const void* tree,
                   const void* Q, const void* K, const void* V, int32_t* sel, int32_t* cnt,
                   int32_t* stats, float* gap, void* O, char* ws, int64_t ws_stride, float* part,
                   unsigned grid, uint32_t tag, hipStream_t s);

// Dense decode on the matrix cores (bf16, d in {64, 128}): S waves per (KV
// cache, 16 query rows), each taking whole 32-token steps; S makes about
// ZHA_DENSE_WAVES waves in all (two per SIMD on 256 CUs), none without a step.
#ifndef ZHA_DENSE_WAVES
#define ZHA_DENSE_WAVES 2048
#endif
inline bool dense_mfma_eligible(int dtype, int d) {
  return dtype == ZHA_BF16 && (d == 64 || d == 128);
}
struct DensePlan {
  int32_t S;    // splits per (cache, 16 rows)
  int64_t tps;  // tokens per split
};
inline DensePlan dense_mfma_plan(int64_t n_trees, int64_t rows, int64_t T) {
  const int64_t units = n_trees * ((rows + 15) / 16);
  int64_t s = (ZHA_DENSE_WAVES + units - 1) / units;
  const int64_t steps = (T + 31) / 32;
  if (s > steps) s = steps;
  if (s > 65535) s = 65535;
  if (s < 1) s = 1;
  // At most 2^22 tokens per split: the kernel addresses a split's rows with
  // 32-bit byte offsets (chunked caches span twice the rows).
  const int64_t smin = (T + (1 << 22) - 1) >> 22;
  if (s < smin) s = smin;
  const int64_t tps = ((T + s - 1) / s + 31) / 32 * 32;
  return DensePlan{(int32_t)((T + tps - 1) / tps), tps};
}

// Split-KV scratch: fp32 partials [n_heads, S, d + 2] (S == 1 needs none).
inline int64_t splitkv_scratch_bytes(int64_t n_heads, int S, int d) {
  return S > 1 ? n_heads * S * (int64_t)(d + 2) * 4 : 0;
}

}  // namespace zha
