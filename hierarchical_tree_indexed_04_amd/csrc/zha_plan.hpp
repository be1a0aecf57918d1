// Planning arithmetic of the balanced split of zha_attn, shared by the
// kernels and by host-side checks of the plan (the includer provides
// __host__ / __device__, i.e. includes the HIP runtime first).
//
// The attended tokens I(q) of every query head of a call (summary page of the
// paper, "Routing": the sink, the selected leaf chunks and the current partial
// chunk) are laid end to end; head h owns positions [P_h, P_{h+1}) of that
// list, P being the exclusive prefix of the per-head counts.  Range w (one
// workgroup) owns [w W, (w + 1) W).  A head attends up to T < 2^31 tokens, so
// a call of kBalMaxHeads heads reaches 2^42 positions: every prefix, range
// bound and width is 64-bit, and only a position inside one head's own list
// fits 32 bits.
#pragma once

#include <stdint.h>

namespace zha {

// Placement of work on the XCDs: workgroup b of a 1-D launch runs on XCD
// b mod kXcds, and each XCD has an L2 of its own.
constexpr int kXcds = 8;

// The work index that gives XCD x the contiguous range [x n / 8, (x + 1) n / 8)
// (exactly, for n divisible by 8; otherwise the identity).
__host__ __device__ inline int64_t xcd_major_index(int64_t i, int64_t n) {
  if (n % kXcds != 0) return i;
  return (i % kXcds) * (n / kXcds) + i / kXcds;
}

// The work index of workgroup b when blocks of q consecutive indexes go to one
// XCD and the blocks are dealt round-robin over the XCDs (a permutation of
// [0, n) for n divisible by 8 q; otherwise the identity).
__host__ __device__ inline int xcd_blocked_index(int b, int n, int q) {
  if (q <= 1 || n % (kXcds * q) != 0) return b;
  const int x = b % kXcds, j = b / kXcds;
  return ((j / q) * kXcds + x) * q + j % q;
}

constexpr int kBalMaxHeads = 2048;  // balanced split-KV: per-head prefix held in LDS
constexpr int kBalMinTokens = 64;   // smallest token range of a workgroup

// |I(q)| of one query head with c selected chunks (first_id the lowest),
// seeing Th tokens: the chunks' tokens, the tail after the last full chunk,
// and the sink unless chunk 0 is selected (or no chunk is complete, when the
// tail starts at token 0).  0 for a failed route (c < 0, c > cap, Th < 0).
__host__ __device__ inline int64_t bal_head_tokens(int64_t c, int32_t first_id, int64_t Th,
                                                   int32_t C, int32_t cap) {
  if (c < 0 || c > cap || Th < 0) return 0;
  const int64_t n1 = Th / C;
  const int64_t sink = (n1 > 0 && (c == 0 || first_id != 0)) ? 1 : 0;
  return c * C + (Th - n1 * C) + sink;
}

// Width of each of `ranges` ranges over `total` positions.
__host__ __device__ inline int64_t bal_width(int64_t total, int64_t ranges) {
  const int64_t w = (total + ranges - 1) / ranges;
  return w < kBalMinTokens ? kBalMinTokens : w;
}

// The head holding position lo: the last h with pre[h] <= lo.  Requires
// pre[0] = 0 <= lo < pre[nh] (pre nondecreasing).
template <typename Pre>
__host__ __device__ inline int bal_first_head(const Pre& pre, int nh, int64_t lo) {
  int h0 = 0, h1 = nh;  // invariant: pre[h0] <= lo < pre[h1]
  while (h1 - h0 > 1) {
    const int mid = (h0 + h1) >> 1;
    if ((int64_t)pre[mid] <= lo) h0 = mid; else h1 = mid;
  }
  return h0;
}

// Positions [x0, x1) of a head's own list ([P0, P1) in the call's list) that
// fall in the range [lo, hi); empty (x0 >= x1) when they do not meet.
struct BalSegment {
  int32_t x0, x1;
};
__host__ __device__ inline BalSegment bal_segment(int64_t P0, int64_t P1, int64_t lo, int64_t hi) {
  const int64_t a = lo > P0 ? lo : P0;
  const int64_t b = hi < P1 ? hi : P1;
  BalSegment s;
  s.x0 = (int32_t)(a - P0);
  s.x1 = (int32_t)(b > a ? b - P0 : a - P0);
  return s;
}

// The ranges holding a head's positions [P0, P1) (P1 > P0): first .. last.
struct BalSpan {
  int64_t first, last;
};
__host__ __device__ inline BalSpan bal_head_span(int64_t P0, int64_t P1, int64_t W) {
  return BalSpan{P0 / W, (P1 - 1) / W};
}

// Partial slot of range w for head h: unique over all (w, h) pairs with h's
// positions in w, below ranges + heads (the slots of one head are consecutive).
__host__ __device__ inline int64_t bal_slot(int64_t w, int64_t h) { return w + h; }

}  // namespace zha
