// Host-side check of the balanced split plan of zha_attn (zha_plan.hpp) at
// sizes where a 32-bit prefix of per-head token counts would wrap.  Built
// host-only with hipcc (the plan functions are __host__ __device__) and run
// on the CPU.  For each case: every position of every head lies in exactly
// one range, a head's segments are consecutive and cover its list, the
// ranges a head meets are exactly those of bal_head_span, and partial slots
// are unique and inside the buffer.  Also the placement of work indexes on
// the XCDs.  Prints one line per case; exit status 0 when all hold.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "zha_plan.hpp"

using namespace zha;

static int fails = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c);             \
      if (++fails > 20) std::exit(1);                                     \
    }                                                                     \
  } while (0)

struct Head {
  int64_t c;
  int32_t first;
  int64_t Th;
};

static void run_case(const char* name, const std::vector<Head>& heads, int C, int cap,
                     int64_t ranges) {
  const int nh = (int)heads.size();
  std::vector<int64_t> tok(nh), pre(nh + 1, 0);
  for (int h = 0; h < nh; ++h) {
    tok[h] = bal_head_tokens(heads[h].c, heads[h].first, heads[h].Th, C, cap);
    CHECK(tok[h] >= 0 && tok[h] < ((int64_t)1 << 31));
    pre[h + 1] = pre[h] + tok[h];
  }
  const int64_t total = pre[nh];
  const int64_t W = bal_width(total, ranges);
  CHECK(W * ranges >= total);
  std::vector<int64_t> covered(nh, 0), next_x(nh, 0);
  std::vector<int64_t> first_seen(nh, -1), last_seen(nh, -1);
  std::set<int64_t> slots;
  for (int64_t w = 0; w < ranges; ++w) {
    const int64_t lo = w * W;
    const int64_t hi = lo + W < total ? lo + W : total;
    if (lo >= hi) continue;
    const int h0 = bal_first_head(pre, nh, lo);
    CHECK(pre[h0] <= lo && lo < pre[h0 + 1]);
    for (int h = h0; h < nh && pre[h] < hi; ++h) {
      if (pre[h + 1] <= lo || pre[h + 1] == pre[h]) continue;  // as the kernel: no tokens
      const BalSegment s = bal_segment(pre[h], pre[h + 1], lo, hi);
      CHECK(s.x0 < s.x1);
      CHECK(s.x0 == next_x[h]);  // consecutive, in range order
      CHECK((int64_t)s.x1 <= tok[h]);
      next_x[h] = s.x1;
      covered[h] += s.x1 - s.x0;
      if (first_seen[h] < 0) first_seen[h] = w;
      last_seen[h] = w;
      const bool whole = s.x0 == 0 && (int64_t)s.x1 == tok[h];
      if (!whole) {
        const int64_t slot = bal_slot(w, h);
        CHECK(slot >= 0 && slot < ranges + nh);
        CHECK(slots.insert(slot).second);
      }
    }
  }
  for (int h = 0; h < nh; ++h) {
    CHECK(covered[h] == tok[h]);
    if (tok[h] == 0) continue;
    const BalSpan sp = bal_head_span(pre[h], pre[h + 1], W);
    CHECK(sp.first == first_seen[h] && sp.last == last_seen[h]);
  }
  std::printf("%s: heads %d, total %lld positions (%s 2^31), width %lld, partial slots %zu\n",
              name, nh, (long long)total, total >= ((int64_t)1 << 31) ? ">=" : "<",
              (long long)W, slots.size());
}

// Work placement (zha_plan.hpp): both maps are permutations of [0, n); where
// they apply, xcd_major_index gives XCD x (workgroups b with b mod 8 = x) the
// contiguous range [x n / 8, (x + 1) n / 8), and xcd_blocked_index puts each
// block of q consecutive indexes on one XCD with every XCD holding n / 8.
static void check_placement() {
  const int ns[] = {7, 100, 256, 512, 768, 1024, 2048, 4096};
  const int qs[] = {1, 2, 3, 4, 8, 16, 32};
  for (int n : ns) {
    std::vector<int> seen(n, 0);
    for (int b = 0; b < n; ++b) {
      const int64_t w = xcd_major_index(b, n);
      CHECK(w >= 0 && w < n);
      if (w >= 0 && w < n) ++seen[w];
      if (n % kXcds == 0) CHECK(w / (n / kXcds) == b % kXcds);
    }
    for (int w = 0; w < n; ++w) CHECK(seen[w] == 1);
    for (int q : qs) {
      std::vector<int> owner(n, -1);
      for (int b = 0; b < n; ++b) {
        const int w = xcd_blocked_index(b, n, q);
        CHECK(w >= 0 && w < n);
        if (w >= 0 && w < n) {
          CHECK(owner[w] == -1);
          owner[w] = b;
        }
      }
      const bool applies = q > 1 && n % (kXcds * q) == 0;
      std::vector<int> per_xcd(kXcds, 0);
      for (int w = 0; w < n; ++w) {
        CHECK(owner[w] >= 0);
        if (owner[w] < 0) continue;
        ++per_xcd[owner[w] % kXcds];
        if (!applies) CHECK(owner[w] == w);
        if (applies && w + 1 < n && (w + 1) % q != 0)
          CHECK(owner[w] % kXcds == owner[w + 1] % kXcds);
      }
      if (n % kXcds == 0)
        for (int x = 0; x < kXcds; ++x) CHECK(per_xcd[x] == n / kXcds);
    }
  }
  std::printf("work placement: xcd_major_index and xcd_blocked_index are permutations%s\n",
              fails ? " (FAILED)" : "");
}

int main() {
  check_placement();
  const int64_t T = ((int64_t)1 << 31) - 3;  // the largest geometry: T < 2^31
  // 2048 heads that keep every chunk (p = 1): ~2^42 positions in all.
  {
    const int C = 16;
    const int64_t n1 = T / C;
    std::vector<Head> hs(kBalMaxHeads, Head{n1, 0, T});
    run_case("p=1, 2048 heads, T=2^31-3", hs, C, (int)n1, 512);
  }
  // 2000 heads over 500 ranges: heads straddle ranges, so partial slots are
  // taken at positions past 2^41.
  {
    const int C = 16;
    const int64_t n1 = T / C;
    std::vector<Head> hs(2000, Head{n1, 0, T});
    for (int h = 1; h < 2000; h += 3) hs[h].c = n1 - 1 - h, hs[h].first = 1;
    run_case("p=1 straddling, 2000 heads, T=2^31-3", hs, C, (int)n1, 500);
  }
  // 2048 heads at 2^20 tokens each, C = 32 (a 2048-head block at 1M with p = 1).
  {
    const int C = 32;
    const int64_t Tm = (int64_t)1 << 20;
    std::vector<Head> hs(kBalMaxHeads, Head{Tm / C, 0, Tm});
    run_case("p=1, 2048 heads, T=2^20", hs, C, (int)(Tm / C), 512);
  }
  // A mix: failed routes, overflowing counts, sink-only heads, causal lengths.
  {
    std::mt19937_64 g(7);
    const int C = 8;
    const int cap = (int)(T / C);
    std::vector<Head> hs;
    for (int h = 0; h < kBalMaxHeads; ++h) {
      const int k = (int)(g() % 6);
      const int64_t Th = k == 5 ? 1 + (int64_t)(g() % T) : T;
      const int64_t n1 = Th / C;
      Head x{0, 0, Th};
      if (k == 0) x.c = -1;                                     // failed route
      else if (k == 1) x.c = cap + 1;                           // more than cap: NaN row
      else if (k == 2) x.c = 0;                                 // sink and tail only
      else { x.c = n1 ? (int64_t)(g() % (n1 + 1)) : 0; x.first = (int32_t)(g() % 2); }
      if (x.c > 0 && x.c > n1) x.c = n1;
      hs.push_back(x);
    }
    run_case("mixed, 2048 heads", hs, C, cap, 512);
  }
  // Small calls: fewer positions than ranges (width clamps to the minimum).
  {
    std::vector<Head> hs(3, Head{2, 0, 100});
    run_case("3 small heads", hs, 16, 64, 512);
    std::vector<Head> one(1, Head{0, 0, 1});
    run_case("one token", one, 16, 64, 512);
  }
  std::printf(fails ? "FAILED\n" : "OK\n");
  return fails ? 1 : 0;
}
