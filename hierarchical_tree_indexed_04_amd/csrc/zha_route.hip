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
// One workgroup per query head walks all levels in one launch.  The
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

#ifndef ZHA_ROUTE_XCD
#define ZHA_ROUTE_XCD 1
#endif
#ifndef ZHA_ROUTE_PROFILE
#define ZHA_ROUTE_PROFILE 0
#endif
constexpr int kMaxChildren = 1024;  // C <= 1024

// Device-memory frontier slots in use (1) or free (0): zero when the code
// object loads, and every holder frees its slot before its kernel ends.
__device__ int32_t g_route_spill_lock[kRouteSpillBlocks];

// Launch shapes of the same kernel body.  Latency shape: 8 waves, 16 rows in
// flight per lane, frontiers up to kRouteFrontierMax; one workgroup per CU, so
// a call with few query heads finishes as fast as one head walks the tree.
// Throughput shape: ZHA_ROUTE_TPUT_THREADS threads (one wave: no barrier
// between waves, no work repeated per wave), ZHA_ROUTE_TPUT_ROWS 16-byte loads
// in flight per lane, frontiers up to ZHA_ROUTE_TPUT_FMAX in LDS; many
// workgroups share a CU, for calls with many query heads (a block of
// positions), so more heads are in flight (measured on the 1M block: 241 us
// against 255 us with two waves and 768 candidates; causal prefill at 128K:
// 23.2 against 27.3 ms of routing).  A head whose frontier outgrows the
// throughput shape is listed in the scratch buffer and routed again by
// persistent workgroups with the latency shape's frontier capacity (4 waves
// each, two per CU).  A head that outgrows that frontier as well (trees with
// more than kRouteFrontierMax level-1 nodes) is routed again by the same
// workgroup with its frontier in device memory, in one of kRouteSpillBlocks
// slots of n_1 candidates in the scratch buffer: routes never fail for size.
#ifndef ZHA_ROUTE_LAT_ROWS
#define ZHA_ROUTE_LAT_ROWS 8  // 256K decode route call: 16 -> 23.4, 8 -> 22.9 us
#endif
#ifndef ZHA_ROUTE_LIST_ROWS
#define ZHA_ROUTE_LIST_ROWS 16
#endif
#ifndef ZHA_ROUTE_TPUT_ROWS
#define ZHA_ROUTE_TPUT_ROWS 8
#endif
#ifndef ZHA_ROUTE_TPUT_THREADS
#define ZHA_ROUTE_TPUT_THREADS 64
#endif
#ifndef ZHA_ROUTE_TPUT_FMAX
#define ZHA_ROUTE_TPUT_FMAX 512
#endif
#ifndef ZHA_ROUTE_TPUT_EU
#define ZHA_ROUTE_TPUT_EU 1
#endif
#ifndef ZHA_ROUTE_LAT_THREADS
#define ZHA_ROUTE_LAT_THREADS 512
#endif
namespace lat {
constexpr int kThreads = ZHA_ROUTE_LAT_THREADS;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = ZHA_ROUTE_LAT_ROWS;
constexpr int kFMax = kRouteFrontierMax;
constexpr int kMinWavesEU = 1;
constexpr bool kSpillInPlace = true;
#include "zha_route_impl.inc"
}  // namespace lat
namespace tput {
constexpr int kThreads = ZHA_ROUTE_TPUT_THREADS;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = ZHA_ROUTE_TPUT_ROWS;
constexpr int kFMax = ZHA_ROUTE_TPUT_FMAX;
constexpr int kMinWavesEU = ZHA_ROUTE_TPUT_EU;
constexpr bool kSpillInPlace = false;  // overflowing heads are listed for the latency shape
#include "zha_route_impl.inc"
}  // namespace tput
// Re-routing shape for the heads the throughput shape lists: the latency
// shape's frontier capacity with 4 waves, so two workgroups share a CU and
// twice as many listed heads are in flight (1M block: 265 listed heads, list
// pass 33 -> ~24 us).
namespace lst {
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = ZHA_ROUTE_LIST_ROWS;
constexpr int kFMax = kRouteFrontierMax;
constexpr int kMinWavesEU = 1;
constexpr bool kSpillInPlace = true;
#include "zha_route_impl.inc"
}  // namespace lst
// kTputMinHeads (query heads per call for the throughput shape) is in zha_internal.hpp.
constexpr unsigned kRouteListBlocks = 512;  // persistent workgroups for the listed heads (2 per CU)

// p >= 1 keeps every candidate at every level, so S_l is all of level l and
// S_1 is every leaf chunk 0 .. n_1 - 1 (orphans included).
__global__ __launch_bounds__(256) void route_keep_all_kernel(RouteArgs a,
                                                                  int32_t* __restrict__ sel,
                                                                  int32_t* __restrict__ cnt,
                                                                  int32_t* __restrict__ stats,
                                                                  float* __restrict__ gapo) {
  const int64_t head = blockIdx.x;
  const int64_t Th = visible_len(a, head);
  if (Th < 0) {  // invalid visible length: a failed route
    if (threadIdx.x == 0) cnt[head] = -1;
    return;
  }
  auto n_at = [&](int l) -> int64_t { return a.ctx == nullptr ? a.lay.n[l] : Th / a.span[l]; };
  const int64_t n1 = n_at(1);
  const int64_t lim = n1 < a.cap ? n1 : a.cap;
  for (int64_t j = threadIdx.x; j < lim; j += blockDim.x) sel[head * a.cap + j] = (int32_t)j;
  if (threadIdx.x < a.lay.L) {
    const int l = threadIdx.x + 1;
    const int64_t o = head * a.lay.L + (l - 1);
    if (stats != nullptr) {
      stats[2 * o] = (int32_t)n_at(l);
      stats[2 * o + 1] = (int32_t)n_at(l);
    }
    if (gapo != nullptr) gapo[o] = INFINITY;
  }
  if (threadIdx.x == 0) cnt[head] = (int32_t)n1;
}

__global__ void route_zero_kernel(int32_t* list) {
  if (threadIdx.x == 0) list[0] = 0;
}

// Launch sequence.  Many heads: the throughput shape, then the latency shape
// on the heads it listed.  Few heads: the latency shape alone.  The latency
// shape routes a head that outgrows its LDS again in place, with a
// device-memory frontier (trees whose level 1 can outgrow the LDS).
template <typename T, int D, bool R1>
void launch_route_kernels(const RouteArgs& a, const char* tree, const T* q, int32_t* sel,
                          int32_t* cnt, int32_t* stats, float* gap, char* scratch,
                          hipStream_t s) {
  const RouteScratch rs = route_scratch_layout(a.n_heads, a.lay.ncap[1]);
  int32_t* list1 = rs.list1 < 0 ? nullptr : reinterpret_cast<int32_t*>(scratch + rs.list1);
  char* ws = rs.ws < 0 ? nullptr : scratch + rs.ws;
  const unsigned blocks = (unsigned)a.n_heads;
  if (a.n_heads >= kTputMinHeads) {
    route_zero_kernel<<<1, 64, 0, s>>>(list1);
    tput::route_kernel<T, D, tput::kFMax, R1><<<blocks, tput::kThreads, 0, s>>>(
        tree, q, a, sel, cnt, stats, gap, list1, nullptr, 0);
    lst::route_list_kernel<T, D, lst::kFMax, R1><<<kRouteListBlocks, lst::kThreads, 0, s>>>(
        tree, q, a, sel, cnt, stats, gap, list1, ws, rs.ws_stride);
  } else {
    lat::route_kernel<T, D, lat::kFMax, R1><<<blocks, lat::kThreads, 0, s>>>(
        tree, q, a, sel, cnt, stats, gap, nullptr, ws, rs.ws_stride);
  }
}

template <typename T, int D>
int launch_route(const RouteArgs& a, const void* tree, const void* Q, int32_t* sel, int32_t* cnt,
                 int32_t* stats, float* gap, void* scratch, hipStream_t s) {
  const char* tr = reinterpret_cast<const char*>(tree);
  const T* q = reinterpret_cast<const T*>(Q);
  char* sc = reinterpret_cast<char*>(scratch);
  if (!(a.p < 1.0f))
    route_keep_all_kernel<<<(unsigned)a.n_heads, 256, 0, s>>>(a, sel, cnt, stats, gap);
  else if (a.lay.R == 1)
    launch_route_kernels<T, D, true>(a, tr, q, sel, cnt, stats, gap, sc, s);
  else
    launch_route_kernels<T, D, false>(a, tr, q, sel, cnt, stats, gap, sc, s);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

}  // namespace

int route_dispatch(const RouteArgs& a, int dtype, int d, const void* tree, const void* Q,
                   int32_t* sel, int32_t* cnt, int32_t* stats, float* gap, void* scratch,
                   hipStream_t s) {
#define ZHA_ROUTE_CASE(TT, DD) \
  if (d == DD) return launch_route<TT, DD>(a, tree, Q, sel, cnt, stats, gap, scratch, s);
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
