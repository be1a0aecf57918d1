// Routing and sparse attention in one launch (the paper's App. D kernel
// inventory lists a "fusion" kernel beside routing and attention).
//
// zha_route followed by zha_attn serialises three launches: the router's
// duration is its slowest head (its levels are dependent memory round trips),
// attention can start only when every head is routed, and the split partials
// are merged by a launch of their own.  Here one persistent launch does all:
//
//   1. Routing.  Workgroups claim query heads one at a time (a device counter)
//      and route each with the router of zha_route (its 8-wave shape, the
//      4096-candidate frontier in LDS, device-memory frontier past it).
//   2. Publishing.  A routed head's attended tokens (the sink, its chunks'
//      tokens, the partial chunk) are cut into np pieces of about
//      kFzPieceTokens; the head's descriptor and then np queue items go to
//      device memory.
//   3. Attention.  A workgroup with no head left to claim takes queue items in
//      order and attends one piece each (attend_segment, the balanced split's
//      code), writing a partial; the piece that completes a head (a per-head
//      counter) merges its partials in piece order.  A head of one piece is
//      written directly.
//
// So a head's attention starts as soon as its route ends, while other heads
// are still being routed, and no launch waits for the slowest head.
//
// Data that crosses workgroups within the launch (chunk lists, descriptors,
// queue items, partials) is written with device-coherent stores, completed
// (s_waitcnt vmcnt(0)) before the item or counter that announces it, and read
// with device-coherent loads; no cache-wide fence is used.  Every wait is
// bounded.  No deadlock: a workgroup waits only for items of heads already
// claimed, and a head is claimed only by a running workgroup.
//
// The queue, counters and descriptors are device globals of the library: zero
// when the code object loads, each item cleared by its consumer, each head's
// counter by its merger, and the counters by the last workgroup to finish, so
// every call starts from zero.  Calls that overlap in time on one device race.

#include "zha_attn_impl.hpp"

namespace zha {
namespace {

#ifndef ZHA_ROUTE_XCD
#define ZHA_ROUTE_XCD 1
#endif
#ifndef ZHA_ROUTE_PROFILE
#define ZHA_ROUTE_PROFILE 0
#endif
constexpr int kMaxChildren = 1024;  // C <= 1024

// Device-memory frontier slots of this file's router (in use: 1).
__device__ int32_t g_route_spill_lock[kRouteSpillBlocks];

// The router in the 8-wave shape of zha_route's latency launch; the
// attention of a piece uses the same 512 threads.
constexpr int kFzThreads = 512;
namespace fz {
constexpr int kThreads = kFzThreads;
constexpr int kWaves = kThreads / kWave;
constexpr int kU = 8;
constexpr int kFMax = kRouteFrontierMax;
constexpr int kMinWavesEU = 1;
constexpr bool kSpillInPlace = true;
#include "zha_route_impl.inc"
}  // namespace fz

// Control state of the fused launch.
struct FzCtl {
  int32_t route_next;  // next query head to claim for routing
  int32_t tail;        // queue items reserved
  int32_t piece_next;  // next queue item to take
  int32_t routed;      // heads routed and published
  int32_t exited;      // workgroups done
  int32_t timeout;     // a bounded wait ran out (sticky, for diagnostics)
};
struct FzHead {
  int32_t base;  // first queue item (and partial slot) of the head
  int32_t np;    // pieces
  int32_t ntok;  // attended tokens
  int32_t c;     // selected chunks (as routed)
  int64_t Th;    // tokens the head sees
};
// Queue items and per-head piece counters carry the call's tag (a nonzero
// number from the host, different for consecutive calls) in their high 32
// bits, so an entry a call did not write is never taken for one of its own.
__device__ FzCtl g_fz;
__device__ uint64_t g_fz_done[kFzMaxHeads];                 // tag << 32 | pieces done
__device__ FzHead g_fz_head[kFzMaxHeads];
__device__ uint64_t g_fz_item[kFzMaxHeads * kFzMaxPieces];  // tag << 32 | head << 16 | piece

constexpr int kFzSpins = 1 << 22;  // polls of one wait before it gives up (seconds)

template <typename TT>
__device__ __forceinline__ void st_coh(TT* p, TT v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename TT>
__device__ __forceinline__ TT ld_coh(const TT* p) {
  return __hip_atomic_load(const_cast<TT*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This thread's stores are complete at device scope.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <typename T, int D>
union FzSmem {
  fz::RouteSmem<fz::kFMax> route;
  SegSmem<T, D, kFzThreads> seg;
};

template <typename T, int D, bool POW2>
__global__ __launch_bounds__(kFzThreads) void route_attn_kernel(
    const char* __restrict__ tree, const T* __restrict__ Q, const T* __restrict__ K,
    const T* __restrict__ V, RouteArgs ra, AttnArgs aa, int32_t* __restrict__ sel,
    int32_t* __restrict__ cnt, int32_t* __restrict__ stats, float* __restrict__ gap,
    T* __restrict__ O, char* __restrict__ ws, int64_t ws_stride, float* __restrict__ part,
    uint32_t tag) {
  __shared__ FzSmem<T, D> sm;
  __shared__ int64_t s_word;
  const int tid = threadIdx.x;
  const int nh = (int)ra.n_heads;
  const int cap = aa.cap;

  // 1-2. Route heads while any is left to claim, publishing each.
  for (;;) {
    if (tid == 0) s_word = atomicAdd(&g_fz.route_next, 1);
    __syncthreads();
    const int h = (int)s_word;
    __syncthreads();  // s_word is reused
    if (h >= nh) break;
    const bool ovf = fz::route_one_head<T, D, fz::kFMax, true>(sm.route, tree, Q, ra, sel, cnt,
                                                                stats, gap, h);
    if (ovf && ws != nullptr) {
      __syncthreads();  // sm is reused
      fz::route_spilled<T, D, fz::kFMax, true>(sm.route, tree, Q, ra, sel, cnt, stats, gap, h, ws,
                                               ws_stride);
    }
    __syncthreads();  // the route's writes are done (and visible to this workgroup)
    const int c = cnt[h];
    const int64_t Th = visible_len(aa, h);
    const bool ok = c >= 0 && c <= cap && Th >= 0;
    const int64_t ntok = ok ? bal_head_tokens(c, c > 0 ? sel[(int64_t)h * cap] : 0, Th, aa.C, cap)
                            : 0;
    int np = 0;
    if (ntok > 0) {
      const int64_t want = (ntok + kFzPieceTokens - 1) / kFzPieceTokens;
      np = (int)min(want, (int64_t)kFzMaxPieces);
      // The chunk list, written by the router with plain stores, again with
      // device-coherent ones for the workgroups that attend the pieces.
      int32_t* ids = sel + (int64_t)h * cap;
      for (int j = tid; j < c; j += kFzThreads) st_coh(ids + j, ids[j]);
    } else {
      // A failed or overflowed route attends nothing: its row is NaN.
      for (int t = tid; t < D; t += kFzThreads)
        store_elem(O + (int64_t)h * D, t, __int_as_float(0x7fc00000));
    }
    if (tid == 0) {
      const int base = np > 0 ? atomicAdd(&g_fz.tail, np) : 0;
      st_coh(&g_fz_head[h].base, base);
      st_coh(&g_fz_head[h].np, np);
      st_coh(&g_fz_head[h].ntok, (int32_t)ntok);
      st_coh(&g_fz_head[h].c, c);
      st_coh(&g_fz_head[h].Th, Th);
      s_word = base;
    }
    wait_stores();
    __syncthreads();
    const int base = (int)s_word;
    for (int k = tid; k < np; k += kFzThreads)
      st_coh(&g_fz_item[base + k], ((uint64_t)tag << 32) | ((uint64_t)h << 16) | (uint32_t)k);
    wait_stores();
    __syncthreads();
    if (tid == 0) atomicAdd(&g_fz.routed, 1);
    __syncthreads();  // s_word is reused
  }

  // 3. Attend queue items until every head is published and every item taken.
  const int64_t n_items = (int64_t)kFzMaxHeads * kFzMaxPieces;
  for (;;) {
    if (tid == 0) {
      const int i = atomicAdd(&g_fz.piece_next, 1);
      uint64_t it = 0;
      for (int spin = 0;; ++spin) {
        if (i < n_items) {
          it = ld_coh(&g_fz_item[i]);
          if ((uint32_t)(it >> 32) == tag) {
            st_coh(&g_fz_item[i], (uint64_t)0);  // taken: clear for the next call
            break;
          }
          it = 0;
        }
        // No item yet: the end, once every head is published and i is past
        // the last reserved item (every reservation precedes its head's count).
        if (ld_coh(&g_fz.routed) >= nh && i >= ld_coh(&g_fz.tail)) break;
        if (spin >= kFzSpins) {
          st_coh(&g_fz.timeout, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      s_word = (int64_t)it;
    }
    __syncthreads();
    const uint64_t it = (uint64_t)s_word;
    __syncthreads();  // s_word is reused
    if (it == 0) break;
    const int h = (int)((it >> 16) & 0xffffu);
    const int k = (int)(it & 0xffffu);
    if (h >= nh) continue;  // cannot happen for an item of this call
    const int base = ld_coh(&g_fz_head[h].base);
    const int np = ld_coh(&g_fz_head[h].np);
    const int ntok = ld_coh(&g_fz_head[h].ntok);
    const int c = ld_coh(&g_fz_head[h].c);
    const int64_t Th = ld_coh(&g_fz_head[h].Th);
    if (np < 1 || np > kFzMaxPieces || k >= np || base < 0 ||
        (int64_t)base + np > (int64_t)nh * kFzMaxPieces || c < 0 || c > cap)
      continue;  // likewise: a descriptor this call did not write
    const int P = (ntok + np - 1) / np;
    const int x0 = k * P, x1 = min(ntok, x0 + P);
    float* prow = np > 1 ? part + (int64_t)(base + k) * (D + 2) : nullptr;
    attend_segment<T, D, POW2, true, true, kFzThreads>(Q, K, V, sel + (int64_t)h * cap, c, Th, aa,
                                                       h, x0, x1, O + (int64_t)h * D, prow,
                                                       sm.seg);
    if (np > 1) {
      wait_stores();
      __syncthreads();
      if (tid == 0) {
        // Count this piece under the call's tag (an older tag counts as 0).
        uint64_t old = ld_coh(&g_fz_done[h]);
        for (;;) {
          const uint64_t n = (uint32_t)(old >> 32) == tag ? old + 1 : ((uint64_t)tag << 32) | 1u;
          if (__hip_atomic_compare_exchange_strong(&g_fz_done[h], &old, n, __ATOMIC_RELAXED,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            break;
        }
        s_word = (uint32_t)(old >> 32) == tag ? (int64_t)(uint32_t)old : 0;
      }
      __syncthreads();
      const bool last = s_word == np - 1;
      __syncthreads();  // s_word is reused
      if (last) {  // every other piece's partial is complete: merge in piece order
        if (tid == 0) st_coh(&g_fz_done[h], (uint64_t)0);
        merge_partials<T, D, true, kFzThreads>(part + (int64_t)base * (D + 2), np,
                                               O + (int64_t)h * D);
        __syncthreads();
      }
    }
  }

  // The last workgroup out clears the counters for the next call.
  if (tid == 0) {
    if (atomicAdd(&g_fz.exited, 1) == (int)gridDim.x - 1) {
      st_coh(&g_fz.route_next, 0);
      st_coh(&g_fz.tail, 0);
      st_coh(&g_fz.piece_next, 0);
      st_coh(&g_fz.routed, 0);
      st_coh(&g_fz.exited, 0);
    }
  }
}

template <typename T, int D>
int launch_fused(const RouteArgs& ra, const AttnArgs& aa, const void* tree, const void* Q,
                 const void* K, const void* V, int32_t* sel, int32_t* cnt, int32_t* stats,
                 float* gap, void* O, char* ws, int64_t ws_stride, float* part, unsigned grid,
                 uint32_t tag, hipStream_t s) {
  const char* tr = reinterpret_cast<const char*>(tree);
  const T* q = reinterpret_cast<const T*>(Q);
  const T* k = reinterpret_cast<const T*>(K);
  const T* v = reinterpret_cast<const T*>(V);
  T* o = reinterpret_cast<T*>(O);
  if (aa.log2C >= 0)
    route_attn_kernel<T, D, true><<<grid, kFzThreads, 0, s>>>(tr, q, k, v, ra, aa, sel, cnt, stats,
                                                            gap, o, ws, ws_stride, part, tag);
  else
    route_attn_kernel<T, D, false><<<grid, kFzThreads, 0, s>>>(tr, q, k, v, ra, aa, sel, cnt, stats,
                                                             gap, o, ws, ws_stride, part, tag);
  return hipGetLastError() == hipSuccess ? ZHA_OK : ZHA_ERR_LAUNCH;
}

}  // namespace

int fused_dispatch(const RouteArgs& ra, const AttnArgs& aa, int dtype, int d, const void* tree,
                   const void* Q, const void* K, const void* V, int32_t* sel, int32_t* cnt,
                   int32_t* stats, float* gap, void* O, char* ws, int64_t ws_stride, float* part,
                   unsigned grid, uint32_t tag, hipStream_t s) {
#define ZHA_FUSED_CASE(TT, DD)                                                                \
  if (d == DD)                                                                                \
    return launch_fused<TT, DD>(ra, aa, tree, Q, K, V, sel, cnt, stats, gap, O, ws, ws_stride, \
                                part, grid, tag, s);
  if (dtype == ZHA_BF16) {
    ZHA_FUSED_CASE(bf16_t, 64)
    ZHA_FUSED_CASE(bf16_t, 128)
    ZHA_FUSED_CASE(bf16_t, 256)
  } else {
    ZHA_FUSED_CASE(float, 64)
    ZHA_FUSED_CASE(float, 128)
    ZHA_FUSED_CASE(float, 256)
  }
#undef ZHA_FUSED_CASE
  return ZHA_ERR_DIM;
}

}  // namespace zha
