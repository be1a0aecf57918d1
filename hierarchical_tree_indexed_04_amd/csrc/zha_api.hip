// C ABI: argument validation, buffer layouts and launches.  Every check runs
// on the host before any launch; nothing here allocates or synchronises.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "zha_internal.hpp"

using namespace zha;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geom(const zha_geom* g) {
  if (g == nullptr) return ZHA_ERR_NULL;
  if (g->dtype != ZHA_F32 && g->dtype != ZHA_BF16) return ZHA_ERR_DTYPE;
  if (g->d != 64 && g->d != 128 && g->d != 256) return ZHA_ERR_DIM;
  if (g->B < 1 || g->H_q < 1 || g->H_kv < 1 || g->H_q % g->H_kv != 0) return ZHA_ERR_GEOM;
  if (g->C < 2 || g->C > 1024 || g->L < 1 || g->L > kMaxLevels || g->R < 1 || g->R > 16)
    return ZHA_ERR_GEOM;
  if (g->T < 1 || g->T >= ((int64_t)1 << 31)) return ZHA_ERR_GEOM;
  if (g->T_cap != 0 && (g->T_cap < g->T || g->T_cap >= ((int64_t)1 << 31))) return ZHA_ERR_GEOM;
  if (g->kv_layout != ZHA_KV_SPLIT && g->kv_layout != ZHA_KV_CHUNKED) return ZHA_ERR_LAYOUT;
  return ZHA_OK;
}

// C^l, saturated past 2^40 (any span above 2^31 > T leaves its level empty).
int64_t next_span(int64_t span, int C) { return span > ((int64_t)1 << 40) ? span : span * C; }

// Token capacity: the strides of the KV cache, the tree and the build scratch.
int64_t capacity(const zha_geom* g) { return g->T_cap != 0 ? g->T_cap : g->T; }

TreeLayout make_layout(const zha_geom* g) {
  TreeLayout lay{};
  lay.L = g->L;
  lay.R = g->R;
  lay.C = g->C;
  const int64_t es = g->dtype == ZHA_BF16 ? 2 : 4;
  int64_t span = 1, off = 0;
  for (int l = 1; l <= g->L; ++l) {
    span = next_span(span, g->C);
    lay.n[l] = g->T / span;
    lay.ncap[l] = capacity(g) / span;
  }
  for (int l = 1; l <= g->L; ++l) {
    lay.khat[l] = off;
    off += align256(lay.ncap[l] * g->R * g->d * es);
  }
  for (int l = 1; l <= g->L; ++l) {
    lay.bhat[l] = off;
    off += align256(lay.ncap[l] * g->R * 4);
  }
  lay.stride = off;
  return lay;
}

BuildArgs make_build_args(const zha_geom* g) {
  BuildArgs a{};
  a.lay = make_layout(g);
  a.n_trees = g->B * g->H_kv;
  a.H_kv = g->H_kv;
  a.d = g->d;
  a.chunked = g->kv_layout == ZHA_KV_CHUNKED;
  a.T = g->T;
  a.Tc = capacity(g);
  return a;
}

// Rotated references: validates and copies the frequencies into the arguments.
int set_rope(const zha_geom* g, const zha_rope* rope, BuildArgs& a) {
  a.rope_dims = 0;
  if (rope == nullptr || rope->dims == 0) return ZHA_OK;
  if (rope->dims < 0 || (rope->dims & 1) || rope->dims > g->d || rope->reserved != 0 ||
      rope->theta == nullptr)
    return ZHA_ERR_ROPE;
  a.rope_dims = rope->dims;
  for (int k = 0; k < rope->dims / 2; ++k) a.theta[k] = rope->theta[k];
  return ZHA_OK;
}

int log2_or_neg(int C) { return (C & (C - 1)) == 0 ? __builtin_ctz((unsigned)C) : -1; }

// K and V pointers per layout: split needs both, chunked takes the KV buffer
// as K and no V.
int check_kv(const zha_geom* g, const void* K, const void* V) {
  if (K == nullptr) return ZHA_ERR_NULL;
  if (g->kv_layout == ZHA_KV_CHUNKED) return V == nullptr ? ZHA_OK : ZHA_ERR_LAYOUT;
  if (V == nullptr) return ZHA_ERR_NULL;
  return aligned16(V) ? ZHA_OK : ZHA_ERR_ALIGN;
}


// Splits per dense-decode unit (and tokens per split on the matrix-core path).
DensePlan dense_plan(const zha_geom* g, int32_t n_pos) {
  if (dense_mfma_eligible(g->dtype, g->d))
    return dense_mfma_plan((int64_t)g->B * g->H_kv, (int64_t)n_pos * (g->H_q / g->H_kv), g->T);
  const int64_t groups = (int64_t)g->B * n_pos * g->H_kv * (g->H_q / g->H_kv / dense_head_tile(g->H_q / g->H_kv));
  int64_t s = (4096 + groups - 1) / groups;
  const int64_t smax = (g->T + 255) / 256;
  if (s > smax) s = smax;
  if (s > 65535) s = 65535;
  if (s < 1) s = 1;
  return DensePlan{(int32_t)s, 0};
}

}  // namespace

extern "C" {

const char* zha_strerror(int code) {
  switch (code) {
    case ZHA_OK: return "success";
    case ZHA_ERR_NULL: return "a required pointer is NULL";
    case ZHA_ERR_GEOM: return "invalid geometry";
    case ZHA_ERR_DTYPE: return "unsupported dtype";
    case ZHA_ERR_DIM: return "unsupported head dimension";
    case ZHA_ERR_P: return "p must be in (0, 1]";
    case ZHA_ERR_ALIGN: return "buffer not 16-byte aligned";
    case ZHA_ERR_CAP: return "cap must be >= 1";
    case ZHA_ERR_LAUNCH: return "kernel launch failed";
    case ZHA_ERR_NPOS: return "n_pos must be >= 1";
    case ZHA_ERR_LAYOUT: return "unknown kv_layout, or V given with the chunked layout";
    case ZHA_ERR_ROPE: return "rope: dims must be even and in [0, d], with theta given";
    case ZHA_ERR_SCRATCH:
      return "the call needs more scratch than zha_attn_noalloc's fixed device buffer holds";
    default: return "unknown error";
  }
}

int zha_tree_bytes(const zha_geom* g, size_t* tree_bytes, size_t* build_scratch_bytes) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (tree_bytes == nullptr || build_scratch_bytes == nullptr) return ZHA_ERR_NULL;
  const BuildArgs a = make_build_args(g);
  *tree_bytes = (size_t)(a.lay.stride * a.n_trees);
  *build_scratch_bytes = (size_t)build_scratch_layout(a).total;
  return ZHA_OK;
}

int zha_tree_level_offset(const zha_geom* g, int32_t level, size_t* khat_offset,
                          size_t* bhat_offset, size_t* tree_stride) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (khat_offset == nullptr || bhat_offset == nullptr || tree_stride == nullptr)
    return ZHA_ERR_NULL;
  if (level < 1 || level > g->L) return ZHA_ERR_GEOM;
  const TreeLayout lay = make_layout(g);
  *khat_offset = (size_t)lay.khat[level];
  *bhat_offset = (size_t)lay.bhat[level];
  *tree_stride = (size_t)lay.stride;
  return ZHA_OK;
}

int zha_build(const zha_geom* g, const void* K, const float* qref, const zha_rope* rope,
              void* tree, void* scratch, void* stream) {
  const int rc = check_geom(g);
  if (rc) return rc;
  BuildArgs a = make_build_args(g);
  const int rr = set_rope(g, rope, a);
  if (rr) return rr;
  const bool need_scratch = build_scratch_layout(a).total > 0;
  if (K == nullptr || tree == nullptr || (need_scratch && scratch == nullptr))
    return ZHA_ERR_NULL;
  if (!aligned16(K) || (qref != nullptr && !aligned16(qref)) || !aligned16(tree) ||
      (need_scratch && !aligned16(scratch)))
    return ZHA_ERR_ALIGN;
  return build_dispatch(a, g->dtype, g->d, K, qref, tree, scratch,
                        reinterpret_cast<hipStream_t>(stream));
}

int zha_tree_update(const zha_geom* g, int64_t T_old, const void* K, const float* qref,
                    const zha_rope* rope, void* tree, void* scratch, void* stream) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (T_old < 0 || T_old > g->T) return ZHA_ERR_GEOM;
  BuildArgs a = make_build_args(g);
  const int rr = set_rope(g, rope, a);
  if (rr) return rr;
  int64_t span = 1;
  for (int l = 1; l <= g->L; ++l) {
    span = next_span(span, g->C);
    a.lo[l] = T_old / span;  // nodes already summarised at the old length
  }
  const bool need_scratch = build_scratch_layout(a).total > 0;
  if (K == nullptr || tree == nullptr || (need_scratch && scratch == nullptr))
    return ZHA_ERR_NULL;
  if (!aligned16(K) || (qref != nullptr && !aligned16(qref)) || !aligned16(tree) ||
      (need_scratch && !aligned16(scratch)))
    return ZHA_ERR_ALIGN;
  return build_dispatch(a, g->dtype, g->d, K, qref, tree, scratch,
                        reinterpret_cast<hipStream_t>(stream));
}

int32_t zha_route_frontier_capacity(void) { return kRouteFrontierMax; }

namespace {
// A level's cut sums one fixed-point mass of up to 2^kMassBits per candidate
// in 64 bits, so a frontier must stay below 2^(64 - kMassBits) candidates;
// the largest frontier is every level-1 node at capacity.
bool route_frontier_fits(const zha_geom* g) {
  return capacity(g) / g->C < ((int64_t)1 << (64 - kMassBits));
}

// Rounds of waiting for a device-memory frontier slot before a head gives up
// (cnt = ZHA_ROUTE_SLOT_BUSY).  ZHA_ROUTE_SPILL_WAIT overrides the default for
// diagnostics; a negative value gives up at once, as if every slot were held.
int32_t spill_wait_rounds() {
  const char* e = getenv("ZHA_ROUTE_SPILL_WAIT");
  if (e == nullptr || *e == 0) return kRouteSpillWaitRounds;
  const long v = strtol(e, nullptr, 10);
  return v < 0 ? -1 : (v > INT32_MAX ? INT32_MAX : (int32_t)v);
}
}  // namespace

int zha_route_scratch_bytes(const zha_geom* g, int32_t n_pos, int32_t cap, size_t* bytes) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (bytes == nullptr) return ZHA_ERR_NULL;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  if (cap < 1) return ZHA_ERR_CAP;
  if (!route_frontier_fits(g)) return ZHA_ERR_GEOM;
  *bytes = (size_t)route_scratch_layout((int64_t)g->B * n_pos * g->H_q, capacity(g) / g->C).bytes;
  return ZHA_OK;
}

}  // extern "C"

namespace {
// Validation and arguments of a route call.
int prepare_route(const zha_geom* g, const void* tree, const void* Q, int32_t n_pos,
                  const int32_t* ctx_len, float p, int32_t* sel, int32_t* cnt, int32_t cap,
                  RouteArgs& a) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (tree == nullptr || Q == nullptr || sel == nullptr || cnt == nullptr) return ZHA_ERR_NULL;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  if (cap < 1) return ZHA_ERR_CAP;
  if (!(p > 0.0f && p <= 1.0f)) return ZHA_ERR_P;
  if (!route_frontier_fits(g)) return ZHA_ERR_GEOM;
  if (!aligned16(tree) || !aligned16(Q)) return ZHA_ERR_ALIGN;
  a = RouteArgs{};
  a.lay = make_layout(g);
  a.T = g->T;
  a.ctx = ctx_len;
  a.span[0] = 1;
  for (int l = 1; l <= g->L; ++l) a.span[l] = next_span(a.span[l - 1], g->C);
  a.n_heads = (int64_t)g->B * n_pos * g->H_q;
  a.n_pos = n_pos;
  a.H_q = g->H_q;
  a.H_kv = g->H_kv;
  a.G = g->H_q / g->H_kv;
  a.cap = cap;
  a.p = p;
  a.cdiv = (uint32_t)(((1ull << 32) + (uint64_t)g->C - 1) / (uint64_t)g->C);
  a.spill_wait = spill_wait_rounds();
  if (a.n_heads > INT32_MAX) return ZHA_ERR_GEOM;
  return ZHA_OK;
}
}  // namespace

extern "C" {

int zha_route(const zha_geom* g, const void* tree, const void* Q, int32_t n_pos,
              const int32_t* ctx_len, float p,
              int32_t* sel, int32_t* cnt, int32_t cap, int32_t* level_stats, float* gap,
              void* scratch, void* stream) {
  RouteArgs a;
  const int rc = prepare_route(g, tree, Q, n_pos, ctx_len, p, sel, cnt, cap, a);
  if (rc) return rc;
  const RouteScratch rs = route_scratch_layout(a.n_heads, a.lay.ncap[1]);
  if (rs.bytes > 0 && scratch == nullptr) return ZHA_ERR_NULL;
  if (rs.bytes > 0 && !aligned16(scratch)) return ZHA_ERR_ALIGN;
  return route_dispatch(a, g->dtype, g->d, tree, Q, sel, cnt, level_stats, gap, scratch,
                        reinterpret_cast<hipStream_t>(stream));
}

int zha_attn_scratch_bytes(const zha_geom* g, int32_t n_pos, int32_t cap, size_t* bytes) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (bytes == nullptr) return ZHA_ERR_NULL;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  if (cap < 1) return ZHA_ERR_CAP;
  const int64_t n_heads = (int64_t)g->B * n_pos * g->H_q;
  *bytes = (size_t)attn_scratch_layout_bytes(n_heads, (int64_t)g->B * g->H_kv, g->T, g->C, g->d,
                                             g->dtype);
  return ZHA_OK;
}

}  // extern "C"

namespace {
// Validation and arguments shared by zha_attn and zha_attn_noalloc; *need is
// the scratch the call's launches use.
int prepare_attn(const zha_geom* g, const void* Q, int32_t n_pos, const int32_t* ctx_len,
                 const void* K, const void* V, const int32_t* sel, const int32_t* cnt,
                 int32_t cap, void* O, AttnArgs& a, int64_t* need) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  if (cap < 1) return ZHA_ERR_CAP;
  a = AttnArgs{};
  a.T = g->T;
  a.Tc = capacity(g);
  a.ctx = ctx_len;
  a.n_heads = (int64_t)g->B * n_pos * g->H_q;
  a.n1 = g->T / g->C;
  a.n_pos = n_pos;
  a.H_q = g->H_q;
  a.H_kv = g->H_kv;
  a.G = g->H_q / g->H_kv;
  a.C = g->C;
  a.log2C = log2_or_neg(g->C);
  a.cap = cap;
  a.S = ZHA_ATTN_BLOCKS;
  a.chunked = g->kv_layout == ZHA_KV_CHUNKED;
  a.dtype = g->dtype;
  *need = attn_scratch_layout_bytes(a.n_heads, (int64_t)g->B * g->H_kv, g->T, g->C, g->d,
                                    g->dtype);
  const int kv = check_kv(g, K, V);
  if (kv) return kv;
  if (Q == nullptr || sel == nullptr || cnt == nullptr || O == nullptr) return ZHA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(O)) return ZHA_ERR_ALIGN;
  if (a.n_heads > INT32_MAX) return ZHA_ERR_GEOM;
  return ZHA_OK;
}
}  // namespace

// The fixed scratch of zha_attn_noalloc.  In host code `scratch` names a host
// stand-in, not the device array: its device address (one per device, each
// device holding its own copy) comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is ever passed on.
static __device__ __align__(256) char scratch[ZHA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call there, then kept).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ZHA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ZHA_ERR_LAUNCH;
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return ZHA_OK;
}
}  // namespace

extern "C" {

int zha_attn(const zha_geom* g, const void* Q, int32_t n_pos, const int32_t* ctx_len,
             const void* K, const void* V,
             const int32_t* sel, const int32_t* cnt, int32_t cap, void* O, void* scratch,
             void* stream) {
  AttnArgs a;
  int64_t need = 0;
  const int rc = prepare_attn(g, Q, n_pos, ctx_len, K, V, sel, cnt, cap, O, a, &need);
  if (rc) return rc;
  if (need > 0 && scratch == nullptr) return ZHA_ERR_NULL;
  if (need > 0 && !aligned16(scratch)) return ZHA_ERR_ALIGN;
  return attn_dispatch(a, g->dtype, g->d, Q, K, V, sel, cnt, O, scratch,
                       reinterpret_cast<hipStream_t>(stream));
}

int zha_attn_noalloc(const zha_geom* g, const void* Q, int32_t n_pos, const int32_t* ctx_len,
                     const void* K, const void* V, const int32_t* sel, const int32_t* cnt,
                     int32_t cap, void* O, void* stream) {
  AttnArgs a;
  int64_t need = 0;
  const int rc = prepare_attn(g, Q, n_pos, ctx_len, K, V, sel, cnt, cap, O, a, &need);
  if (rc) return rc;
  if (need > (int64_t)ZHA_NOALLOC_SCRATCH_BYTES) return ZHA_ERR_SCRATCH;
  void* buf = nullptr;
  if (need > 0) {
    const int sr = noalloc_scratch(&buf);
    if (sr) return sr;
  }
  return attn_dispatch(a, g->dtype, g->d, Q, K, V, sel, cnt, O, buf,
                       reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {
// zha_route_attn scratch: zha_route's, then either the fused launch's partials
// or zha_attn's scratch (whichever is larger).
struct RouteAttnScratch {
  int64_t route, attn, total;
};
RouteAttnScratch route_attn_layout(const zha_geom* g, int64_t n_heads) {
  RouteAttnScratch l{};
  l.route = align256(route_scratch_layout(n_heads, capacity(g) / g->C).bytes);
  const int64_t fused = n_heads <= kFzMaxHeads ? n_heads * kFzMaxPieces * (int64_t)(g->d + 2) * 4 : 0;
  const int64_t attn = attn_scratch_layout_bytes(n_heads, (int64_t)g->B * g->H_kv, g->T, g->C, g->d,
                                                 g->dtype);
  l.attn = align256(fused > attn ? fused : attn);
  l.total = l.route + l.attn;
  return l;
}
}  // namespace

extern "C" {

int zha_route_attn_scratch_bytes(const zha_geom* g, int32_t n_pos, int32_t cap, size_t* bytes) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (bytes == nullptr) return ZHA_ERR_NULL;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  if (cap < 1) return ZHA_ERR_CAP;
  if (!route_frontier_fits(g)) return ZHA_ERR_GEOM;
  *bytes = (size_t)route_attn_layout(g, (int64_t)g->B * n_pos * g->H_q).total;
  return ZHA_OK;
}

int zha_route_attn(const zha_geom* g, const void* tree, const void* Q, int32_t n_pos,
                   const int32_t* ctx_len, float p, const void* K, const void* V, int32_t* sel,
                   int32_t* cnt, int32_t cap, int32_t* level_stats, float* gap, void* O,
                   void* scratch, void* stream) {
  RouteArgs ra;
  int rc = prepare_route(g, tree, Q, n_pos, ctx_len, p, sel, cnt, cap, ra);
  if (rc) return rc;
  AttnArgs aa;
  int64_t need_attn = 0;
  rc = prepare_attn(g, Q, n_pos, ctx_len, K, V, sel, cnt, cap, O, aa, &need_attn);
  if (rc) return rc;
  const RouteAttnScratch l = route_attn_layout(g, ra.n_heads);
  if (l.total > 0 && scratch == nullptr) return ZHA_ERR_NULL;
  if (l.total > 0 && !aligned16(scratch)) return ZHA_ERR_ALIGN;
  char* scr = reinterpret_cast<char*>(scratch);
  char* ascr = l.attn > 0 ? scr + l.route : nullptr;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t kv_bytes = kv_block_elems(aa.Tc, g->C, g->d, aa.chunked) *
                           (g->dtype == ZHA_BF16 ? 2 : 4);
  if (fused_eligible(ra.n_heads, g->R, g->C, p, kv_bytes)) {
    const RouteScratch rs = route_scratch_layout(ra.n_heads, ra.lay.ncap[1]);
    char* ws = rs.ws < 0 ? nullptr : scr + rs.ws;
    // A nonzero tag, different for consecutive calls (the launch's queue items
    // and piece counters carry it).
    static std::atomic<uint32_t> g_tag{0};
    uint32_t tag = ++g_tag;
    if (tag == 0) tag = ++g_tag;
    return fused_dispatch(ra, aa, g->dtype, g->d, tree, Q, K, V, sel, cnt, level_stats, gap, O, ws,
                          rs.ws_stride, reinterpret_cast<float*>(ascr), kFzGrid, tag, s);
  }
  rc = route_dispatch(ra, g->dtype, g->d, tree, Q, sel, cnt, level_stats, gap, scratch, s);
  if (rc) return rc;
  return attn_dispatch(aa, g->dtype, g->d, Q, K, V, sel, cnt, O, ascr, s);
}

int zha_dense_decode_scratch_bytes(const zha_geom* g, int32_t n_pos, size_t* bytes) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (bytes == nullptr) return ZHA_ERR_NULL;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  const int64_t n_heads = (int64_t)g->B * n_pos * g->H_q;
  *bytes = (size_t)splitkv_scratch_bytes(n_heads, dense_plan(g, n_pos).S, g->d);
  return ZHA_OK;
}

int zha_dense_decode(const zha_geom* g, const void* Q, int32_t n_pos, const void* K,
                     const void* V, void* O, void* scratch, void* stream) {
  const int rc = check_geom(g);
  if (rc) return rc;
  if (n_pos < 1) return ZHA_ERR_NPOS;
  DenseArgs a{};
  a.T = g->T;
  a.Tc = capacity(g);
  a.n_heads = (int64_t)g->B * n_pos * g->H_q;
  a.n_pos = n_pos;
  a.H_q = g->H_q;
  a.H_kv = g->H_kv;
  a.G = g->H_q / g->H_kv;
  const DensePlan plan = dense_plan(g, n_pos);
  a.S = plan.S;
  a.tps = plan.tps;
  a.C = g->C;
  a.log2C = log2_or_neg(g->C);
  a.chunked = g->kv_layout == ZHA_KV_CHUNKED;
  const int kv = check_kv(g, K, V);
  if (kv) return kv;
  if (Q == nullptr || O == nullptr || (a.S > 1 && scratch == nullptr)) return ZHA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(O) || (a.S > 1 && !aligned16(scratch)))
    return ZHA_ERR_ALIGN;
  if (a.n_heads > INT32_MAX) return ZHA_ERR_GEOM;
  return dense_dispatch(a, g->dtype, g->d, Q, K, V, O, scratch,
                        reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
