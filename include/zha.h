/*
 * zha.h - C ABI of the ZHA hot-path library for AMD Instinct MI355X (gfx950).
 *
 * Zyphra Hierarchical Attention ("Subquadratic Attention with a Hierarchical
 * Tree-Structured Indexer") replaces dense decode attention by three steps,
 * each one entry point here:
 *
 *   zha_build         tree of recursively compressed key summaries over a KV
 *                     cache (paper §III-A "Tree Construction", App. D-B2);
 *   zha_route         top-down routing of every query head through its KV
 *                     head's tree, keeping at each level the smallest top-p
 *                     set of the frontier (paper §III-C; the summary page's
 *                     "Routing": m_ell(q) and the final index set I(q));
 *   zha_attn          exact softmax attention over the surviving tokens,
 *                     o(q) = Attn(q, K_I(q), V_I(q)) (summary page "Routing").
 *
 * plus zha_dense_decode, full attention over every cached key, the baseline
 * the sparse path is measured against (paper App. D-A, dense decode model).
 *
 * Conventions for every call
 * --------------------------
 * - Pointers named as device buffers must be device memory (or memory mapped
 *   for the device); the caller owns every buffer.  The library never
 *   allocates, never synchronises, and keeps no state between calls.  Calls
 *   are asynchronous on `stream` (a hipStream_t; NULL is the null stream).
 * - Return value 0 is success.  A negative value is an error detected on the
 *   host before anything is launched (ZHA_ERR_*); nothing has been written.
 *   zha_strerror() names it.  ZHA_ERR_LAUNCH reports a failed kernel launch.
 * - Layouts are dense, row-major, head dimension fastest:
 *     Q, O   [B, n_pos, H_q, d]   storage dtype
 *   and the KV cache in one of two layouts (zha_geom.kv_layout), with Tc =
 *   zha_geom.T_cap (or T when T_cap is 0) token rows per (b, kvh):
 *     ZHA_KV_SPLIT    K, V  [B, H_kv, Tc, d] each
 *     ZHA_KV_CHUNKED  KV    [B, H_kv, ceil(Tc / C), 2, C, d]: page c holds the
 *                     keys of tokens c*C .. c*C + C - 1, then their values;
 *                     rows past T are never read.  The buffer is passed as
 *                     K, and V must be NULL.
 *   The chunked layout keeps each level-1 chunk's keys and values in one
 *   contiguous page, so the sparse gather reads 2 C d-element runs instead of
 *   two runs of C rows in separate arrays.
 *   Query head h reads KV head h / (H_q / H_kv).  Each (b, kvh) pair owns one
 *   tree; its G = H_q / H_kv query heads share it (paper §III-B).
 * - All n_pos positions of a call attend to the same T cached keys.
 *
 * Geometry (zha_geom): n_l = floor(T / C^l) full nodes at level l = 1..L;
 * level 1 nodes are chunks of C consecutive keys, a level-l node has the C
 * level-(l-1) nodes below it as children.  Requirements: B, H_q, H_kv >= 1,
 * H_q % H_kv == 0, d in {64, 128, 256}, 2 <= C <= 1024, 1 <= L <= 16,
 * 1 <= R <= 16, 1 <= T < 2^31, and T_cap == 0 or T <= T_cap < 2^31.
 * A context shorter than C^L leaves the upper levels empty (n_l = 0): an
 * empty level keeps nothing and every node of the level below joins that
 * level's frontier as a node without a complete parent (App. E-E), so the
 * walk is the one through a tree of depth max {l : n_l >= 1}; with T < C no
 * chunk is complete and I(q) is every cached token.
 *
 * Capacity (T_cap): the strides of the KV cache, of the tree blob and of the
 * build scratch follow Tc (T_cap, or T when it is 0); every count follows T.
 * A cache allocated for Tc tokens, and its tree, can then grow token by token
 * in place during decode: append the token's K/V rows, call zha_tree_update
 * with the old and new T, and route and attend with the new T (paper §III-A
 * and App. D-B2: a leaf is summarised when its chunk completes, a parent when
 * its last child completes; the route adds the nodes whose parent is not
 * complete yet, App. E-E).
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage dtype of K, V, Q, O and of the stored summary keys k_hat. */
enum { ZHA_F32 = 0, ZHA_BF16 = 1 };

/* KV cache layout (see the conventions above). */
enum { ZHA_KV_SPLIT = 0, ZHA_KV_CHUNKED = 1 };

enum {
  ZHA_OK = 0,
  ZHA_ERR_NULL = -1,   /* a required pointer is NULL */
  ZHA_ERR_GEOM = -2,   /* geometry violates the requirements above */
  ZHA_ERR_DTYPE = -3,  /* dtype is not ZHA_F32 / ZHA_BF16 */
  ZHA_ERR_DIM = -4,    /* head dimension d not supported */
  ZHA_ERR_P = -5,      /* p is not in (0, 1] (or is NaN) */
  ZHA_ERR_ALIGN = -6,  /* a buffer is not 16-byte aligned */
  ZHA_ERR_CAP = -7,    /* cap < 1 */
  ZHA_ERR_LAUNCH = -8, /* a kernel launch failed */
  ZHA_ERR_NPOS = -9,   /* n_pos < 1 */
  ZHA_ERR_LAYOUT = -10, /* unknown kv_layout, or V given with ZHA_KV_CHUNKED */
  ZHA_ERR_ROPE = -11,   /* rope->dims odd, negative or > d, or theta NULL */
  ZHA_ERR_SCRATCH = -12 /* zha_attn_noalloc: the call needs more than its fixed buffer */
};

/* Values of a failed route's cnt entry (written by the device, see zha_route). */
enum {
  ZHA_ROUTE_BAD_CTX = -1,   /* the position's ctx_len entry is outside [1, T] */
  ZHA_ROUTE_SLOT_BUSY = -2  /* no device-memory frontier slot came free in time */
};

typedef struct {
  int32_t B;     /* sequences */
  int32_t H_q;   /* query heads */
  int32_t H_kv;  /* key/value heads (one tree each) */
  int32_t d;     /* head dimension */
  int64_t T;     /* cached tokens per sequence */
  int32_t C;     /* chunk size = children per node */
  int32_t L;     /* tree depth */
  int32_t R;     /* reference queries per tree */
  int32_t dtype; /* ZHA_F32 or ZHA_BF16 */
  int32_t kv_layout; /* ZHA_KV_SPLIT or ZHA_KV_CHUNKED */
  int64_t T_cap; /* token capacity of the KV cache and tree layout; 0 means T */
} zha_geom;

/* Rotary position embedding of the model, for re-anchoring the tree's
 * reference queries (paper §III-B, reference queries).  Token t sits at
 * position t.  A node's references are rotated to the last position of its
 * span, (i + 1) C^l - 1: for k < dims / 2 the pair (q_k, q_{k + dims/2}) turns
 * by the angle position * theta[k] (a RoFormer rotation in rotate-half
 * pairing); dims from `dims` on are not rotated.  Before a merge each child's
 * log-mass is moved to the parent's reference, F_c + <k_hat_c, q_P - q_c> /
 * sqrt(d), which is the child's tangent evaluated at q_P.
 *   dims   even, 0 <= dims <= d (0: no rotation)
 *   theta  host, dims / 2 angular frequencies in radians per position; read
 *          during the call only */
typedef struct {
  int32_t dims;
  int32_t reserved; /* must be 0 */
  const double* theta;
} zha_rope;

/* Human-readable text for a return code. */
const char* zha_strerror(int code);

/* ---------------------------------------------------------------------------
 * Tree blob
 *
 * For each (b, kvh), at byte offset (b * H_kv + kvh) * tree_stride, the tree
 * holds for every level l = 1..L (nc_l = floor(Tc / C^l) rows of capacity, the
 * first n_l of them valid):
 *   k_hat_l [nc_l, R, d]  storage dtype, at khat_offset(l)
 *   b_hat_l [nc_l, R]     fp32,          at bhat_offset(l)
 * Every array starts on a 256-byte boundary.  k_hat_{l,i,r} is the tangent
 * summary of node i for reference r, rounded to nearest-even from the exact
 * value; b_hat is the matching bias rounded to fp32 (paper §III-A: t_r(q) =
 * q . k_hat_r / sqrt(d) + b_hat_r).
 *
 * tree_stride depends on Tc, C, L, R, d and the dtype only, never on B or
 * H_kv, so the trees of consecutive sequences, or the tree of one KV head of
 * one sequence, form the tree blob of a geometry with fewer sequences (or with
 * H_kv = 1 and H_q = G), as the matching rows of the KV cache form its cache.
 * Independent parts of a batch can therefore be routed and attended by calls
 * of their own over pointers into the same tree, cache and Q (the Q rows of
 * the part must be contiguous: consecutive sequences, or a KV head's G query
 * heads laid out on their own), each with its own scratch, for example on
 * separate streams; each call gives the routes of the full call exactly.
 * ------------------------------------------------------------------------- */

/* Bytes of the tree blob and of the zha_build scratch buffer. */
int zha_tree_bytes(const zha_geom* g, size_t* tree_bytes, size_t* build_scratch_bytes);

/* Byte offsets, inside one tree, of level `level` (1..L) and the per-tree stride. */
int zha_tree_level_offset(const zha_geom* g, int32_t level, size_t* khat_offset,
                          size_t* bhat_offset, size_t* tree_stride);

/* Build every tree (paper §III-A recursive summaries; App. D-B2 baseline merge).
 *   K       device, the keys in g->kv_layout (split: [B, H_kv, T, d]; chunked:
 *           the KV buffer, of which only the key rows are read)
 *   qref    device [H_kv, R, d] fp32 reference queries (all zero gives the
 *           plain mean of each span's keys, with b_hat = ln(span)), or NULL:
 *           every reference is zero (the same trees, bit for bit, and the
 *           build skips the kernels that serve nonzero references)
 *   rope    host, NULL (or dims 0) for shared references; else every node is
 *           summarised at its rotated references and children are re-anchored
 *           to the parent's (zha_rope above).  ZHA_ERR_ROPE if invalid.
 *   tree    device, zha_tree_bytes() bytes, written (the n_l valid rows)
 *   scratch device, build_scratch_bytes: receives the fp64 summaries that a
 *           later merge reads (the nodes of a level a separate merge launch
 *           combines, and every node whose parent is not complete yet, which
 *           zha_tree_update merges when it completes; a full build keeps the
 *           fp64 of complete subtrees on chip), so keep it with the tree
 * Leaves: F = LSE_j(q_r . k_j / sqrt(d)), k_hat = softmax-weighted key mean,
 * b_hat = F - q_r . k_hat / sqrt(d).  Parents, per reference: F_P = LSE_c F_c,
 * k_hat_P = sum_c exp(F_c - F_P) k_hat_c.  Accumulation is fp64, so the stored
 * copies are the correctly rounded values of the exact summaries. */
int zha_build(const zha_geom* g, const void* K, const float* qref, const zha_rope* rope,
              void* tree, void* scratch, void* stream);

/* Extend trees built (or updated) for T_old tokens to g->T tokens, in place
 * (decode-time maintenance, paper §III-A / App. D-B2: the nodes whose spans
 * completed between T_old and T are summarised; nothing else is touched).
 *   T_old   0 <= T_old <= g->T; the tree and scratch hold the result of a
 *           zha_build or zha_tree_update for T_old tokens with this same
 *           geometry otherwise (T_old == 0: nothing built yet)
 *   K, qref, rope, tree, scratch as for zha_build (the same rope as the
 *           build; scratch carries the fp64 child summaries the new parents
 *           are merged from)
 * Leaves [n_1(T_old), n_1(T)) are summarised and, at every level l >= 2, the
 * parents [n_l(T_old), n_l(T)) are merged from their children, so the result
 * is bit-identical to zha_build at T.  Returns ZHA_ERR_GEOM for T_old outside
 * [0, T]. */
int zha_tree_update(const zha_geom* g, int64_t T_old, const void* K, const float* qref,
                    const zha_rope* rope, void* tree, void* scratch, void* stream);

/* ---------------------------------------------------------------------------
 * Routing (paper §III-C; summary page "Routing")
 *
 * For every query head, from the top level down: the frontier starts as all
 * n_L top nodes; each candidate i is scored s_i = max_r (q . k_hat_{r,i} /
 * sqrt(d) + b_hat_{r,i}); candidates are ordered by score, descending, ties
 * to the lower node id; the kept set S_l is the shortest prefix whose share
 * of sum_i exp(s_i) over the frontier reaches p (p == 1 keeps all); the next
 * frontier is the children of S_l, ascending, followed by the level-(l-1)
 * nodes whose parent is incomplete (paper App. E-E).
 * ------------------------------------------------------------------------- */

/* Scratch bytes zha_route needs (0: any pointer, NULL included, may be passed).
 * zha_route and this call return ZHA_ERR_GEOM when level 1 could hold 2^24 or
 * more nodes (floor(T_cap / C), T_cap or T): a level's cut sums a 40-bit
 * fixed-point mass per candidate in 64 bits, so a frontier must stay below 2^24
 * candidates.  Scratch holds:
 *   - calls of 4096 or more query heads (B * n_pos * H_q) route most heads
 *     with a smaller-frontier launch and list there the heads whose frontier
 *     outgrew it: (heads + 1) int32;
 *   - trees whose level 1 can hold more than zha_route_frontier_capacity()
 *     nodes (n_1 at the capacity T_cap, else T): a head whose frontier
 *     outgrows the on-chip capacity is routed again with its frontier in
 *     device memory, in one of 8 slots of 12 * n_1 bytes (ids and scores;
 *     about 100 MB at 2^24 tokens with C = 16).
 * The size depends on the capacity, not on T, so one buffer serves every
 * length up to it.  Calls that overlap in time on the same buffer race. */
int zha_route_scratch_bytes(const zha_geom* g, int32_t n_pos, int32_t cap, size_t* bytes);

/*   tree        device, built by zha_build for the same geometry
 *   Q           device [B, n_pos, H_q, d] storage dtype
 *   ctx_len     device [B, n_pos] int32 or NULL: tokens visible to each
 *               position (NULL: all T).  A position seeing T_t tokens routes
 *               through the nodes complete within them, n_l(T_t) =
 *               floor(T_t / C^l), with orphans taken relative to T_t; causal
 *               prefill passes T_t = t + 1 for the token at cache position t
 *               (paper §V, Q(T) = T: every query sees the nodes completed
 *               before it and its own partial chunk).  A value outside [1, T]
 *               fails that position: cnt = ZHA_ROUTE_BAD_CTX (-1),
 *               level_stats and gap unwritten.
 *   p           top-p threshold in (0, 1]
 *   sel         device [B, n_pos, H_q, cap] int32, written: the level-1 chunk
 *               ids of S_1 in ascending order; entries past min(cnt, cap) are
 *               left untouched
 *   cnt         device [B, n_pos, H_q] int32, written: |S_1|, the true count
 *               even when it exceeds cap (then sel holds the cap lowest ids);
 *               ZHA_ROUTE_BAD_CTX (-1) for a position whose ctx_len entry
 *               is invalid; ZHA_ROUTE_SLOT_BUSY (-2) for a head whose
 *               frontier outgrew the on-chip capacity and found no free
 *               device-memory frontier slot within the wait bound (about a
 *               second; a holder frees its slot as soon as its head is
 *               routed, so this means a stuck or killed holder): sel is then
 *               unwritten and level_stats / gap hold only the levels above
 *               the overflow; calling zha_route again routes such heads.
 *               The environment variable ZHA_ROUTE_SPILL_WAIT, read at each
 *               call, sets the bound in rounds of ~1 us (negative: give up
 *               without waiting), for diagnostics.
 *   level_stats device [B, n_pos, H_q, L, 2] int32 or NULL: for level l at
 *               index l-1, (frontier size K_l, kept count |S_l|)
 *   gap         device [B, n_pos, H_q, L] fp32 or NULL: s_(m) - s_(m+1) at
 *               each level's cut, +inf when the whole frontier is kept
 *   scratch     device, zha_route_scratch_bytes() bytes (ZHA_ERR_NULL if needed
 *               and NULL) */
int zha_route(const zha_geom* g, const void* tree, const void* Q, int32_t n_pos,
              const int32_t* ctx_len, float p,
              int32_t* sel, int32_t* cnt, int32_t cap, int32_t* level_stats, float* gap,
              void* scratch, void* stream);

/* Largest frontier (candidates at one level of one query head) that zha_route
 * holds on chip; larger ones go through the scratch buffer (slower, same
 * result). */
int32_t zha_route_frontier_capacity(void);

/* ---------------------------------------------------------------------------
 * Sparse attention (summary page "Routing": I(q) and o(q))
 *
 * For query head h at position t, seeing T_t tokens (ctx_len, else T), the
 * attended token set is
 *   I = {0} U {c*C .. c*C + C - 1 : c in sel[.., :cnt]} U [n_1*C, T_t)
 * with n_1 = floor(T_t / C) (token 0 is the attention sink, counted once; the
 * tail after the last full chunk is the current partial chunk) and
 *   O = sum_{j in I} softmax_j(q . k_j / sqrt(d)) v_j
 * computed with fp32 arithmetic and rounded nearest-even to the storage dtype.
 * ------------------------------------------------------------------------- */

/* Scratch of zha_attn (and of zha_dense_decode below): split-KV partials
 * (fp32, d + 2 values per query head and split).  Calls that overlap in time
 * on the same buffer race.  0 bytes means no scratch is needed. */
int zha_attn_scratch_bytes(const zha_geom* g, int32_t n_pos, int32_t cap, size_t* bytes);

/*   Q        device, layout above
 *   ctx_len  device [B, n_pos] int32 or NULL, as for zha_route (the same
 *            array); a value outside [1, T] gives a NaN row
 *   K, V     device, the KV cache in g->kv_layout (chunked: K is the KV
 *            buffer and V must be NULL)
 *   sel, cnt device, as written by zha_route (ascending, distinct ids < n_1)
 *   O        device [B, n_pos, H_q, d], written; rows whose cnt is negative or
 *            exceeds cap are written as NaN
 *   scratch  device, zha_attn_scratch_bytes() bytes
 * Split partials are merged in split order, so results do not depend on
 * scheduling. */
int zha_attn(const zha_geom* g, const void* Q, int32_t n_pos, const int32_t* ctx_len,
             const void* K, const void* V,
             const int32_t* sel, const int32_t* cnt, int32_t cap, void* O, void* scratch,
             void* stream);

/* ---------------------------------------------------------------------------
 * Routing and attention in one call (the paper's App. D kernel inventory
 * lists a "fusion" kernel beside routing and attention)
 *
 * zha_route followed by zha_attn, with the same arguments and results: sel,
 * cnt, level_stats and gap as zha_route writes them (bit for bit), O as
 * zha_attn computes it (the same tokens and arithmetic; split points differ,
 * so fp32 summation order and hence the last bits may).  Calls of up to 2048
 * query heads with R = 1, a power-of-two C, p < 1 and a KV cache of less than
 * 2^31 bytes per (b, kvh) run as one launch in which a head's attention
 * starts as soon as its route ends, while other heads are still routed;
 * other calls run zha_route then zha_attn.  The single launch keeps its work
 * queue and counters in device memory of the library (each call leaves them
 * cleared), so calls of zha_route_attn that overlap in time on one device
 * race, whatever their streams and scratch buffers.
 * ------------------------------------------------------------------------- */

/* Scratch of zha_route_attn: zha_route's, then room for the attention
 * (partials of up to 64 pieces per query head, or zha_attn's scratch). */
int zha_route_attn_scratch_bytes(const zha_geom* g, int32_t n_pos, int32_t cap, size_t* bytes);

/*   tree, Q, ctx_len, p, sel, cnt, cap, level_stats, gap  as for zha_route
 *   K, V, O                                               as for zha_attn
 *   scratch  device, zha_route_attn_scratch_bytes() bytes */
int zha_route_attn(const zha_geom* g, const void* tree, const void* Q, int32_t n_pos,
                   const int32_t* ctx_len, float p, const void* K, const void* V, int32_t* sel,
                   int32_t* cnt, int32_t cap, int32_t* level_stats, float* gap, void* O,
                   void* scratch, void* stream);

/* Size of the device buffer zha_attn_noalloc uses in place of a scratch
 * argument (the library holds one on each device it runs on). */
#define ZHA_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* zha_attn for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no scratch argument: the split-KV plan and partials go to a fixed
 * buffer of ZHA_NOALLOC_SCRATCH_BYTES inside the library, one per device,
 * held from the first call on that device until the process ends; the call
 * itself allocates nothing.  Arguments, results and errors as zha_attn, plus
 * ZHA_ERR_SCRATCH (before any launch) for a call whose
 * zha_attn_scratch_bytes() exceeds ZHA_NOALLOC_SCRATCH_BYTES: up to 2048
 * query heads per call always fit at d <= 256 (about 2.7 MB at d = 256); more
 * heads fit only where they need no scratch (fp32, d = 256 or C outside
 * {8, 16, 32, 64}).  Every call on one device shares that device's buffer,
 * which keeps the last call's contents (nothing in it needs to start at zero:
 * a call writes everything it reads), so calls that overlap in time on one
 * device race, whatever their streams. */
int zha_attn_noalloc(const zha_geom* g, const void* Q, int32_t n_pos, const int32_t* ctx_len,
                     const void* K, const void* V, const int32_t* sel, const int32_t* cnt,
                     int32_t cap, void* O, void* stream);

/* ---------------------------------------------------------------------------
 * Dense decode baseline: O = softmax(q K^T / sqrt(d)) V over all T keys.
 * ------------------------------------------------------------------------- */

/* Same scratch contract as zha_attn; K and V as for zha_attn. */
int zha_dense_decode_scratch_bytes(const zha_geom* g, int32_t n_pos, size_t* bytes);

int zha_dense_decode(const zha_geom* g, const void* Q, int32_t n_pos, const void* K,
                     const void* V, void* O, void* scratch, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */
