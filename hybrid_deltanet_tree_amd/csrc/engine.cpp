// engine.cpp - host side of libhdt: validation, launch planning and the
// pending-round bookkeeping behind the C ABI declared in include/hdt.h.
//
// The verbs follow "Adding a model" (step 4 of "The adapter path in ten
// steps": forward_tree, forward_block, commit_tree, rollback_to, kv.length,
// reset) and the round of "One request, end to end" (section 2.6: one pass
// over the merged tree, then the accepted path's KV rows and recurrent state
// are committed).  Each call is step-granular and keeps activations on the
// device ("How ignis serves a request", "The shape of the process").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "hdt.h"
#include "launch.h"

using namespace hdt;

namespace {

constexpr int kSplitCUs = 256;      // splits are sized so one layer spreads over this many items
constexpr int64_t kSplitMin = 256;  // float32 attention: smallest split, in keys
constexpr int64_t kSplitMax = 16384;
constexpr float kConvEps = 1e-6f;      // GDN conv: epsilon of the q/k L2 norm, y / sqrt(sum y^2 + eps)
constexpr int64_t kKvSplitMin = 128;  // bf16 attention: smallest split (> kKvTile - 1 + kMaxNodes - 1)
constexpr int kProfKinds = 10;        // kernel classes of hdt_profile_read
constexpr int32_t kPfPiece = 2048;    // chunked prefill: tokens per piece (one pass through every layer)
constexpr int32_t kPfMaxSplits = 8;   // chunked prefill: most key splits of an attention layer
constexpr int32_t kPfItems = 768;     // chunked prefill: attention items aimed at per layer (3 per CU)

// The scratch of one slot's round: what commit needs of the pass, the attention
// partials and the conv staging.  Nothing in it has to start at zero: every value is
// written by the pass before anything reads it.
struct Scratch {
  float *u_pend = nullptr;    // [n_gdn][max_nodes][hv][dv] delta-rule corrections
  void *k_pend = nullptr;     // [n_gdn][max_nodes][hk][dk] copies of k (io dtype)
  void *a_pend = nullptr;     // [n_gdn][max_nodes][hv] copies of alpha (io dtype)
  float *part_acc = nullptr;  // float32 attention: partials [hkv][nsplit][rows][D]
  float *part_ml = nullptr;   // [hkv][nsplit][rows][2]
  void *part_o = nullptr;     // bf16 attention: normalised bf16 partials [hkv][nsplit][rows][D]
  float *carry_acc = nullptr; // bf16 attention: state of split n_full below tb0 [hkv][rows][D]
  float *carry_ml = nullptr;  // [hkv][rows][2]
  void *conv_out = nullptr;   // GDN conv: post-conv q | k | v of one layer [max_nodes][..] each
  void *x_pend = nullptr;     // GDN conv: pre-conv rows of the tree [n_gdn][max_nodes][C]
};
constexpr int kScratchParts = 10;

struct SlotState {
  hdt_slot_desc d{};
  int32_t split = 0;          // float32 attention: keys per split (bf16 splits follow each row's position)
  int32_t nsplit_cap = 0;
  Scratch own;                // allocated by the engine at its first launching call
  Scratch sc;                 // the scratch of the pending round (own, or carved from the
                              // library's static array by hdt_forward_tree_noalloc)
  int32_t static_dev = -1;    // sc is the static array of this device ...
  uint64_t static_gen = 0;    // ... as handed out by this call (a later call reuses it)
  bool pending = false;
  bool walk_pending = false;  // an accept walk's commit is in flight: length not yet known
  int64_t anchor_every = 0;   // state anchors: anchor k holds position (k + 1) * every
  int32_t anchor_n = 0;
  float *anchor_state = nullptr;
  void *anchor_conv = nullptr;
  std::vector<bool> anchor_ok;
  hipEvent_t walk_ev = nullptr;
  int32_t n = 0;
  int32_t chain = 0;
  int8_t parent[kMaxNodes]{};
  int8_t depth[kMaxNodes]{};
};

struct EventPair {
  hipEvent_t a, b;
  int kind;
};

}  // namespace

struct hdt_engine {
  hdt_model_desc desc{};
  std::vector<uint8_t> kind;
  std::vector<int32_t> kind_index;  // index of layer l among layers of its kind
  int32_t n_gdn = 0, n_attn = 0;
  int32_t esz = 2;
  std::vector<SlotState> slots;
  std::string err;
  bool allocated = false;
  int max_lds = 0;  // dynamic LDS a workgroup may use on the device
  bool profiling = false;
  bool no_events = false;  // the launch in progress may create no events (hdt_forward_tree_noalloc)
  std::vector<EventPair> ev_live;
  std::vector<EventPair> ev_pool;
  int32_t conv_C = 0;  // channels through the GDN conv: 2 hk dk + hv dv
  int32_t *walk_m = nullptr;      // pinned host copy of each slot's last accept-walk length
  int64_t kv_per_head = 1;        // bf16 attention: most splits a row may have
  std::vector<int32_t> kv_ladder;  // bf16 attention: split sizes, ascending
  double prof_ms[kProfKinds] = {};
  int64_t prof_count[kProfKinds] = {};
  // chunked prefill (hdt_forward_chunked): scratch for one piece of up to kPfPiece
  // tokens, allocated at its first call
  struct {
    uint16_t *w_hi = nullptr, *w_lo = nullptr, *mq_hi = nullptr, *mq_lo = nullptr, *kt = nullptr, *qc = nullptr;
    float *ut = nullptr, *g = nullptr, *part_acc = nullptr, *part_ml = nullptr;
    void *conv = nullptr;  // post-conv q, k, v of a piece (models with the short conv)
    bool allocated = false;
  } pf;
};

namespace {

hdt_status fail(hdt_engine *e, hdt_status code, const char *fmt, ...) {
  if (e) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    e->err = buf;
  }
  return code;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t pow2_floor(int64_t x) {
  int64_t p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}

// Split sizes.  A row's fold structure must not depend on how many of its keys are
// committed, or a verified row would differ from the decoded row.
//  float32 storage: a slot's split depends on its capacity alone: a power of two
//    between kSplitMin and kSplitMax chosen so that a full cache gives about
//    kSplitCUs (kv head, split) items;
//  bf16 storage: a row's split depends on its own position alone (and on the
//    engine's shape): the row that sees K keys takes the smallest rung of the
//    ladder kKvSplitMin, then s + max(kKvTile, s / 32) rounded up to kKvTile, ...
//    that cuts K keys into at most per_head splits, per_head = kSplitCUs /
//    (H_kv row_groups).  So at any length a layer is about one wave of
//    kSplitCUs (kv head, split, row group) workgroups, a slot's capacity does not
//    matter, and the rungs are close enough (3-6 %) that a layer rarely holds rows
//    of two split sizes.

// Row groups of the split pass for the engine's largest tree (bf16 attention).
int32_t kv_row_groups(const hdt_model_desc &m) {
  if (m.attn_hkv <= 0) return 1;
  const int64_t rows = static_cast<int64_t>(m.max_nodes) * (m.attn_hq / m.attn_hkv);
  return static_cast<int32_t>(std::max<int64_t>(1, (rows + kKvRowsPerItem - 1) / kKvRowsPerItem));
}

int32_t split_for(int64_t capacity, int32_t hkv) {
  int64_t s = pow2_floor(std::max<int64_t>(1, capacity * hkv / kSplitCUs));
  s = std::max(kSplitMin, std::min(kSplitMax, s));
  return static_cast<int32_t>(s);
}

int64_t kv_per_head(const hdt_model_desc &m) {
  return std::max<int64_t>(1, kSplitCUs / (static_cast<int64_t>(std::max(1, m.attn_hkv)) * kv_row_groups(m)));
}

// The rungs up to the first one that serves max_keys.
std::vector<int32_t> kv_ladder(int64_t max_keys, int64_t per_head) {
  std::vector<int32_t> r;
  int64_t s = kKvSplitMin;
  const int64_t need = (max_keys + per_head - 1) / per_head;
  while (true) {
    r.push_back(static_cast<int32_t>(s));
    if (s >= need) break;
    s = (s + std::max<int64_t>(kKvTile, s / 32) + kKvTile - 1) / kKvTile * kKvTile;
  }
  return r;
}

// Validates a parent array and fills depth; returns false for a non-tree.
bool plan_tree(int32_t n, const int32_t *parent, int8_t *par, int8_t *dep, int32_t *chain) {
  if (n < 1 || n > kMaxNodes || !parent || parent[0] != -1) return false;
  for (int i = 1; i < n; ++i)
    if (parent[i] < 0 || parent[i] >= i) return false;
  for (int i = 0; i < n; ++i) {
    par[i] = static_cast<int8_t>(parent[i]);
    dep[i] = static_cast<int8_t>(i == 0 ? 0 : dep[parent[i]] + 1);
  }
  int c = 1;
  while (c < n && parent[c] == c - 1) ++c;
  *chain = c;
  return true;
}

// States the GDN walk keeps in LDS: node p's, when a later child c of p does not
// directly follow p (parent[c] != c - 1), so the walk restores S_p from LDS
// instead of replaying p's root path.  Slots go to the first kGdnSaves such nodes;
// returns how many were used.
int plan_saves(int n, const int8_t *par, int8_t *save) {
  std::memset(save, -1, kMaxNodes);
  int used = 0;
  for (int c = 1; c < n; ++c) {
    const int p = par[c];
    if (p != c - 1 && save[p] < 0 && used < kGdnSaves) save[p] = static_cast<int8_t>(used++);
  }
  return used;
}

hdt_status check_hip(hdt_engine *e, hipError_t r, const char *what) {
  if (r != hipSuccess) return fail(e, HDT_E_HIP, "%s: %s", what, hipGetErrorString(r));
  return HDT_OK;
}

// Bytes of each part of one slot's scratch, in the order of the Scratch fields.
void scratch_sizes(const hdt_engine *e, const SlotState &s, size_t (&b)[kScratchParts]) {
  const hdt_model_desc &m = e->desc;
  for (auto &x : b) x = 0;
  const size_t nm = static_cast<size_t>(m.max_nodes);
  if (e->n_gdn > 0) {
    const size_t ng = static_cast<size_t>(e->n_gdn);
    b[0] = ng * nm * m.gdn_hv * m.gdn_dv * sizeof(float);
    b[1] = ng * nm * m.gdn_hk * m.gdn_dk * e->esz;
    b[2] = ng * nm * m.gdn_hv * e->esz;
    if (m.gdn_conv > 0) {
      b[8] = nm * e->conv_C * e->esz;
      b[9] = ng * nm * e->conv_C * e->esz;
    }
  }
  if (e->n_attn > 0) {
    const size_t G = static_cast<size_t>(m.attn_hq / m.attn_hkv);
    const size_t rows = nm * G;
    const size_t base = static_cast<size_t>(m.attn_hkv) * s.nsplit_cap * rows;
    const size_t carry = static_cast<size_t>(m.attn_hkv) * rows;
    b[4] = base * 2 * sizeof(float);
    if (m.io_dtype == HDT_BF16) {
      b[5] = base * m.attn_d * 2;
      b[6] = carry * m.attn_d * sizeof(float);
      b[7] = carry * 2 * sizeof(float);
    } else {
      b[3] = base * m.attn_d * sizeof(float);
    }
  }
}

void **scratch_part(Scratch &x, int i) {
  void **p[kScratchParts] = {reinterpret_cast<void **>(&x.u_pend), &x.k_pend, &x.a_pend,
                             reinterpret_cast<void **>(&x.part_acc), reinterpret_cast<void **>(&x.part_ml),
                             &x.part_o, reinterpret_cast<void **>(&x.carry_acc),
                             reinterpret_cast<void **>(&x.carry_ml), &x.conv_out, &x.x_pend};
  return p[i];
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Bytes of one slot's scratch carved from one block, each part 256-byte aligned.
size_t scratch_bytes(const hdt_engine *e, const SlotState &s) {
  size_t b[kScratchParts], total = 0;
  scratch_sizes(e, s, b);
  for (size_t x : b) total += align256(x);
  return total;
}

// The device's LDS limit per workgroup (an attribute query; nothing is allocated).
hdt_status query_lds(hdt_engine *e) {
  if (e->max_lds > 0) return HDT_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&e->max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return fail(e, HDT_E_HIP, "cannot query the current HIP device");
  return HDT_OK;
}

// The pinned word and the event of each slot that hdt_walk_commit uses.
hdt_status ensure_walk(hdt_engine *e) {
  if (e->walk_m) return HDT_OK;
  if (hipHostMalloc(reinterpret_cast<void **>(&e->walk_m), e->slots.size() * sizeof(int32_t)) != hipSuccess) {
    e->walk_m = nullptr;
    return fail(e, HDT_E_HIP, "hipHostMalloc of the walk results failed");
  }
  for (auto &s : e->slots)
    if (hipEventCreateWithFlags(&s.walk_ev, hipEventDisableTiming) != hipSuccess)
      return fail(e, HDT_E_HIP, "hipEventCreate failed");
  return HDT_OK;
}

// The engine's own scratch, allocated at the first call that launches with it.
hdt_status ensure_alloc(hdt_engine *e) {
  if (e->allocated) return HDT_OK;
  hdt_status st = query_lds(e);
  if (st != HDT_OK) return st;
  for (auto &s : e->slots) {
    size_t b[kScratchParts];
    scratch_sizes(e, s, b);
    for (int i = 0; i < kScratchParts; ++i)
      if (b[i] > 0 && hipMalloc(scratch_part(s.own, i), b[i]) != hipSuccess)
        return fail(e, HDT_E_HIP, "hipMalloc of the slot scratch failed");
  }
  st = ensure_walk(e);
  if (st != HDT_OK) return st;
  e->allocated = true;
  return HDT_OK;
}

void free_scratch(hdt_engine *e) {
  for (auto &s : e->slots) {
    for (int i = 0; i < kScratchParts; ++i) {
      void **p = scratch_part(s.own, i);
      (void)hipFree(*p);
      *p = nullptr;
    }
    s.sc = Scratch{};
    if (s.walk_ev) (void)hipEventDestroy(s.walk_ev);
    s.walk_ev = nullptr;
  }
  if (e->walk_m) (void)hipHostFree(e->walk_m);
  e->walk_m = nullptr;
  e->allocated = false;
  void *pf[] = {e->pf.w_hi, e->pf.w_lo, e->pf.mq_hi, e->pf.mq_lo, e->pf.kt, e->pf.qc,
                e->pf.ut, e->pf.g, e->pf.part_acc, e->pf.part_ml, e->pf.conv};
  for (void *p : pf) (void)hipFree(p);
  e->pf = {};
}

// When profiling is on, hands one launch an event pair that its dispatch records
// (kernel start and end), and keeps the pair for hdt_profile_read.
struct ProfScope {
  hdt_engine *e;
  EventPair ev{};
  bool on = false;
  ProfScope(hdt_engine *e_, int k) : e(e_) {
    if (!e->profiling || e->no_events) return;
    if (!e->ev_pool.empty()) {
      ev = e->ev_pool.back();
      e->ev_pool.pop_back();
    } else if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess) {
      return;
    }
    ev.kind = k;
    on = true;
  }
  KernelEvents events() const {
    KernelEvents k;
    if (on) {
      k.start = ev.a;
      k.stop = ev.b;
    }
    return k;
  }
  ~ProfScope() {
    if (on) e->ev_live.push_back(ev);
  }
};

// bf16 attention: split size of a row that sees K keys (K <= the largest capacity).
int32_t kv_split_of(const hdt_engine *e, int64_t K) {
  const int64_t need = (K + e->kv_per_head - 1) / e->kv_per_head;
  const auto it = std::lower_bound(e->kv_ladder.begin(), e->kv_ladder.end(), need);
  return it == e->kv_ladder.end() ? e->kv_ladder.back() : *it;
}

// Split sizes of a tree's rows in ascending order, and the nodes of each (ascending
// tree index).  Usually one size; a tree whose rows straddle a rung has two.
struct KvGroups {
  int count = 0;
  int32_t split[kMaxNodes];
  int32_t n[kMaxNodes];
  int8_t nodes[kMaxNodes][kMaxNodes];
};

void plan_kv_groups(const hdt_engine *e, int64_t L, int32_t n, const int8_t *dep, KvGroups &g) {
  int32_t sz[kMaxNodes];
  g.count = 0;
  for (int i = 0; i < n; ++i) {
    sz[i] = kv_split_of(e, L + dep[i] + 1);
    int k = 0;
    while (k < g.count && g.split[k] != sz[i]) ++k;
    if (k == g.count) g.split[g.count++] = sz[i];
  }
  std::sort(g.split, g.split + g.count);
  for (int k = 0; k < g.count; ++k) {
    g.n[k] = 0;
    for (int i = 0; i < n; ++i)
      if (sz[i] == g.split[k]) g.nodes[k][g.n[k]++] = static_cast<int8_t>(i);
  }
}

// One attention layer with bf16 storage, for group gr of every tree that has one:
// the split pass over the committed rows, then the tree pass (tree tiles, fold,
// output, pending rows).
hdt_status launch_kv_group(hdt_engine *e, int32_t n_trees, const hdt_tree *trees,
                           const int8_t (*par)[kMaxNodes], const int8_t (*dep)[kMaxNodes],
                           const KvGroups *groups, int gr, int l, int ki, hipStream_t stream) {
  const hdt_model_desc &m = e->desc;
  const int G = m.attn_hq / m.attn_hkv;
  KvLaunch a;
  std::memset(&a, 0, sizeof a);
  a.hq = m.attn_hq;
  a.hkv = m.attn_hkv;
  a.c2 = m.attn_scale * 1.4426950408889634f;
  // Split-pass shape: 6 waves that compute one 16-row block each beside 2 waves that
  // only issue the tile loads, kKvRowsPerItem rows per workgroup; a tree with more
  // rows takes several row groups, placed on one XCD so that they read each tile
  // through the same L2.
  int32_t items_a = 0, items_b = 0, tiles_b = 1;
  for (int t = 0; t < n_trees; ++t) {
    if (gr >= groups[t].count) continue;
    const hdt_tree &tr = trees[t];
    SlotState &s = e->slots[tr.slot];
    const hdt_layer_io &io = tr.io[l];
    KvTree &x = a.t[a.n_trees++];
    const int32_t split = groups[t].split[gr];
    x.gn = groups[t].n[gr];
    std::memcpy(x.nodes, groups[t].nodes[gr], kMaxNodes);
    const size_t view = static_cast<size_t>(m.attn_hkv) * s.d.capacity * m.attn_d * 2;
    x.q = io.q;
    x.kt = io.k;
    x.vt = io.v;
    x.kc = static_cast<char *>(s.d.k_cache) + static_cast<size_t>(ki) * view;
    x.vc = static_cast<char *>(s.d.v_cache) + static_cast<size_t>(ki) * view;
    x.o = io.o;
    x.part_o = s.sc.part_o;
    x.part_ml = s.sc.part_ml;
    x.carry_acc = s.sc.carry_acc;
    x.carry_ml = s.sc.carry_ml;
    x.L = s.d.length;
    x.cap = s.d.capacity;
    x.n = tr.n_nodes;
    x.split = split;
    x.nsplit_cap = s.nsplit_cap;
    x.rows_cap = m.max_nodes * G;
    x.n_full = static_cast<int32_t>(s.d.length / split);
    const int64_t tb0 = s.d.length / kKvTile * kKvTile;
    x.carry_tiles = static_cast<int32_t>((tb0 - static_cast<int64_t>(x.n_full) * split) / kKvTile);
    x.row_groups = (x.gn * G + kKvRowsPerItem - 1) / kKvRowsPerItem;
    x.a_splits = x.n_full + (x.carry_tiles > 0 ? 1 : 0);
    const int pairs = m.attn_hkv * x.a_splits;  // (kv head, split)
    items_a = std::max(items_a, (pairs + 7) / 8 * 8 * x.row_groups);
    items_b = std::max(items_b, m.attn_hkv * x.gn * kKvQuarters);
    for (int i = 0; i < x.gn; ++i) {  // tiles from tb0 to each node's position
      const int64_t pos = s.d.length + dep[t][static_cast<int>(x.nodes[i])];
      tiles_b = std::max(tiles_b, static_cast<int32_t>((pos / kKvTile * kKvTile - tb0) / kKvTile + 1));
    }
    std::memcpy(x.parent, par[t], kMaxNodes);
    std::memcpy(x.depth, dep[t], kMaxNodes);
  }
  if (items_a > 0) {
    ProfScope p(e, 1);
    hdt_status st = check_hip(e, launch_kv_split(a, m.attn_d, items_a, stream, p.events()),
                              "attention split launch");
    if (st != HDT_OK) return st;
  }
  ProfScope p(e, 2);
  return check_hip(e, launch_kv_tree(a, m.attn_d, items_b, tiles_b, stream, p.events()), "attention tree launch");
}

// One attention layer with bf16 storage: one launch pair per group of nodes that
// share a split size (one group, unless a tree's rows straddle a rung).
hdt_status launch_kv_layer(hdt_engine *e, int32_t n_trees, const hdt_tree *trees,
                           const int8_t (*par)[kMaxNodes], const int8_t (*dep)[kMaxNodes],
                           const KvGroups *groups, int l, int ki, hipStream_t stream) {
  int max_groups = 0;
  for (int t = 0; t < n_trees; ++t) max_groups = std::max(max_groups, groups[t].count);
  for (int gr = 0; gr < max_groups; ++gr) {
    hdt_status st = launch_kv_group(e, n_trees, trees, par, dep, groups, gr, l, ki, stream);
    if (st != HDT_OK) return st;
  }
  return HDT_OK;
}

// The short causal conv in front of GDN layer l (its ki-th GDN layer), every tree at once.
hdt_status launch_conv_layer(hdt_engine *e, int32_t n_trees, const hdt_tree *trees,
                             const int8_t (*par)[kMaxNodes], const int8_t (*dep)[kMaxNodes], int l,
                             int ki, int32_t n_max, hipStream_t stream) {
  const hdt_model_desc &m = e->desc;
  ConvLaunch c;
  std::memset(&c, 0, sizeof c);
  c.n_trees = n_trees;
  c.n_max = n_max;
  c.width = m.gdn_conv;
  c.hk = m.gdn_hk;
  c.dk = m.gdn_dk;
  c.hv = m.gdn_hv;
  c.dv = m.gdn_dv;
  c.eps = kConvEps;
  c.weight = m.gdn_conv_weight + static_cast<size_t>(ki) * e->conv_C * m.gdn_conv;
  const size_t nm = static_cast<size_t>(m.max_nodes);
  const size_t row = static_cast<size_t>(e->conv_C) * e->esz;
  const size_t cq = nm * m.gdn_hk * m.gdn_dk * e->esz;
  for (int t = 0; t < n_trees; ++t) {
    const hdt_tree &tr = trees[t];
    SlotState &s = e->slots[tr.slot];
    const hdt_layer_io &io = tr.io[l];
    ConvTree &x = c.t[t];
    x.q = io.q;
    x.k = io.k;
    x.v = io.v;
    x.tail = static_cast<const char *>(s.d.gdn_conv_state) + static_cast<size_t>(ki) * (m.gdn_conv - 1) * row;
    x.qo = s.sc.conv_out;
    x.ko = static_cast<char *>(s.sc.conv_out) + cq;
    x.vo = static_cast<char *>(s.sc.conv_out) + 2 * cq;
    x.x_pend = static_cast<char *>(s.sc.x_pend) + static_cast<size_t>(ki) * nm * row;
    x.n = tr.n_nodes;
    std::memcpy(x.parent, par[t], kMaxNodes);
    std::memcpy(x.depth, dep[t], kMaxNodes);
  }
  ProfScope p(e, 4);
  return check_hip(e, launch_gdn_conv(c, m.io_dtype == HDT_BF16, stream, p.events()), "GDN conv launch");
}

// chain_commit: every tree is a chain that will be committed whole (a prefill span):
// the GDN walk writes each layer's final state straight to the committed state.
hdt_status launch_forward(hdt_engine *e, int32_t n_trees, const hdt_tree *trees, const int8_t (*par)[kMaxNodes],
                          const int8_t (*dep)[kMaxNodes], hipStream_t stream, bool chain_commit = false) {
  const hdt_model_desc &m = e->desc;
  const int bf = m.io_dtype == HDT_BF16;
  const int G = m.attn_hkv > 0 ? m.attn_hq / m.attn_hkv : 1;
  int32_t n_max = 0;
  for (int t = 0; t < n_trees; ++t) n_max = std::max(n_max, trees[t].n_nodes);
  // bf16 attention: every row's split size, the same for all layers of the pass
  KvGroups groups[kMaxTrees];
  if (bf && e->n_attn > 0)
    for (int t = 0; t < n_trees; ++t)
      plan_kv_groups(e, e->slots[trees[t].slot].d.length, trees[t].n_nodes, dep[t], groups[t]);

  for (int l = 0; l < m.n_layers; ++l) {
    const int ki = e->kind_index[l];
    if (e->kind[l] == 0) {
      if (m.gdn_conv > 0) {
        hdt_status st = launch_conv_layer(e, n_trees, trees, par, dep, l, ki, n_max, stream);
        if (st != HDT_OK) return st;
      }
      GdnLaunch a;
      std::memset(&a, 0, sizeof a);
      a.n_trees = n_trees;
      a.hk = m.gdn_hk;
      a.hv = m.gdn_hv;
      a.dv = m.gdn_dv;
      a.n_max = n_max;
      a.scale = m.gdn_scale;
      for (int t = 0; t < n_trees; ++t) {
        const hdt_tree &tr = trees[t];
        SlotState &s = e->slots[tr.slot];
        const hdt_layer_io &io = tr.io[l];
        GdnTree &g = a.t[t];
        if (m.gdn_conv > 0) {  // the walk reads the conv output of this layer
          const size_t cq = static_cast<size_t>(m.max_nodes) * m.gdn_hk * m.gdn_dk * e->esz;
          g.q = s.sc.conv_out;
          g.k = static_cast<char *>(s.sc.conv_out) + cq;
          g.v = static_cast<char *>(s.sc.conv_out) + 2 * cq;
        } else {
          g.q = io.q;
          g.k = io.k;
          g.v = io.v;
        }
        g.alpha = io.alpha;
        g.beta = io.beta;
        g.o = io.o;
        const size_t hs = static_cast<size_t>(m.gdn_hv) * m.gdn_dv * m.gdn_dk;
        g.state = s.d.gdn_state + static_cast<size_t>(ki) * hs;
        g.commit_state = chain_commit ? s.d.gdn_state + static_cast<size_t>(ki) * hs : nullptr;
        const size_t nm = static_cast<size_t>(m.max_nodes);
        g.u_pend = s.sc.u_pend + static_cast<size_t>(ki) * nm * m.gdn_hv * m.gdn_dv;
        g.k_pend = static_cast<char *>(s.sc.k_pend) +
                   static_cast<size_t>(ki) * nm * m.gdn_hk * m.gdn_dk * e->esz;
        g.a_pend = static_cast<char *>(s.sc.a_pend) + static_cast<size_t>(ki) * nm * m.gdn_hv * e->esz;
        g.n = tr.n_nodes;
        std::memcpy(g.parent, par[t], kMaxNodes);
        std::memcpy(g.depth, dep[t], kMaxNodes);
        a.n_saves = std::max(a.n_saves, plan_saves(tr.n_nodes, par[t], g.save));
        g.need_anc = 0;  // a restore without a kept state replays the parent's root path
        for (int c = 1; c < tr.n_nodes; ++c) {
          if (par[t][c] != c - 1) {
            g.restore_mask |= uint64_t{1} << c;
            if (g.save[par[t][c]] < 0) g.need_anc = a.any_anc = 1;
          }
        }
        for (int c = 0; c < tr.n_nodes; ++c)
          if (g.save[c] >= 0) g.keep_mask |= uint64_t{1} << c;
      }
      ProfScope p(e, 0);
      hdt_status st =
          check_hip(e, launch_gdn_tree(a, m.gdn_dk, bf, stream, p.events()), "GDN tree launch");
      if (st != HDT_OK) return st;
    } else if (bf) {
      hdt_status st = launch_kv_layer(e, n_trees, trees, par, dep, groups, l, ki, stream);
      if (st != HDT_OK) return st;
    } else {
      AttnLaunch a;
      std::memset(&a, 0, sizeof a);
      a.n_trees = n_trees;
      a.hq = m.attn_hq;
      a.hkv = m.attn_hkv;
      a.n_max = n_max;
      a.c2 = m.attn_scale * 1.4426950408889634f;
      FoldLaunch f;
      std::memset(&f, 0, sizeof f);
      f.n_trees = n_trees;
      f.hq = m.attn_hq;
      f.hkv = m.attn_hkv;
      int32_t items = 0, rows = 0;
      for (int t = 0; t < n_trees; ++t) {
        const hdt_tree &tr = trees[t];
        SlotState &s = e->slots[tr.slot];
        const hdt_layer_io &io = tr.io[l];
        AttnTree &x = a.t[t];
        const size_t view = static_cast<size_t>(m.attn_hkv) * s.d.capacity * m.attn_d * e->esz;
        x.q = io.q;
        x.kt = io.k;
        x.vt = io.v;
        x.kc = static_cast<char *>(s.d.k_cache) + static_cast<size_t>(ki) * view;
        x.vc = static_cast<char *>(s.d.v_cache) + static_cast<size_t>(ki) * view;
        x.part_acc = s.sc.part_acc;
        x.part_ml = s.sc.part_ml;
        x.L = s.d.length;
        x.cap = s.d.capacity;
        x.n = tr.n_nodes;
        x.split = s.split;
        x.n_shared = static_cast<int32_t>(s.d.length / s.split);
        x.nsplit_cap = s.nsplit_cap;
        x.rows_cap = m.max_nodes * G;
        x.item_begin = items;
        const int tn = attn_nodes_per_tail(bf), rpi = attn_rows_per_item(bf);
        x.tail_nodes = tn;
        x.n_tail_items = m.attn_hkv * ((tr.n_nodes + tn - 1) / tn);
        x.row_groups = (tr.n_nodes * G + rpi - 1) / rpi;
        std::memcpy(x.parent, par[t], kMaxNodes);
        std::memcpy(x.depth, dep[t], kMaxNodes);
        items += x.n_tail_items + m.attn_hkv * x.n_shared * x.row_groups;

        FoldTree &y = f.t[t];
        y.part_acc = s.sc.part_acc;
        y.part_ml = s.sc.part_ml;
        y.o = io.o;
        y.L = s.d.length;
        y.n = tr.n_nodes;
        y.split = s.split;
        y.nsplit_cap = s.nsplit_cap;
        y.rows_cap = x.rows_cap;
        y.row_begin = rows;
        std::memcpy(y.depth, dep[t], kMaxNodes);
        rows += tr.n_nodes * m.attn_hq;
      }
      {
        ProfScope p(e, 1);
        hdt_status st = check_hip(e, launch_attn_split(a, m.attn_d, bf, items, stream, p.events()),
                                  "attention split launch");
        if (st != HDT_OK) return st;
      }
      {
        ProfScope p(e, 2);
        hdt_status st = check_hip(e, launch_attn_fold(f, m.attn_d, bf, rows, stream, p.events()),
                                  "attention fold launch");
        if (st != HDT_OK) return st;
      }
    }
  }
  return HDT_OK;
}

// Commits a root path of the pending tree: from the host (path, m_len), or, with
// dev_out set, from the accept walk's output in device memory (m_len is then the
// tree's node count, the most the path can hold); the caller updates the length.
// tails_only: a prefill chain whose states and cache rows are already in place; only
// the conv tails roll.
hdt_status do_commit(hdt_engine *e, int32_t slot, const int32_t *path, int32_t m_len,
                     const int32_t *dev_out, hipStream_t stream, bool tails_only = false) {
  const hdt_model_desc &m = e->desc;
  SlotState &s = e->slots[slot];
  CommitLaunch c;
  std::memset(&c, 0, sizeof c);
  c.state = s.d.gdn_state;
  c.u_pend = s.sc.u_pend;
  c.k_pend = s.sc.k_pend;
  c.a_pend = s.sc.a_pend;
  c.kc = s.d.k_cache;
  c.vc = s.d.v_cache;
  c.L = s.d.length;
  c.cap = s.d.capacity;
  c.n_gdn = e->n_gdn;
  c.n_attn = e->n_attn;
  c.max_nodes = m.max_nodes;
  c.hk = m.gdn_hk;
  c.hv = m.gdn_hv;
  c.dv = m.gdn_dv;
  c.hkv = m.attn_hkv;
  c.D = m.attn_d;
  c.gdn_blocks = e->n_gdn > 0 && !tails_only ? e->n_gdn * m.gdn_hv * (m.gdn_dv / (kGdnCols * kCommitCols)) : 0;
  c.kv_blocks = e->n_attn > 0 && !tails_only ? e->n_attn * m.attn_hkv : 0;
  int conv_blocks = 0;
  if (e->n_gdn > 0 && m.gdn_conv > 1) {
    c.conv_state = s.d.gdn_conv_state;
    c.x_pend = s.sc.x_pend;
    c.conv_width = m.gdn_conv;
    c.conv_C = e->conv_C;
    const int64_t chunks = static_cast<int64_t>(e->conv_C) * e->esz / 16;
    c.conv_blocks_per_layer = static_cast<int32_t>((chunks + kGdnThreads - 1) / kGdnThreads);
    conv_blocks = e->n_gdn * c.conv_blocks_per_layer;
  }
  c.m = m_len;
  c.dev_out = dev_out;
  if (!dev_out)
    for (int d = 0; d < m_len; ++d) c.path[d] = static_cast<int8_t>(path[d]);
  const int blocks = c.gdn_blocks + c.kv_blocks + conv_blocks;
  if (blocks > 0) {
    ProfScope p(e, 3);
    const int dk = e->n_gdn > 0 ? m.gdn_dk : 64;
    hdt_status st = check_hip(e, launch_commit(c, dk, m.io_dtype == HDT_BF16, blocks, stream, p.events()),
                              "commit launch");
    if (st != HDT_OK) return st;
  }
  s.pending = false;
  return HDT_OK;
}

size_t gdn_state_bytes(const hdt_engine *e) {
  return static_cast<size_t>(e->n_gdn) * e->desc.gdn_hv * e->desc.gdn_dv * e->desc.gdn_dk * sizeof(float);
}

size_t conv_tail_bytes(const hdt_engine *e) {
  return e->desc.gdn_conv > 1 ? static_cast<size_t>(e->n_gdn) * (e->desc.gdn_conv - 1) * e->conv_C * e->esz : 0;
}

// Copies the slot's recurrent state (and conv tails) to or from anchor k.
hdt_status anchor_copy(hdt_engine *e, int32_t slot, int32_t k, bool save, hipStream_t stream) {
  SlotState &s = e->slots[slot];
  const size_t sb = gdn_state_bytes(e), cb = conv_tail_bytes(e);
  char *as = reinterpret_cast<char *>(s.anchor_state) + static_cast<size_t>(k) * sb;
  if (sb > 0 && hipMemcpyAsync(save ? as : static_cast<void *>(s.d.gdn_state), save ? s.d.gdn_state : static_cast<void *>(as),
                               sb, hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return fail(e, HDT_E_HIP, "anchor copy of the state failed");
  if (cb > 0) {
    char *ac = static_cast<char *>(s.anchor_conv) + static_cast<size_t>(k) * cb;
    if (hipMemcpyAsync(save ? ac : s.d.gdn_conv_state, save ? s.d.gdn_conv_state : static_cast<void *>(ac), cb,
                       hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return fail(e, HDT_E_HIP, "anchor copy of the conv tails failed");
  }
  if (save) s.anchor_ok[k] = true;
  return HDT_OK;
}

// Shape signature of a state snapshot: FNV-1a over every field that fixes the layout of
// the state sections (layer kinds in order, GDN heads and dims, conv width, io dtype) and
// the attention shape the length is measured against.
uint64_t shape_signature(const hdt_engine *e) {
  const hdt_model_desc &m = e->desc;
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&h](int64_t x) {
    for (int b = 0; b < 8; ++b) {
      h ^= static_cast<uint64_t>(x >> (8 * b)) & 0xFFu;
      h *= 0x100000001b3ull;
    }
  };
  mix(m.n_layers);
  for (int l = 0; l < m.n_layers; ++l) mix(e->kind[l]);
  for (int64_t x : {int64_t(m.gdn_hk), int64_t(m.gdn_hv), int64_t(m.gdn_dk), int64_t(m.gdn_dv),
                    int64_t(m.gdn_conv), int64_t(m.attn_hq), int64_t(m.attn_hkv), int64_t(m.attn_d),
                    int64_t(m.io_dtype)})
    mix(x);
  return h;
}

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t snapshot_bytes(const hdt_engine *e) {
  return kSnapshotHeaderBytes + round256(static_cast<int64_t>(gdn_state_bytes(e))) +
         static_cast<int64_t>(conv_tail_bytes(e));
}

// hdt_forward_tree_noalloc hands out the library's static scratch array of a device to
// one call at a time; each call takes the next generation, and a pending round whose
// generation is no longer the latest has had its scratch reused.
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
uint64_t g_static_gen[kMaxDevices] = {};

hdt_status check_round_scratch(hdt_engine *e, const SlotState &s) {
  if (s.static_gen == 0) return HDT_OK;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (g_static_gen[s.static_dev] != s.static_gen)
    return fail(e, HDT_E_ORDER, "the pending round's static scratch was reused by a later "
                "hdt_forward_tree_noalloc call on this device");
  return HDT_OK;
}

// After an accept walk, the slot's new length is known once the device has run the
// walk: wait for it and take m from the pinned copy.
hdt_status settle(hdt_engine *e, int32_t slot) {
  SlotState &s = e->slots[slot];
  if (!s.walk_pending) return HDT_OK;
  if (hipEventSynchronize(s.walk_ev) != hipSuccess)
    return fail(e, HDT_E_HIP, "waiting for the accept walk of slot %d failed", slot);
  s.d.length += e->walk_m[slot];
  s.walk_pending = false;
  return HDT_OK;
}

}  // namespace

extern "C" {

hdt_status hdt_create(const hdt_model_desc *desc, int32_t n_slots, const hdt_slot_desc *slots,
                      hdt_engine **out) {
  if (!out) return HDT_E_INVALID;
  *out = nullptr;
  if (!desc || !slots || n_slots < 1) return HDT_E_INVALID;
  const hdt_model_desc &m = *desc;
  if (m.n_layers < 1 || !m.layer_kind) return HDT_E_INVALID;
  int n_gdn = 0, n_attn = 0;
  for (int l = 0; l < m.n_layers; ++l) {
    if (m.layer_kind[l] > 1) return HDT_E_INVALID;
    (m.layer_kind[l] == 0 ? n_gdn : n_attn)++;
  }
  if (m.io_dtype != HDT_F32 && m.io_dtype != HDT_BF16) return HDT_E_INVALID;
  if (m.max_nodes < 1 || m.max_nodes > HDT_MAX_NODES) return HDT_E_INVALID;
  if (n_gdn > 0) {
    if (m.gdn_hk < 1 || m.gdn_hv < m.gdn_hk || m.gdn_hv % m.gdn_hk != 0) return HDT_E_INVALID;
    if (m.gdn_dk != m.gdn_dv || (m.gdn_dk != 64 && m.gdn_dk != 128)) return HDT_E_UNSUPPORTED;
  }
  if (m.gdn_conv < 0) return HDT_E_INVALID;
  if (m.gdn_conv > kConvMaxWidth) return HDT_E_UNSUPPORTED;
  if (m.gdn_conv > 0 && n_gdn > 0 && (!m.gdn_conv_weight || !aligned16(m.gdn_conv_weight)))
    return HDT_E_INVALID;
  if (n_attn > 0) {
    if (m.attn_hkv < 1 || m.attn_hq < m.attn_hkv || m.attn_hq % m.attn_hkv != 0)
      return HDT_E_INVALID;
    if (m.attn_hq / m.attn_hkv > 16) return HDT_E_UNSUPPORTED;
    // bf16 storage: one fold thread per (q head, column pair) of a quarter row block
    if (m.io_dtype == HDT_BF16 && (m.attn_hq / m.attn_hkv) * (m.attn_d / 8) > 192) return HDT_E_UNSUPPORTED;
    if (m.attn_d != 64 && m.attn_d != 256) return HDT_E_UNSUPPORTED;
    if (m.io_dtype == HDT_F32 && m.attn_d != 64) return HDT_E_UNSUPPORTED;
  }
  for (int i = 0; i < n_slots; ++i) {
    const hdt_slot_desc &s = slots[i];
    if (s.capacity < 1 || s.length < 0 || s.length > s.capacity) return HDT_E_INVALID;
    if (s.capacity > (int64_t(1) << 31)) return HDT_E_UNSUPPORTED;
    // buffer resources address one kv head's rows with 32-bit byte offsets
    if (n_attn > 0 && s.capacity * m.attn_d * (m.io_dtype == HDT_BF16 ? 2 : 4) > INT32_MAX)
      return HDT_E_UNSUPPORTED;
    if (n_gdn > 0 && (!s.gdn_state || !aligned16(s.gdn_state))) return HDT_E_INVALID;
    if (n_gdn > 0 && m.gdn_conv > 1 && (!s.gdn_conv_state || !aligned16(s.gdn_conv_state)))
      return HDT_E_INVALID;
    if (n_attn > 0 && (!s.k_cache || !s.v_cache || !aligned16(s.k_cache) || !aligned16(s.v_cache)))
      return HDT_E_INVALID;
  }
  hdt_engine *e = new (std::nothrow) hdt_engine();
  if (!e) return HDT_E_INVALID;
  e->desc = m;
  e->kind.assign(m.layer_kind, m.layer_kind + m.n_layers);
  e->desc.layer_kind = e->kind.data();
  if (e->desc.gdn_scale <= 0.0f && n_gdn > 0) e->desc.gdn_scale = 1.0f / std::sqrt(float(m.gdn_dk));
  if (e->desc.attn_scale <= 0.0f && n_attn > 0) e->desc.attn_scale = 1.0f / std::sqrt(float(m.attn_d));
  e->n_gdn = n_gdn;
  e->n_attn = n_attn;
  e->esz = m.io_dtype == HDT_BF16 ? 2 : 4;
  if (n_gdn == 0) e->desc.gdn_conv = 0;
  e->conv_C = n_gdn > 0 ? 2 * m.gdn_hk * m.gdn_dk + m.gdn_hv * m.gdn_dv : 0;
  int gi = 0, ai = 0;
  for (int l = 0; l < m.n_layers; ++l) e->kind_index.push_back(m.layer_kind[l] == 0 ? gi++ : ai++);
  e->slots.resize(n_slots);
  int64_t max_cap = 1;
  for (int i = 0; i < n_slots; ++i) max_cap = std::max(max_cap, slots[i].capacity);
  if (m.io_dtype == HDT_BF16) {
    e->kv_per_head = kv_per_head(m);
    e->kv_ladder = kv_ladder(max_cap, e->kv_per_head);
  }
  for (int i = 0; i < n_slots; ++i) {
    SlotState &s = e->slots[i];
    s.d = slots[i];
    if (m.io_dtype == HDT_BF16) {  // splits per row position: at most per_head of them
      s.split = 0;
      s.nsplit_cap = static_cast<int32_t>(e->kv_per_head);
    } else {
      s.split = split_for(s.d.capacity, std::max(1, m.attn_hkv));
      s.nsplit_cap = static_cast<int32_t>((s.d.capacity + s.split - 1) / s.split);
    }
  }
  *out = e;
  return HDT_OK;
}

void hdt_destroy(hdt_engine *e) {
  if (!e) return;
  if (e->allocated || e->pf.allocated || !e->ev_live.empty() || !e->ev_pool.empty()) (void)hipDeviceSynchronize();
  free_scratch(e);
  for (auto &p : e->ev_live) {
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  for (auto &p : e->ev_pool) {
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  delete e;
}

}  // extern "C"

// A reusable graph of the verify pass: two instantiated graphs used in turn, each with
// the event recorded after its last launch.
struct hdt_graph {
  hdt_engine *e = nullptr;
  hipStream_t cap = nullptr;  // the private stream the pass is captured on
  hipGraphExec_t exec[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
  bool launched[2] = {false, false};
  int next = 0;
  int64_t instantiations = 0, updates = 0;
};

namespace {

// The pass as one graph launch: captured on the graph's stream, then either an update in
// place of the instantiated graph whose turn it is (same kernel sequence) or a new
// instantiation.  That graph is touched only once its previous launch has finished.
hdt_status launch_graph(hdt_engine *e, hdt_graph *g, int32_t n_trees, const hdt_tree *trees,
                        const int8_t (*par)[kMaxNodes], const int8_t (*dep)[kMaxNodes], hipStream_t stream) {
  const int k = g->next;
  if (g->launched[k] && hipEventSynchronize(g->done[k]) != hipSuccess)
    return fail(e, HDT_E_HIP, "waiting for the graph's previous launch failed");
  if (hipStreamBeginCapture(g->cap, hipStreamCaptureModeThreadLocal) != hipSuccess)
    return fail(e, HDT_E_HIP, "graph capture could not begin");
  const hdt_status st = launch_forward(e, n_trees, trees, par, dep, g->cap);
  hipGraph_t graph = nullptr;
  const hipError_t ce = hipStreamEndCapture(g->cap, &graph);
  if (st != HDT_OK || ce != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return st != HDT_OK ? st : fail(e, HDT_E_HIP, "graph capture failed");
  }
  if (g->exec[k]) {
    hipGraphNode_t bad = nullptr;
    hipGraphExecUpdateResult res = hipGraphExecUpdateError;
    if (hipGraphExecUpdate(g->exec[k], graph, &bad, &res) == hipSuccess && res == hipGraphExecUpdateSuccess) {
      ++g->updates;
    } else {
      (void)hipGetLastError();  // a refused update is not an error of the pass
      (void)hipGraphExecDestroy(g->exec[k]);
      g->exec[k] = nullptr;
    }
  }
  if (!g->exec[k]) {
    if (hipGraphInstantiate(&g->exec[k], graph, nullptr, nullptr, 0) != hipSuccess) {
      g->exec[k] = nullptr;
      (void)hipGraphDestroy(graph);
      return fail(e, HDT_E_HIP, "graph instantiation failed");
    }
    ++g->instantiations;
  }
  (void)hipGraphDestroy(graph);
  if (check_hip(e, hipGraphLaunch(g->exec[k], stream), "graph launch") != HDT_OK) return HDT_E_HIP;
  if (check_hip(e, hipEventRecord(g->done[k], stream), "graph event") != HDT_OK) return HDT_E_HIP;
  g->launched[k] = true;
  g->next = 1 - k;
  return HDT_OK;
}

// forward_tree with the engine's own scratch (allocated at the first call), or with
// `noalloc` the scratch carved from the library's static array of the current device;
// with `g` the kernels go out as one launch of that reusable graph.
hdt_status forward_trees(hdt_engine *e, int32_t n_trees, const hdt_tree *trees, void *stream, bool noalloc,
                         hdt_graph *g = nullptr) {
  if (!e) return HDT_E_INVALID;
  if (n_trees < 1 || n_trees > HDT_MAX_TREES || !trees)
    return fail(e, HDT_E_INVALID, "n_trees must be 1..%d", HDT_MAX_TREES);
  const hdt_model_desc &m = e->desc;
  int8_t par[HDT_MAX_TREES][kMaxNodes];
  int8_t dep[HDT_MAX_TREES][kMaxNodes];
  int32_t chain[HDT_MAX_TREES];
  for (int t = 0; t < n_trees; ++t) {
    const hdt_tree &tr = trees[t];
    if (tr.slot < 0 || tr.slot >= static_cast<int32_t>(e->slots.size()))
      return fail(e, HDT_E_INVALID, "tree %d: slot %d out of range", t, tr.slot);
    for (int u = 0; u < t; ++u)
      if (trees[u].slot == tr.slot) return fail(e, HDT_E_INVALID, "slot %d appears twice", tr.slot);
    if (settle(e, tr.slot) != HDT_OK) return HDT_E_HIP;
    const SlotState &s = e->slots[tr.slot];
    if (s.pending) return fail(e, HDT_E_ORDER, "slot %d has a pending round", tr.slot);
    if (tr.n_nodes < 1 || tr.n_nodes > m.max_nodes)
      return fail(e, HDT_E_INVALID, "tree %d: %d nodes (max_nodes %d)", t, tr.n_nodes, m.max_nodes);
    std::memset(par[t], 0, kMaxNodes);
    std::memset(dep[t], 0, kMaxNodes);
    if (!plan_tree(tr.n_nodes, tr.parent, par[t], dep[t], &chain[t]))
      return fail(e, HDT_E_TREE, "tree %d: parent array is not a tree", t);
    if (s.d.length + tr.n_nodes > s.d.capacity)
      return fail(e, HDT_E_CAPACITY, "slot %d: length %lld + %d nodes exceeds capacity %lld",
                  tr.slot, (long long)s.d.length, tr.n_nodes, (long long)s.d.capacity);
    if (!tr.io) return fail(e, HDT_E_INVALID, "tree %d: io is NULL", t);
    for (int l = 0; l < m.n_layers; ++l) {
      const hdt_layer_io &io = tr.io[l];
      if (!io.q || !io.k || !io.v || !io.o)
        return fail(e, HDT_E_INVALID, "tree %d layer %d: NULL q/k/v/o", t, l);
      if (e->kind[l] == 0 && (!io.alpha || !io.beta))
        return fail(e, HDT_E_INVALID, "tree %d layer %d: NULL alpha/beta", t, l);
      if (e->kind[l] == 0 && m.gdn_conv > 0 && (!aligned16(io.q) || !aligned16(io.k) || !aligned16(io.v)))
        return fail(e, HDT_E_INVALID, "tree %d layer %d: conv inputs must be 16-byte aligned", t, l);
      if (e->kind[l] == 1 && (!aligned16(io.q) || !aligned16(io.k) || !aligned16(io.v) ||
                              !aligned16(io.o)))
        return fail(e, HDT_E_INVALID, "tree %d layer %d: attention buffers must be 16-byte aligned",
                    t, l);
    }
  }
  hdt_status st = HDT_OK;
  Scratch carved[HDT_MAX_TREES];
  int dev = 0;
  uint64_t gen = 0;
  if (noalloc) {
    size_t need = 0;
    for (int t = 0; t < n_trees; ++t) need += scratch_bytes(e, e->slots[trees[t].slot]);
    if (need > kStaticScratchBytes)
      return fail(e, HDT_E_CAPACITY, "the pass needs %zu bytes of scratch; the static scratch holds %zu",
                  need, static_cast<size_t>(kStaticScratchBytes));
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
      return fail(e, HDT_E_HIP, "no current HIP device");
    void *base = nullptr;
    if (check_hip(e, static_scratch_address(&base), "resolving the static scratch") != HDT_OK) return HDT_E_HIP;
    st = query_lds(e);
    if (st != HDT_OK) return st;
    size_t off = 0;
    for (int t = 0; t < n_trees; ++t) {
      size_t b[kScratchParts];
      scratch_sizes(e, e->slots[trees[t].slot], b);
      for (int i = 0; i < kScratchParts; ++i) {
        *scratch_part(carved[t], i) = b[i] > 0 ? static_cast<char *>(base) + off : nullptr;
        off += align256(b[i]);
      }
    }
    std::lock_guard<std::mutex> lock(g_static_mu);
    gen = ++g_static_gen[dev];
  } else {
    if (!e->allocated) {
      // the scratch is allocated by the first forward, which must not be captured
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess ||
          cs != hipStreamCaptureStatusNone)
        return fail(e, HDT_E_ORDER, "the first forward allocates scratch: run it outside graph capture");
    }
    st = ensure_alloc(e);
    if (st != HDT_OK) return st;
  }
  for (int t = 0; t < n_trees; ++t) {
    SlotState &s = e->slots[trees[t].slot];
    s.sc = noalloc ? carved[t] : s.own;
    s.static_dev = noalloc ? dev : -1;
    s.static_gen = gen;
  }
  {
    int32_t n_max = 0;
    for (int t = 0; t < n_trees; ++t) n_max = std::max(n_max, trees[t].n_nodes);
    const size_t need_g = e->n_gdn > 0 ? gdn_lds_bytes(m.gdn_dk, n_max, kGdnSaves, 1) : 0;
    const size_t need_a = e->n_attn > 0 ? attn_lds_bytes(m.attn_d, m.io_dtype == HDT_BF16, n_max) : 0;
    if (need_g > static_cast<size_t>(e->max_lds) || need_a > static_cast<size_t>(e->max_lds))
      return fail(e, HDT_E_UNSUPPORTED, "kernels need %zu / %zu bytes of LDS; the device allows %d",
                  need_g, need_a, e->max_lds);
  }
  e->no_events = noalloc || g;  // a noalloc or graph call creates no profiling events either
  st = g ? launch_graph(e, g, n_trees, trees, par, dep, static_cast<hipStream_t>(stream))
         : launch_forward(e, n_trees, trees, par, dep, static_cast<hipStream_t>(stream));
  e->no_events = false;
  if (st != HDT_OK) return st;
  for (int t = 0; t < n_trees; ++t) {
    SlotState &s = e->slots[trees[t].slot];
    s.pending = true;
    s.n = trees[t].n_nodes;
    s.chain = chain[t];
    std::memcpy(s.parent, par[t], kMaxNodes);
    std::memcpy(s.depth, dep[t], kMaxNodes);
  }
  e->err.clear();
  return HDT_OK;
}

}  // namespace

extern "C" {

hdt_status hdt_forward_tree(hdt_engine *e, int32_t n_trees, const hdt_tree *trees, void *stream) {
  return forward_trees(e, n_trees, trees, stream, false);
}

hdt_status hdt_forward_tree_noalloc(hdt_engine *e, int32_t n_trees, const hdt_tree *trees, void *stream) {
  return forward_trees(e, n_trees, trees, stream, true);
}

hdt_status hdt_graph_create(hdt_engine *e, hdt_graph **out) {
  if (!e || !out) return HDT_E_INVALID;
  *out = nullptr;
  hdt_graph *g = new (std::nothrow) hdt_graph;
  if (!g) return fail(e, HDT_E_INVALID, "out of host memory");
  g->e = e;
  bool ok = hipStreamCreateWithFlags(&g->cap, hipStreamNonBlocking) == hipSuccess;
  for (int k = 0; k < 2 && ok; ++k) ok = hipEventCreateWithFlags(&g->done[k], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    hdt_graph_destroy(g);
    return fail(e, HDT_E_HIP, "graph stream or events could not be created");
  }
  *out = g;
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_graph_forward(hdt_graph *g, int32_t n_trees, const hdt_tree *trees, void *stream) {
  if (!g || !g->e) return HDT_E_INVALID;
  return forward_trees(g->e, n_trees, trees, stream, false, g);
}

hdt_status hdt_graph_stats(const hdt_graph *g, int64_t *instantiations, int64_t *updates) {
  if (!g || !instantiations || !updates) return HDT_E_INVALID;
  *instantiations = g->instantiations;
  *updates = g->updates;
  return HDT_OK;
}

void hdt_graph_destroy(hdt_graph *g) {
  if (!g) return;
  for (int k = 0; k < 2; ++k) {
    if (g->launched[k]) (void)hipEventSynchronize(g->done[k]);
    if (g->exec[k]) (void)hipGraphExecDestroy(g->exec[k]);
    if (g->done[k]) (void)hipEventDestroy(g->done[k]);
  }
  if (g->cap) (void)hipStreamDestroy(g->cap);
  delete g;
}

hdt_status hdt_forward_block(hdt_engine *e, int32_t slot, int32_t n, const hdt_layer_io *io,
                             void *stream) {
  if (!e) return HDT_E_INVALID;
  if (n < 1 || n > HDT_MAX_NODES) return fail(e, HDT_E_INVALID, "block of %d tokens", n);
  int32_t parent[HDT_MAX_NODES];
  for (int i = 0; i < n; ++i) parent[i] = i - 1;
  hdt_tree t{slot, n, parent, io};
  return hdt_forward_tree(e, 1, &t, stream);
}

hdt_status hdt_commit_tree(hdt_engine *e, int32_t slot, const int32_t *path, int32_t m,
                           void *stream) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  if (!s.pending) return fail(e, HDT_E_ORDER, "slot %d has no pending round", slot);
  if (check_round_scratch(e, s) != HDT_OK) return HDT_E_ORDER;
  if (!path || m < 1 || m > s.n) return fail(e, HDT_E_PATH, "path length %d (tree of %d)", m, s.n);
  if (path[0] != 0) return fail(e, HDT_E_PATH, "path must start at the root");
  for (int d = 1; d < m; ++d)
    if (path[d] < 0 || path[d] >= s.n || s.parent[path[d]] != path[d - 1])
      return fail(e, HDT_E_PATH, "path[%d] = %d is not a child of %d", d, path[d], path[d - 1]);
  if (commit_lds_bytes(e->desc.attn_d, e->desc.io_dtype == HDT_BF16, m) > static_cast<size_t>(e->max_lds))
    return fail(e, HDT_E_UNSUPPORTED, "commit of %d rows needs more LDS than the device allows", m);
  hdt_status st = do_commit(e, slot, path, m, nullptr, static_cast<hipStream_t>(stream));
  if (st != HDT_OK) return st;
  s.d.length += m;
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_rollback_to(hdt_engine *e, int32_t slot, int64_t n, void *stream) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  const int64_t L = s.d.length;
  if (n < L) {
    const int64_t k = s.anchor_every > 0 && n % s.anchor_every == 0 ? n / s.anchor_every - 1 : -1;
    if (k < 0 || k >= s.anchor_n || !s.anchor_ok[k])
      return fail(e, HDT_E_UNSUPPORTED, "rollback to %lld below the committed length needs an anchor there",
                  (long long)n);
    hdt_status st = anchor_copy(e, slot, static_cast<int32_t>(k), false, static_cast<hipStream_t>(stream));
    if (st != HDT_OK) return st;
    for (int32_t j = static_cast<int32_t>(k) + 1; j < s.anchor_n; ++j) s.anchor_ok[j] = false;
    s.d.length = n;
    s.pending = false;
    e->err.clear();
    return HDT_OK;
  }
  if (n == L) {
    s.pending = false;
    e->err.clear();
    return HDT_OK;
  }
  if (!s.pending) return fail(e, HDT_E_ORDER, "rollback_to(%lld) past length %lld with no pending round",
                              (long long)n, (long long)L);
  if (n > L + s.chain)
    return fail(e, HDT_E_INVALID, "rollback_to(%lld): only the leading chain of %d can be kept",
                (long long)n, s.chain);
  if (check_round_scratch(e, s) != HDT_OK) return HDT_E_ORDER;
  int32_t path[HDT_MAX_NODES];
  const int32_t m = static_cast<int32_t>(n - L);
  for (int d = 0; d < m; ++d) path[d] = d;
  hdt_status st = do_commit(e, slot, path, m, nullptr, static_cast<hipStream_t>(stream));
  if (st != HDT_OK) return st;
  s.d.length += m;
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_forward_span(hdt_engine *e, int32_t slot, int32_t T, const hdt_layer_io *io, void *stream) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (T < 1 || !io) return fail(e, HDT_E_INVALID, "span of %d tokens", T);
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  const hdt_model_desc &m = e->desc;
  if (s.pending) return fail(e, HDT_E_ORDER, "slot %d has a pending round", slot);
  if (s.d.length + T > s.d.capacity)
    return fail(e, HDT_E_CAPACITY, "slot %d: length %lld + %d tokens exceeds capacity %lld", slot,
                (long long)s.d.length, T, (long long)s.d.capacity);
  for (int l = 0; l < m.n_layers; ++l) {
    const hdt_layer_io &x = io[l];
    if (!x.q || !x.k || !x.v || !x.o) return fail(e, HDT_E_INVALID, "layer %d: NULL q/k/v/o", l);
    if (e->kind[l] == 0 && (!x.alpha || !x.beta)) return fail(e, HDT_E_INVALID, "layer %d: NULL alpha/beta", l);
    if (e->kind[l] == 1 && (!aligned16(x.q) || !aligned16(x.k) || !aligned16(x.v) || !aligned16(x.o)))
      return fail(e, HDT_E_INVALID, "layer %d: attention buffers must be 16-byte aligned", l);
    if (e->kind[l] == 0 && m.gdn_conv > 0 && (!aligned16(x.q) || !aligned16(x.k) || !aligned16(x.v)))
      return fail(e, HDT_E_INVALID, "layer %d: conv inputs must be 16-byte aligned", l);
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!e->allocated) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return fail(e, HDT_E_ORDER, "the first forward allocates scratch: run it outside graph capture");
  }
  hdt_status r = ensure_alloc(e);
  if (r != HDT_OK) return r;
  s.sc = s.own;
  s.static_dev = -1;
  s.static_gen = 0;
  if (gdn_lds_bytes(m.gdn_dk, m.max_nodes, kGdnSaves, 1) > static_cast<size_t>(e->max_lds) && e->n_gdn > 0)
    return fail(e, HDT_E_UNSUPPORTED, "a chain of %d needs more LDS than the device allows", m.max_nodes);
  // bytes per row of each io array, by layer kind
  const size_t z = e->esz;
  int32_t chain[kMaxNodes], path[kMaxNodes];
  for (int i = 0; i < kMaxNodes; ++i) {
    chain[i] = i - 1;
    path[i] = i;
  }
  std::vector<hdt_layer_io> cio(m.n_layers);
  for (int32_t t0 = 0; t0 < T;) {
    int32_t c = std::min<int32_t>(m.max_nodes, T - t0);
    if (s.anchor_every > 0) {  // end a chain at every anchor position
      const int64_t next = (s.d.length / s.anchor_every + 1) * s.anchor_every;
      c = static_cast<int32_t>(std::min<int64_t>(c, next - s.d.length));
    }
    for (int l = 0; l < m.n_layers; ++l) {
      const hdt_layer_io &x = io[l];
      const size_t t = static_cast<size_t>(t0);
      size_t bq, bk, bv, bo, bg = 0;
      if (e->kind[l] == 0) {
        bq = bk = static_cast<size_t>(m.gdn_hk) * m.gdn_dk * z;
        bv = bo = static_cast<size_t>(m.gdn_hv) * m.gdn_dv * z;
        bg = static_cast<size_t>(m.gdn_hv) * z;
      } else {
        bq = bo = static_cast<size_t>(m.attn_hq) * m.attn_d * z;
        bk = bv = static_cast<size_t>(m.attn_hkv) * m.attn_d * z;
      }
      cio[l].q = static_cast<const char *>(x.q) + t * bq;
      cio[l].k = static_cast<const char *>(x.k) + t * bk;
      cio[l].v = static_cast<const char *>(x.v) + t * bv;
      cio[l].o = static_cast<char *>(x.o) + t * bo;
      cio[l].alpha = x.alpha ? static_cast<const char *>(x.alpha) + t * bg : nullptr;
      cio[l].beta = x.beta ? static_cast<const char *>(x.beta) + t * bg : nullptr;
    }
    int8_t par[1][kMaxNodes], dep[1][kMaxNodes];
    int32_t cl;
    std::memset(par, 0, sizeof par);
    std::memset(dep, 0, sizeof dep);
    plan_tree(c, chain, par[0], dep[0], &cl);
    const hdt_tree tr{slot, c, chain, cio.data()};
    r = launch_forward(e, 1, &tr, par, dep, st, /*chain_commit=*/true);
    if (r != HDT_OK) return r;
    s.n = c;
    std::memcpy(s.parent, par[0], kMaxNodes);
    std::memcpy(s.depth, dep[0], kMaxNodes);
    // the walk wrote each GDN layer's final state and the tree pass wrote the rows in
    // chain order at L..L+c-1: only the conv tails remain to be rolled
    r = do_commit(e, slot, path, c, nullptr, st, /*tails_only=*/true);
    if (r != HDT_OK) return r;
    s.d.length += c;
    if (s.anchor_every > 0 && s.d.length % s.anchor_every == 0) {
      const int64_t k = s.d.length / s.anchor_every - 1;
      if (k < s.anchor_n) {
        r = anchor_copy(e, slot, static_cast<int32_t>(k), true, st);
        if (r != HDT_OK) return r;
      }
    }
    t0 += c;
  }
  e->err.clear();
  return HDT_OK;
}

}  // extern "C"

namespace {

// Key splits of a prefill attention layer with `tiles_heads` (row tile, kv head) pairs:
// enough for about kPfItems workgroups (a few per CU, so that none waits on a last one),
// at most kPfMaxSplits.  The split itself is then rounded up to whole tiles, which can
// only lower the count.
int32_t pf_splits(int32_t tiles_heads) {
  return std::max(1, std::min(kPfMaxSplits, (kPfItems + tiles_heads - 1) / tiles_heads));
}

// Sizes of the chunked-prefill scratch for one piece of kPfPiece tokens.
struct PfSizes {
  size_t w, mq, kq, ut, g, acc, ml, conv;
};
PfSizes pf_sizes(const hdt_model_desc &m) {
  const size_t nch = kPfPiece / kWyChunk + 1, C = kWyChunk;
  PfSizes z{};
  if (m.gdn_hv > 0) {
    z.w = nch * m.gdn_hv * C * m.gdn_dk * 2;
    z.mq = nch * m.gdn_hv * C * C * 2;
    z.kq = nch * m.gdn_hk * C * m.gdn_dk * 2;
    z.ut = nch * m.gdn_hv * C * m.gdn_dv * 4;
    z.g = nch * m.gdn_hv * 3 * C * 4;
    if (m.gdn_conv > 0)
      z.conv = static_cast<size_t>(kPfPiece) * (2 * m.gdn_hk * m.gdn_dk + m.gdn_hv * m.gdn_dv) *
               (m.io_dtype == HDT_BF16 ? 2 : 4);
  }
  if (m.attn_hkv > 0) {
    const size_t G = m.attn_hq / m.attn_hkv;
    // the most (kv head, split, row tile) items any piece length takes
    size_t items = 0;
    for (int32_t p = 1; p <= kPfPiece; ++p) {
      const int32_t th = static_cast<int32_t>((p * G + kPfRows - 1) / kPfRows) * m.attn_hkv;
      items = std::max(items, static_cast<size_t>(th) * pf_splits(th));
    }
    z.acc = items * kPfRows * m.attn_d * 4;
    z.ml = items * kPfRows * 2 * 4;
  }
  return z;
}

hdt_status ensure_pf_alloc(hdt_engine *e) {
  if (e->pf.allocated) return HDT_OK;
  const PfSizes z = pf_sizes(e->desc);
  struct {
    void **p;
    size_t n;
  } parts[] = {{reinterpret_cast<void **>(&e->pf.w_hi), z.w},   {reinterpret_cast<void **>(&e->pf.w_lo), z.w},
               {reinterpret_cast<void **>(&e->pf.mq_hi), z.mq}, {reinterpret_cast<void **>(&e->pf.mq_lo), z.mq},
               {reinterpret_cast<void **>(&e->pf.kt), z.kq},    {reinterpret_cast<void **>(&e->pf.qc), z.kq},
               {reinterpret_cast<void **>(&e->pf.ut), z.ut},    {reinterpret_cast<void **>(&e->pf.g), z.g},
               {reinterpret_cast<void **>(&e->pf.part_acc), z.acc},
               {reinterpret_cast<void **>(&e->pf.part_ml), z.ml},
               {&e->pf.conv, z.conv}};
  for (auto &x : parts)
    if (x.n > 0 && hipMalloc(x.p, x.n) != hipSuccess) return fail(e, HDT_E_HIP, "hipMalloc of the prefill scratch failed");
  e->pf.allocated = true;
  return HDT_OK;
}

// One piece of p tokens (span rows [t0, t0 + p)) through every layer, in layer order.
hdt_status chunked_piece(hdt_engine *e, SlotState &s, const hdt_layer_io *io, int32_t t0, int32_t p,
                         hipStream_t st) {
  const hdt_model_desc &m = e->desc;
  const size_t z = e->esz, t = static_cast<size_t>(t0);
  const int64_t L = s.d.length;
  for (int l = 0; l < m.n_layers; ++l) {
    const hdt_layer_io &x = io[l];
    const int32_t ki = e->kind_index[l];
    if (e->kind[l] == 0) {
      const size_t bqk = static_cast<size_t>(m.gdn_hk) * m.gdn_dk * z, bv = static_cast<size_t>(m.gdn_hv) * m.gdn_dv * z,
                   bg = static_cast<size_t>(m.gdn_hv) * z;
      WyPrep a{};
      a.q = static_cast<const char *>(x.q) + t * bqk;
      a.k = static_cast<const char *>(x.k) + t * bqk;
      a.v = static_cast<const char *>(x.v) + t * bv;
      if (m.gdn_conv > 0) {
        // the short conv over the piece after the layer's tail; the WY kernels read its
        // output, and the tail rolls to the piece's last rows
        PfConv c{};
        c.q = a.q;
        c.k = a.k;
        c.v = a.v;
        c.tail = static_cast<char *>(s.d.gdn_conv_state) +
                 static_cast<size_t>(ki) * (m.gdn_conv - 1) * e->conv_C * z;
        c.qo = e->pf.conv;
        c.ko = static_cast<char *>(e->pf.conv) + static_cast<size_t>(p) * bqk;
        c.vo = static_cast<char *>(e->pf.conv) + 2 * static_cast<size_t>(p) * bqk;
        c.weight = m.gdn_conv_weight + static_cast<size_t>(ki) * e->conv_C * m.gdn_conv;
        c.T = p;
        c.width = m.gdn_conv;
        c.hk = m.gdn_hk;
        c.dk = m.gdn_dk;
        c.hv = m.gdn_hv;
        c.dv = m.gdn_dv;
        c.eps = kConvEps;
        {
          ProfScope ps(e, 4);
          if (launch_pf_conv(c, m.io_dtype == HDT_BF16, st, ps.events()) != hipSuccess)
            return fail(e, HDT_E_HIP, "layer %d: span conv launch failed", l);
        }
        a.q = c.qo;
        a.k = c.ko;
        a.v = c.vo;
      }
      a.alpha = static_cast<const char *>(x.alpha) + t * bg;
      a.beta = static_cast<const char *>(x.beta) + t * bg;
      a.T = p;
      a.off = static_cast<int32_t>(L % kWyChunk);
      a.n_chunks = (a.off + p + kWyChunk - 1) / kWyChunk;
      a.hk = m.gdn_hk;
      a.hv = m.gdn_hv;
      a.scale = m.gdn_scale;
      a.w_hi = e->pf.w_hi;
      a.w_lo = e->pf.w_lo;
      a.mq_hi = e->pf.mq_hi;
      a.mq_lo = e->pf.mq_lo;
      a.kt = e->pf.kt;
      a.qc = e->pf.qc;
      a.ut = e->pf.ut;
      a.g = e->pf.g;
      {
        ProfScope ps(e, 6);
        if (launch_wy_prep(a, m.gdn_dk, st, ps.events()) != hipSuccess)
          return fail(e, HDT_E_HIP, "layer %d: WY prep launch failed", l);
      }
      WyScan b{};
      b.w_hi = a.w_hi;
      b.w_lo = a.w_lo;
      b.mq_hi = a.mq_hi;
      b.mq_lo = a.mq_lo;
      b.kt = a.kt;
      b.qc = a.qc;
      b.ut = a.ut;
      b.g = a.g;
      b.state = s.d.gdn_state + static_cast<size_t>(ki) * m.gdn_hv * m.gdn_dv * m.gdn_dk;
      b.o = static_cast<char *>(x.o) + t * bv;
      b.T = p;
      b.off = a.off;
      b.n_chunks = a.n_chunks;
      b.hk = m.gdn_hk;
      b.hv = m.gdn_hv;
      ProfScope ps(e, 7);
      if (launch_wy_scan(b, m.gdn_dk, st, ps.events()) != hipSuccess)
        return fail(e, HDT_E_HIP, "layer %d: WY scan launch failed", l);
    } else {
      const size_t bq = static_cast<size_t>(m.attn_hq) * m.attn_d * z, bk = static_cast<size_t>(m.attn_hkv) * m.attn_d * z;
      const size_t view = static_cast<size_t>(m.attn_hkv) * s.d.capacity * m.attn_d * z;
      PfCopy c{};
      c.k = static_cast<const char *>(x.k) + t * bk;
      c.v = static_cast<const char *>(x.v) + t * bk;
      c.kc = static_cast<char *>(s.d.k_cache) + static_cast<size_t>(ki) * view;
      c.vc = static_cast<char *>(s.d.v_cache) + static_cast<size_t>(ki) * view;
      c.cap = s.d.capacity;
      c.L = L;
      c.T = p;
      c.hkv = m.attn_hkv;
      if (launch_pf_copy(c, m.attn_d, st) != hipSuccess) return fail(e, HDT_E_HIP, "layer %d: row copy failed", l);
      PfAttn a{};
      const int32_t G = m.attn_hq / m.attn_hkv;
      a.q = static_cast<const char *>(x.q) + t * bq;
      a.kc = c.kc;
      a.vc = c.vc;
      a.o = static_cast<char *>(x.o) + t * bq;
      a.part_acc = e->pf.part_acc;
      a.part_ml = e->pf.part_ml;
      a.cap = s.d.capacity;
      a.L = L;
      a.T = p;
      a.hq = m.attn_hq;
      a.hkv = m.attn_hkv;
      a.row_tiles = (p * G + kPfRows - 1) / kPfRows;
      a.rows_cap = a.row_tiles * kPfRows;
      const int32_t tiles_heads = a.row_tiles * m.attn_hkv;
      a.nsplit = pf_splits(tiles_heads);
      const int64_t keys = L + p;
      a.split = static_cast<int32_t>(((keys + a.nsplit - 1) / a.nsplit + kKvTile - 1) / kKvTile * kKvTile);
      a.nsplit = static_cast<int32_t>((keys + a.split - 1) / a.split);
      a.items = (tiles_heads * a.nsplit + 7) / 8 * 8;
      a.c2 = m.attn_scale * 1.4426950408889634f;
      {
        ProfScope ps(e, 8);
        if (launch_pf_attn(a, m.attn_d, st, ps.events()) != hipSuccess)
          return fail(e, HDT_E_HIP, "layer %d: prefill attention launch failed", l);
      }
      if (a.nsplit > 1) {
        ProfScope ps(e, 9);
        if (launch_pf_fold(a, m.attn_d, st, ps.events()) != hipSuccess)
          return fail(e, HDT_E_HIP, "layer %d: prefill fold launch failed", l);
      }
    }
  }
  return HDT_OK;
}

}  // namespace

extern "C" {

hdt_status hdt_forward_chunked(hdt_engine *e, int32_t slot, int32_t T, const hdt_layer_io *io, void *stream) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (T < 1 || !io) return fail(e, HDT_E_INVALID, "span of %d tokens", T);
  const hdt_model_desc &m = e->desc;
  if (m.io_dtype != HDT_BF16) return fail(e, HDT_E_UNSUPPORTED, "the chunked prefill needs bf16 storage");
  if (e->n_gdn > 0 && (m.gdn_dk != 128 || m.gdn_dv != 128))
    return fail(e, HDT_E_UNSUPPORTED, "the chunked prefill needs GDN heads of 128 by 128");
  if (e->n_attn > 0 && m.attn_d != 256) return fail(e, HDT_E_UNSUPPORTED, "the chunked prefill needs attn_d = 256");
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  if (s.pending) return fail(e, HDT_E_ORDER, "slot %d has a pending round", slot);
  if (s.d.length + T > s.d.capacity)
    return fail(e, HDT_E_CAPACITY, "slot %d: length %lld + %d tokens exceeds capacity %lld", slot,
                (long long)s.d.length, T, (long long)s.d.capacity);
  for (int l = 0; l < m.n_layers; ++l) {
    const hdt_layer_io &x = io[l];
    if (!x.q || !x.k || !x.v || !x.o) return fail(e, HDT_E_INVALID, "layer %d: NULL q/k/v/o", l);
    if (e->kind[l] == 0 && (!x.alpha || !x.beta)) return fail(e, HDT_E_INVALID, "layer %d: NULL alpha/beta", l);
    if (!aligned16(x.q) || !aligned16(x.k) || !aligned16(x.v) || !aligned16(x.o))
      return fail(e, HDT_E_INVALID, "layer %d: buffers must be 16-byte aligned", l);
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (!e->pf.allocated) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return fail(e, HDT_E_ORDER, "the first chunked prefill allocates scratch: run it outside graph capture");
  }
  hdt_status r = ensure_pf_alloc(e);
  if (r != HDT_OK) return r;
  for (int32_t t0 = 0; t0 < T;) {
    int32_t p = std::min(kPfPiece, T - t0);
    if (s.anchor_every > 0) {  // a piece ends at every anchor position
      const int64_t next = (s.d.length / s.anchor_every + 1) * s.anchor_every;
      p = static_cast<int32_t>(std::min<int64_t>(p, next - s.d.length));
    }
    r = chunked_piece(e, s, io, t0, p, st);
    if (r != HDT_OK) return r;
    s.d.length += p;
    if (s.anchor_every > 0 && s.d.length % s.anchor_every == 0) {
      const int64_t k = s.d.length / s.anchor_every - 1;
      if (k < s.anchor_n) {
        r = anchor_copy(e, slot, static_cast<int32_t>(k), true, st);
        if (r != HDT_OK) return r;
      }
    }
    t0 += p;
  }
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_set_anchors(hdt_engine *e, int32_t slot, int64_t every, int32_t n_max, float *state,
                           void *conv) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  SlotState &s = e->slots[slot];
  if (every < 0 || (every > 0 && n_max < 1)) return fail(e, HDT_E_INVALID, "anchors every %lld, %d of them",
                                                         (long long)every, n_max);
  if (every > 0 && e->n_gdn > 0 && (!state || !aligned16(state)))
    return fail(e, HDT_E_INVALID, "anchor state buffer missing or not 16-byte aligned");
  if (every > 0 && conv_tail_bytes(e) > 0 && (!conv || !aligned16(conv)))
    return fail(e, HDT_E_INVALID, "anchor conv buffer missing or not 16-byte aligned");
  s.anchor_every = every;
  s.anchor_n = every > 0 ? n_max : 0;
  s.anchor_state = state;
  s.anchor_conv = conv;
  s.anchor_ok.assign(static_cast<size_t>(s.anchor_n), false);
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_anchor_below(const hdt_engine *e, int32_t slot, int64_t n, int64_t *out) {
  if (!e || !out || slot < 0 || slot >= static_cast<int32_t>(e->slots.size())) return HDT_E_INVALID;
  const SlotState &s = e->slots[slot];
  *out = -1;
  for (int32_t k = s.anchor_n - 1; k >= 0; --k)
    if (s.anchor_ok[k] && (k + 1) * s.anchor_every <= n) {
      *out = (k + 1) * s.anchor_every;
      break;
    }
  return HDT_OK;
}

hdt_status hdt_walk_commit(hdt_engine *e, int32_t slot, const int32_t *draft, const int32_t *target,
                           int32_t *out, void *stream) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (!draft || !target || !out) return fail(e, HDT_E_INVALID, "NULL draft, target or out");
  if ((reinterpret_cast<uintptr_t>(draft) | reinterpret_cast<uintptr_t>(target) |
       reinterpret_cast<uintptr_t>(out)) & 3u)
    return fail(e, HDT_E_INVALID, "token buffers must be 4-byte aligned");
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  if (!s.pending) return fail(e, HDT_E_ORDER, "slot %d has no pending round", slot);
  if (check_round_scratch(e, s) != HDT_OK) return HDT_E_ORDER;
  if (commit_lds_bytes(e->desc.attn_d, e->desc.io_dtype == HDT_BF16, s.n) > static_cast<size_t>(e->max_lds))
    return fail(e, HDT_E_UNSUPPORTED, "commit of %d rows needs more LDS than the device allows", s.n);
  if (ensure_walk(e) != HDT_OK) return HDT_E_HIP;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  WalkLaunch w;
  std::memset(&w, 0, sizeof w);
  w.draft = draft;
  w.target = target;
  w.out = out;
  w.n = s.n;
  for (int i = 0; i < s.n; ++i) w.anc[i] = (i == 0 ? 0 : w.anc[s.parent[i]]) | (uint64_t(1) << i);
  {
    ProfScope p(e, 5);
    hdt_status r = check_hip(e, launch_walk(w, st, p.events()), "accept walk launch");
    if (r != HDT_OK) return r;
  }
  hdt_status r = do_commit(e, slot, nullptr, s.n, out, st);
  if (r != HDT_OK) return r;
  if (hipMemcpyAsync(&e->walk_m[slot], out, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipEventRecord(s.walk_ev, st) != hipSuccess)
    return fail(e, HDT_E_HIP, "recording the accept walk's length failed");
  s.walk_pending = true;
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_kv_length(const hdt_engine *e, int32_t slot, int64_t *out) {
  if (!e || !out || slot < 0 || slot >= static_cast<int32_t>(e->slots.size())) return HDT_E_INVALID;
  // waiting for an accept walk only resolves a length that is already determined
  if (settle(const_cast<hdt_engine *>(e), slot) != HDT_OK) return HDT_E_HIP;
  *out = e->slots[slot].d.length;
  return HDT_OK;
}

hdt_status hdt_reset(hdt_engine *e, int32_t slot, int64_t length) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  if (length < 0 || length > s.d.capacity)
    return fail(e, HDT_E_INVALID, "length %lld outside [0, %lld]", (long long)length,
                (long long)s.d.capacity);
  s.d.length = length;
  s.pending = false;
  for (int32_t j = 0; j < s.anchor_n; ++j)
    if ((j + 1) * s.anchor_every > length) s.anchor_ok[j] = false;
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_state_bytes(const hdt_engine *e, int64_t *out) {
  if (!e || !out) return HDT_E_INVALID;
  *out = snapshot_bytes(e);
  return HDT_OK;
}

hdt_status hdt_state_copy(hdt_engine *e, int32_t slot, void *buf, int64_t buf_bytes, int32_t restore,
                          void *stream) {
  if (!e) return HDT_E_INVALID;
  if (slot < 0 || slot >= static_cast<int32_t>(e->slots.size()))
    return fail(e, HDT_E_INVALID, "slot %d out of range", slot);
  if (!buf || (reinterpret_cast<uintptr_t>(buf) & 255u))
    return fail(e, HDT_E_INVALID, "snapshot buffer missing or not 256-byte aligned");
  const int64_t need = snapshot_bytes(e);
  if (buf_bytes < need)
    return fail(e, HDT_E_INVALID, "snapshot buffer of %lld bytes; the state needs %lld", (long long)buf_bytes,
                (long long)need);
  if (settle(e, slot) != HDT_OK) return HDT_E_HIP;
  SlotState &s = e->slots[slot];
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t sb = static_cast<int64_t>(gdn_state_bytes(e)), cb = static_cast<int64_t>(conv_tail_bytes(e));
  char *state_sec = static_cast<char *>(buf) + kSnapshotHeaderBytes;
  char *conv_sec = state_sec + round256(sb);
  if (!restore) {
    SnapshotHeader h{};
    h.magic = kSnapshotMagic;
    h.signature = shape_signature(e);
    h.length = s.d.length;
    h.state_bytes = sb;
    h.conv_bytes = cb;
    if (check_hip(e, launch_snapshot_header(h, buf, st), "snapshot header launch") != HDT_OK) return HDT_E_HIP;
    if (sb > 0 && hipMemcpyAsync(state_sec, s.d.gdn_state, sb, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return fail(e, HDT_E_HIP, "copy of the state section failed");
    if (cb > 0 && hipMemcpyAsync(conv_sec, s.d.gdn_conv_state, cb, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return fail(e, HDT_E_HIP, "copy of the conv tail section failed");
    e->err.clear();
    return HDT_OK;
  }
  SnapshotHeader h{};
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(&h, buf, sizeof h, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(e, HDT_E_HIP, "reading the snapshot header failed");
  if (h.magic != kSnapshotMagic) return fail(e, HDT_E_INVALID, "the buffer holds no state snapshot");
  if (h.signature != shape_signature(e) || h.state_bytes != sb || h.conv_bytes != cb)
    return fail(e, HDT_E_INVALID, "the snapshot was taken from a model of another shape");
  if (h.length < 0 || h.length > s.d.length)
    return fail(e, HDT_E_INVALID, "the snapshot holds %lld rows; the slot has %lld committed (a restore keeps "
                "rows the cache still holds)", (long long)h.length, (long long)s.d.length);
  if (sb > 0 && hipMemcpyAsync(s.d.gdn_state, state_sec, sb, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return fail(e, HDT_E_HIP, "restore of the state section failed");
  if (cb > 0 && hipMemcpyAsync(s.d.gdn_conv_state, conv_sec, cb, hipMemcpyDeviceToDevice, st) != hipSuccess)
    return fail(e, HDT_E_HIP, "restore of the conv tail section failed");
  s.d.length = h.length;
  s.pending = false;
  for (int32_t j = 0; j < s.anchor_n; ++j)
    if ((j + 1) * s.anchor_every > s.d.length) s.anchor_ok[j] = false;
  e->err.clear();
  return HDT_OK;
}

hdt_status hdt_tree_meta(int32_t n, const int32_t *parent, int64_t L, int32_t *depth,
                         uint64_t *mask, int32_t *anc, int64_t *pos) {
  int8_t par[kMaxNodes], dep[kMaxNodes];
  int32_t chain;
  if (!plan_tree(n, parent, par, dep, &chain)) return HDT_E_TREE;
  uint64_t mk[kMaxNodes];
  for (int i = 0; i < n; ++i) {
    mk[i] = (i == 0 ? 0 : mk[par[i]]) | (uint64_t(1) << i);
    if (depth) depth[i] = dep[i];
    if (mask) mask[i] = mk[i];
    if (pos) pos[i] = L + dep[i];
    if (anc) {
      for (int d = 0; d < kMaxNodes; ++d) anc[i * kMaxNodes + d] = -1;
      for (int x = i; x >= 0; x = par[x]) anc[i * kMaxNodes + dep[x]] = x;
    }
  }
  return HDT_OK;
}

hdt_status hdt_split_size(const hdt_engine *e, int32_t slot, int64_t position, int64_t *out) {
  if (!e || !out || slot < 0 || slot >= static_cast<int32_t>(e->slots.size())) return HDT_E_INVALID;
  const SlotState &s = e->slots[slot];
  if (position < 0 || position >= s.d.capacity) return HDT_E_INVALID;
  *out = e->desc.io_dtype == HDT_BF16 ? kv_split_of(e, position + 1) : s.split;
  return HDT_OK;
}

hdt_status hdt_profile(hdt_engine *e, int32_t enable) {
  if (!e) return HDT_E_INVALID;
  e->profiling = enable != 0;
  return HDT_OK;
}

hdt_status hdt_profile_read(hdt_engine *e, int32_t kind, double *ms, int64_t *launches) {
  if (!e || kind < 0 || kind >= kProfKinds || !ms || !launches) return HDT_E_INVALID;
  for (auto &p : e->ev_live) {
    if (hipEventSynchronize(p.b) != hipSuccess) return fail(e, HDT_E_HIP, "event wait failed");
    float t = 0.0f;
    if (hipEventElapsedTime(&t, p.a, p.b) != hipSuccess) return fail(e, HDT_E_HIP, "event time failed");
    e->prof_ms[p.kind] += t;
    e->prof_count[p.kind] += 1;
    e->ev_pool.push_back(p);
  }
  e->ev_live.clear();
  *ms = e->prof_ms[kind];
  *launches = e->prof_count[kind];
  e->prof_ms[kind] = 0.0;
  e->prof_count[kind] = 0;
  return HDT_OK;
}

const char *hdt_last_error(const hdt_engine *e) { return e ? e->err.c_str() : "no engine"; }

}  // extern "C"
