// launch.h - argument blocks passed by value from the host engine to the kernels.
//
// Every launch covers one layer (or, for commit, every layer) of up to
// kMaxTrees trees; in the tree kernels a workgroup's tree is its grid row
// (blockIdx.y), except in the float32 attention path, which places trees by
// per-tree *_begin offsets along x.  All sizes were validated on the host
// before a block is filled in, so the kernels index without further checks
// beyond what the tree itself bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hdt {

constexpr int kMaxNodes = 64;
constexpr int kMaxTrees = 8;
constexpr int kTile = 64;          // float32 attention: keys per tile, anchored at absolute positions
constexpr int kAttnWaves = 8;      // waves per attention workgroup (float32 storage)
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kKvTile = 32;        // bf16 attention: keys per tile, anchored at absolute positions
constexpr int kKvWaves = 4;        // bf16 attention: waves per tree-pass workgroup, one per SIMD
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kMaxDynamicLds = 160 * 1024;  // gfx950 LDS per workgroup
constexpr int kKvRowsPerItem = 96; // bf16 attention: query rows per split-pass workgroup (6 blocks of 16)
constexpr int kKvStages = 4;       // bf16 attention: LDS tile ring of the split pass
constexpr int kKvQuarters = 4;     // bf16 attention: output columns split over this many blocks
constexpr int kGdnThreads = 256;   // commit: 4 waves
constexpr int kCommitCols = 2;     // commit: 16-column groups per GDN workgroup (state slices per lane)
constexpr int kGdnCols = 16;       // value columns per GDN workgroup
// GDN walk: lanes per value column (16: one DPP row; 32 would put two waves on a
// SIMD, which measured no faster: the per-column reduction work doubles)
constexpr int kGdnLanes = 16;
constexpr int gdn_threads(int dk) { return (void)dk, kGdnCols * kGdnLanes; }
constexpr int kGdnSaves = 8;       // GDN: states kept in LDS for later siblings (branch points)
constexpr int kFoldThreads = 256;  // 4 waves per output row

// ---------------------------------------------------------------- GDN tree walk
struct GdnTree {
  const void *q, *k, *v, *alpha, *beta;  // tree inputs of this layer (io dtype)
  void *o;                               // [n][hv][dv] out
  const float *state;                    // committed state of this layer [hv][dv][dk]
  float *commit_state;                   // non-null (a chain committed whole): the last node's
                                         // state is written here, the same address as `state`
  float *u_pend;                         // [max_nodes][hv][dv]: delta-rule corrections u_i
  void *k_pend;                          // [max_nodes][hk][dk]: copy of k (io dtype)
  void *a_pend;                          // [max_nodes][hv]:     copy of alpha (io dtype)
  int32_t n;
  int32_t need_anc;                      // some restore replays a root path (a branch point
                                         // beyond the kept states): build the ancestor table
  int8_t parent[kMaxNodes];
  int8_t depth[kMaxNodes];
  int8_t save[kMaxNodes];                // LDS slot that keeps node i's state, or -1
  uint64_t restore_mask;                 // bit i: node i's parent is not node i - 1 (the walk
                                         // restores the parent's state before node i)
  uint64_t keep_mask;                    // bit i: save[i] >= 0
};
static_assert(sizeof(GdnTree) <= 384, "a tree descriptor is pulled into the scalar cache whole");

struct GdnLaunch {
  GdnTree t[kMaxTrees];
  int32_t n_trees;
  int32_t hk, hv, dv;
  int32_t n_max;                         // largest n over the trees (sizes LDS)
  int32_t n_saves;                       // largest number of kept states over the trees
  int32_t any_anc;                       // some tree replays a root path (need_anc): LDS holds the
                                         // ancestor table
  float scale;
};

// ---------------------------------------------------------------- GDN short conv
// Depthwise causal convolution of width `width` over each tree node's root path
// (ancestors, then the committed tail before the root), SiLU, and per-head L2
// norm of q and k.  Channels of a token: q (hk*dk), k (hk*dk), v (hv*dv).
constexpr int kConvMaxWidth = 4;
constexpr int kConvThreads = 64;   // one wave: more, smaller workgroups spread the conv over more CUs
constexpr int kPfConvThreads = 256; // the span conv over a prefill piece (8 tokens a thread)
struct ConvTree {
  const void *q, *k, *v;                 // pre-conv inputs [n][hk][dk], [n][hk][dk], [n][hv][dv]
  const void *tail;                      // committed tail of this layer [width-1][C]
  void *qo, *ko, *vo;                    // post-conv outputs, same layouts as the inputs
  void *x_pend;                          // [max_nodes][C]: the tree's pre-conv rows, for commit
  int32_t n;
  int8_t parent[kMaxNodes];
  int8_t depth[kMaxNodes];
};

struct ConvLaunch {
  ConvTree t[kMaxTrees];
  const float *weight;                   // this layer's taps [C][width]
  int32_t n_trees, n_max;
  int32_t width, hk, dk, hv, dv;
  float eps;
};

// The conv over a prefill span of T tokens (rows [0, T) of q, k, v) after the slot's
// tail, in front of the chunked GDN layer; then the tail is rolled to the span's last
// width - 1 rows.
struct PfConv {
  const void *q, *k, *v;                 // pre-conv span rows [T][hk][dk], [T][hk][dk], [T][hv][dv]
  void *tail;                            // this layer's tail [width-1][C], read, then rolled
  void *qo, *ko, *vo;                    // post-conv rows, same layouts as the inputs
  const float *weight;                   // this layer's taps [C][width]
  int32_t T, width, hk, dk, hv, dv;
  float eps;
};

// ---------------------------------------------------------------- attention split pass
// Work items of one tree, in block order: first the tail items (kv head x group of
// up to kAttnWaves nodes), which cover every position from the first split that is
// not wholly committed up to each node's own position; then the shared items
// (kv head x committed split x row group), which cover whole splits below L for every
// (node, q head) row of the kv head at once.
struct AttnTree {
  const void *q;                          // [n][hq][D]
  const void *kt, *vt;                    // tree rows [n][hkv][D]
  void *kc, *vc;                          // cache of this layer [hkv][cap][D]
  float *part_acc;                        // [hkv][nsplit_cap][rows_cap][D]
  float *part_ml;                         // [hkv][nsplit_cap][rows_cap][2]: running max, sum
  int64_t L, cap;
  int32_t n;
  int32_t split;                          // keys per split (multiple of kTile)
  int32_t n_shared;                       // splits wholly below L = L / split
  int32_t nsplit_cap, rows_cap;
  int32_t item_begin;                     // first block of this tree
  int32_t n_tail_items;                   // hkv * node groups
  int32_t tail_nodes;                     // nodes per tail item (one per wave)
  int32_t row_groups;                     // row groups per shared split
  int8_t parent[kMaxNodes];
  int8_t depth[kMaxNodes];
};

struct AttnLaunch {
  AttnTree t[kMaxTrees];
  int32_t n_trees;
  int32_t hq, hkv;
  int32_t n_max;
  float c2;                               // softmax scale times log2(e)
};

// ---------------------------------------------------------------- attention, bf16 storage
// Positions are cut into splits of `split` keys and splits into kKvTile-key tiles,
// both anchored at absolute positions.  A row's split size is a function of its own
// position (the number of keys it sees), so the nodes of one tree can fall on two
// split sizes; each launch pair then covers one group of nodes that share a split
// size (`nodes`, `gn`), and a second pair covers the rest.  The split pass
// (kv_split_kernel) streams every split wholly below L for all (node, q head) rows
// of the group's nodes of a kv head and writes one normalised bf16 partial per
// (row, split); it also runs the tiles of split n_full = L / split that lie below
// tb0 = kKvTile * (L / kKvTile) and leaves their float32 running state (the carry).
// The tree pass (kv_tree_kernel) takes one (kv head, node, column quarter): it
// continues from the carry through the tiles from tb0 to the node's own position,
// whose rows at or past L are the node's ancestors, and folds every split of the
// row in ascending order.  Partial and carry rows are numbered within the group.
struct KvTree {
  const void *q;                          // [n][hq][D]
  const void *kt, *vt;                    // tree rows [n][hkv][D]
  void *kc, *vc;                          // cache of this layer [hkv][cap][D]
  void *o;                                // [n][hq][D]
  void *part_o;                           // bf16 [hkv][nsplit_cap][rows_cap][D]
  float *part_ml;                         // [hkv][nsplit_cap][rows_cap][2]: max (base 2), sum
  float *carry_acc;                       // [hkv][rows_cap][D]
  float *carry_ml;                        // [hkv][rows_cap][2]
  int64_t L, cap;
  int32_t n;                              // nodes of the tree
  int32_t gn;                             // nodes of this launch's group
  int32_t split;                          // keys per split of the group's rows
  int32_t nsplit_cap, rows_cap;
  int32_t n_full;                         // splits wholly below L
  int32_t carry_tiles;                    // tiles of split n_full below tb0
  int32_t row_groups;                     // split pass: row groups of kKvRowsPerItem rows
  int32_t a_splits;                       // split pass: splits per kv head (n_full, + 1 with a carry)
  alignas(4) int8_t parent[kMaxNodes];    // read as 32-bit words
  alignas(4) int8_t depth[kMaxNodes];
  alignas(4) int8_t nodes[kMaxNodes];     // tree index of the group's i-th node
};

struct KvLaunch {
  KvTree t[kMaxTrees];
  int32_t n_trees;
  int32_t hq, hkv;
  float c2;                               // softmax scale times log2(e)
};

// ---------------------------------------------------------------- attention fold
struct FoldTree {
  const float *part_acc, *part_ml;
  void *o;                                // [n][hq][D]
  int64_t L;
  int32_t n, split, nsplit_cap, rows_cap;
  int32_t row_begin;                      // first block: one block per (node, q head)
  int8_t depth[kMaxNodes];
};

struct FoldLaunch {
  FoldTree t[kMaxTrees];
  int32_t n_trees;
  int32_t hq, hkv;
};

// ---------------------------------------------------------------- commit
struct CommitLaunch {
  float *state;                           // [n_gdn][hv][dv][dk]
  const float *u_pend;                    // [n_gdn][max_nodes][hv][dv]
  const void *k_pend;                     // [n_gdn][max_nodes][hk][dk]
  const void *a_pend;                     // [n_gdn][max_nodes][hv]
  void *kc, *vc;                          // [n_attn][hkv][cap][D]
  int64_t L, cap;
  int32_t n_gdn, n_attn, max_nodes;
  int32_t hk, hv, dv;
  int32_t hkv, D;
  int32_t gdn_blocks;                     // blocks [0, gdn_blocks) commit states
  int32_t kv_blocks;                      // then kv_blocks gather K/V rows
  // then conv_blocks roll the conv tails: tail <- last width-1 rows of (tail, path rows)
  void *conv_state;                       // [n_gdn][width-1][C]
  const void *x_pend;                     // [n_gdn][max_nodes][C]
  int32_t conv_width, conv_C, conv_blocks_per_layer;
  int32_t m;
  int8_t path[kMaxNodes];
  const int32_t *dev_out;                 // non-null: m and the path come from the accept
                                          // walk's output {m, bonus, path[m]} instead
};

// ---------------------------------------------------------------- accept walk
struct WalkLaunch {
  const int32_t *draft, *target;          // [n]: each node's token; the model's own next token
  int32_t *out;                           // [2 + n]: m, bonus token, path[m]
  uint64_t anc[kMaxNodes];                // ancestor-or-self bits of each node
  int32_t n;
};

// ---------------------------------------------------------------- state snapshot header
// The first bytes of a state snapshot (hdt_state_copy): written by a one-wave kernel from
// its arguments, read back by the host before a restore.
struct SnapshotHeader {
  uint64_t magic;       // kSnapshotMagic
  uint64_t signature;   // shape of the engine that wrote it
  int64_t length;       // committed rows when it was taken
  int64_t state_bytes;  // GDN state section
  int64_t conv_bytes;   // conv tail section
  int64_t reserved[3];
};
constexpr uint64_t kSnapshotMagic = 0x3150414E53544448ull;  // "HDTSNAP1" little-endian
constexpr int64_t kSnapshotHeaderBytes = 256;                // sections start 256-byte aligned
static_assert(sizeof(SnapshotHeader) == 64, "eight 64-bit words");

// ---------------------------------------------------------------- chunked prefill
// A span of T tokens after the slot's L committed ones.  GDN layers run the chunked
// (WY) form of the delta rule over chunks anchored at absolute multiples of kWyChunk:
// chunk c covers span rows [max(0, kWyChunk c - off), min(T, kWyChunk (c + 1) - off)),
// off = L mod kWyChunk.  Attention layers run causal attention over the cache after
// the span's own rows were copied into it.
constexpr int kWyChunk = 64;
constexpr int kPfRows = 128;   // prefill attention: query rows per workgroup (4 waves x 32)
constexpr int kPfStages = 5;   // prefill attention: LDS tile ring

struct WyPrep {
  const void *q, *k, *v, *alpha, *beta;  // span rows of this layer (bf16)
  int32_t T, off, n_chunks, hk, hv;
  float scale;                           // readout scale s
  uint16_t *w_hi, *w_lo;                 // [n_chunks][hv][64][dk] W = T diag(b g) K, split in two bf16
  uint16_t *mq_hi, *mq_lo;               // [n_chunks][hv][64][64] s (g_i / g_j) q_i.k_j, j <= i
  uint16_t *kt;                          // [n_chunks][hk][dk][64] K transposed, zero past the chunk
  uint16_t *qc;                          // [n_chunks][hk][64][dk] Q, zero past the chunk
  float *ut;                             // [n_chunks][hv][64][dv] U~ = T diag(b) V
  float *g;                              // [n_chunks][hv][3][64] s g_i | g_n / g_j | g_n at [2][0]
};

struct WyScan {
  const uint16_t *w_hi, *w_lo, *mq_hi, *mq_lo, *kt, *qc;
  const float *ut, *g;
  float *state;                          // [hv][dv][dk] this layer's state, advanced in place
  void *o;                               // [T][hv][dv] out (bf16)
  int32_t T, off, n_chunks, hk, hv;
};

struct PfCopy {
  const void *k, *v;                     // [T][hkv][D] span rows
  void *kc, *vc;                         // [hkv][cap][D] caches of this layer
  int64_t cap, L;
  int32_t T, hkv;
};

struct PfAttn {
  const void *q;                         // [T][hq][D] span queries (bf16)
  const void *kc, *vc;                   // [hkv][cap][D], span rows already at [L, L + T)
  void *o;                               // [T][hq][D] out (bf16), written here when nsplit = 1
  float *part_acc;                       // [hkv][nsplit][rows_cap][D] unnormalised sums (nsplit > 1)
  float *part_ml;                        // [hkv][nsplit][rows_cap][2] running max (base 2), sum
  int64_t cap, L;
  int32_t T, hq, hkv;
  int32_t row_tiles, rows_cap;           // rows_cap = kPfRows row_tiles
  int32_t nsplit, split;                 // key splits of `split` keys (a multiple of kKvTile)
  int32_t items;                         // hkv nsplit row_tiles, padded to a multiple of 8
  float c2;                              // softmax scale times log2(e)
};

// ---------------------------------------------------------------- host entry points
// Each returns the result of hipGetLastError() after enqueueing.  With ev0 / ev1
// set, the dispatch itself records its start and end time into them (the
// launch goes through hipExtLaunchKernel), so an event pair times the kernel
// alone, not the queueing around it.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
hipError_t launch_gdn_tree(const GdnLaunch &a, int dk, int bf16, hipStream_t s, KernelEvents ev);
hipError_t launch_attn_split(const AttnLaunch &a, int D, int bf16, int n_blocks, hipStream_t s,
                             KernelEvents ev);
hipError_t launch_attn_fold(const FoldLaunch &a, int D, int bf16, int n_blocks, hipStream_t s,
                            KernelEvents ev);
hipError_t launch_kv_split(const KvLaunch &a, int D, int max_items, hipStream_t s,
                           KernelEvents ev);
// Tree pass; `tiles` (1..3) is the most kKvTile-key tiles from tb0 to a node's position
// over the launch's nodes.
hipError_t launch_kv_tree(const KvLaunch &a, int D, int max_items, int tiles, hipStream_t s,
                          KernelEvents ev);
hipError_t launch_commit(const CommitLaunch &a, int dk, int bf16, int n_blocks, hipStream_t s,
                         KernelEvents ev);
hipError_t launch_gdn_conv(const ConvLaunch &a, int bf16, hipStream_t s, KernelEvents ev);
// pf_conv_kernel over the span, then (width > 1) pf_conv_tail_kernel rolls the tail.
hipError_t launch_pf_conv(const PfConv &a, int bf16, hipStream_t s, KernelEvents ev);
hipError_t launch_walk(const WalkLaunch &a, hipStream_t s, KernelEvents ev);
hipError_t launch_snapshot_header(const SnapshotHeader &h, void *dst, hipStream_t s);
hipError_t launch_wy_prep(const WyPrep &a, int dk, hipStream_t s, KernelEvents ev);
hipError_t launch_wy_scan(const WyScan &a, int dk, hipStream_t s, KernelEvents ev);
hipError_t launch_pf_copy(const PfCopy &a, int D, hipStream_t s);
hipError_t launch_pf_attn(const PfAttn &a, int D, hipStream_t s, KernelEvents ev);
hipError_t launch_pf_fold(const PfAttn &a, int D, hipStream_t s, KernelEvents ev);

// The library's static scratch array (hdt_forward_tree_noalloc): kStaticScratchBytes per
// device, held until the process ends.  static_scratch_address resolves its device
// address on the current device (once per device) and returns it.
constexpr size_t kStaticScratchBytes = size_t(48) << 20;
hipError_t static_scratch_address(void **out);
// Channels one conv thread handles (16 bytes of io dtype).
constexpr int conv_channels_per_thread(int bf16) { return bf16 ? 8 : 4; }

// Dynamic LDS bytes each kernel asks for (the host checks them against the device).
size_t gdn_lds_bytes(int dk, int n_max, int n_saves, int anc);
size_t attn_lds_bytes(int D, int bf16, int n_max);
// Work decomposition of the float32 attention split pass: rows per shared item
// and nodes per tail item.
int attn_rows_per_item(int bf16);
int attn_nodes_per_tail(int bf16);
size_t commit_lds_bytes(int D, int bf16, int m);

}  // namespace hdt
