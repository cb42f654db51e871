// launch.h - argument blocks passed by value from the host engine to the kernels.
//
// Every launch covers one layer (or, for commit, every layer) of up to
// kMaxTrees trees; a workgroup finds its tree from its block index and the
// per-tree *_begin offsets.  All sizes were validated on the host before a
// block is filled in, so the kernels index without further checks beyond
// what the tree itself bounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hdt {

constexpr int kMaxNodes = 64;
constexpr int kMaxTrees = 8;
constexpr int kTile = 64;          // attention keys per tile, anchored at absolute positions
constexpr int kAttnWaves = 8;      // waves per attention workgroup (float32 storage)
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kAttn2Waves = 4;     // bf16 storage: waves per workgroup, one per SIMD
constexpr int kAttn2Threads = kAttn2Waves * 64;
constexpr int kAttn2Blocks = 2;    // bf16 storage: 16-row blocks per wave
constexpr int kGdnThreads = 256;   // 4 waves x 4 value columns x 16 lanes per column
constexpr int kGdnCols = 16;       // value columns per GDN workgroup
constexpr int kFoldThreads = 256;  // 4 waves per output row

// ---------------------------------------------------------------- GDN tree walk
struct GdnTree {
  const void *q, *k, *v, *alpha, *beta;  // tree inputs of this layer (io dtype)
  void *o;                               // [n][hv][dv] out
  const float *state;                    // committed state of this layer [hv][dv][dk]
  float *u_pend;                         // [max_nodes][hv][dv]: delta-rule corrections u_i
  void *k_pend;                          // [max_nodes][hk][dk]: copy of k (io dtype)
  void *a_pend;                          // [max_nodes][hv]:     copy of alpha (io dtype)
  int32_t n;
  int32_t wg_begin;                      // first workgroup of this tree
  int8_t parent[kMaxNodes];
  int8_t depth[kMaxNodes];
};

struct GdnLaunch {
  GdnTree t[kMaxTrees];
  int32_t n_trees;
  int32_t hk, hv, dv;
  int32_t n_max;                         // largest n over the trees (sizes LDS)
  float scale;
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
  int32_t m;
  int8_t path[kMaxNodes];
};

// ---------------------------------------------------------------- host entry points
// Each returns the result of hipGetLastError() after enqueueing.
hipError_t launch_gdn_tree(const GdnLaunch &a, int dk, int bf16, hipStream_t s);
hipError_t launch_attn_split(const AttnLaunch &a, int D, int bf16, int n_blocks, hipStream_t s);
hipError_t launch_attn_fold(const FoldLaunch &a, int D, int bf16, int n_blocks, hipStream_t s);
hipError_t launch_commit(const CommitLaunch &a, int dk, int bf16, int n_blocks, hipStream_t s);

// Dynamic LDS bytes each kernel asks for (the host checks them against the device).
size_t gdn_lds_bytes(int dk, int n_max);
size_t attn_lds_bytes(int D, int bf16, int n_max);
// Work decomposition of the attention split pass for a storage dtype: rows per
// shared item and nodes per tail item.
int attn_rows_per_item(int bf16);
int attn_nodes_per_tail(int bf16);
size_t commit_lds_bytes(int D, int bf16, int m);

}  // namespace hdt
