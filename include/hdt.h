/*
 * hdt.h - C ABI of the tree-verify library (libhdt.so) for AMD MI355X (gfx950).
 *
 * The library verifies a merged draft tree through a stack of Gated DeltaNet
 * (GDN) and attention layers in one pass, then keeps or drops the result.  It
 * is called once per step, never once per operator, and activations stay on
 * the device: the step-granular flat C ABI described in "How ignis serves a
 * request" ("The shape of the process").  The verbs follow the hot verbs of
 * "Adding a model" (step 4 of "The adapter path in ten steps"): forward_tree,
 * forward_block, commit_tree, rollback_to, kv.length and reset.
 *
 * Conventions for every call:
 *  - Device pointers are HIP device memory owned by the caller; the library
 *    never frees them.  Host pointers are read during the call only.
 *  - A stream argument is a hipStream_t passed as void* (NULL = the default
 *    stream).  Work is enqueued asynchronously on it; nothing waits for the GPU.
 *  - Every argument and ordering check runs on the host before anything is
 *    enqueued.  A call that returns an error changed nothing: no slot state,
 *    length or pending round moved, and no kernel was launched.
 *  - hdt_last_error() returns a text for the last failed call on that engine.
 *  - An engine is not thread-safe: use one per thread or serialise calls.
 *  - No C++ exception crosses this interface.
 *
 * Tree convention (the pages give the tree as "one tree" per round, section
 * 2.6 "The decode loop" of "One request, end to end"; the array form is ours):
 *  parent[0] = -1 (node 0 is the root: the model's own token from the last
 *  round, not yet in the cache) and 0 <= parent[i] < i.  Node i sits at
 *  position L + depth(i), L being the slot's committed length, and sees every
 *  committed row plus its ancestors-or-self.  At most HDT_MAX_NODES nodes.
 */
#ifndef HDT_H
#define HDT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HDT_MAX_NODES 64 /* nodes per tree (ancestor masks are 64-bit)   */
#define HDT_MAX_TREES 8  /* trees (slots) in one joint forward_tree call */

typedef enum {
  HDT_OK = 0,
  HDT_E_INVALID = -1,     /* bad argument, descriptor or shape            */
  HDT_E_TREE = -2,        /* parent array is not a valid tree             */
  HDT_E_PATH = -3,        /* commit path is not a root path of the tree   */
  HDT_E_CAPACITY = -4,    /* the slot's buffers cannot hold the rows      */
  HDT_E_ORDER = -5,       /* verb out of sequence (pending round rules)   */
  HDT_E_HIP = -6,         /* a HIP runtime call failed                    */
  HDT_E_UNSUPPORTED = -7  /* valid request the library does not implement */
} hdt_status;

typedef enum { HDT_F32 = 0, HDT_BF16 = 1 } hdt_dtype;

/*
 * Model descriptor, fixed at hdt_create.
 *  layer_kind: host array of n_layers entries, 0 = GDN, 1 = attention ("Adding
 *    a model", "What is still specific to Qwen3.8": a hybrid of Gated DeltaNet
 *    and attention layers).  Layers run in index order.
 *  GDN: gdn_hk query/key heads, gdn_hv value heads (gdn_hv % gdn_hk == 0; v head
 *    h reads q/k head h / (gdn_hv / gdn_hk)); gdn_dk = gdn_dv in {64, 128}
 *    (state heads of 128 by 128 in the pages); gdn_dv % 16 == 0.
 *  Attention: attn_hq query heads, attn_hkv kv heads (q head j reads kv head
 *    j / (attn_hq / attn_hkv), at most 16 q heads per kv head, and with bf16
 *    storage at most 6 at attn_d = 256), head dim attn_d in {64, 256}.
 *  io_dtype: storage of q, k, v, gates, outputs and the K/V cache (HDT_BF16,
 *    or HDT_F32 with attn_d = 64).  The GDN state is always float32.
 *  gdn_scale: readout scale s in o = S^T (s q); <= 0 selects 1/sqrt(gdn_dk).
 *  attn_scale: softmax scale; <= 0 selects 1/sqrt(attn_d).
 *  max_nodes: largest tree any call will pass (1..HDT_MAX_NODES); sizes the
 *    library's own scratch.
 *  gdn_conv: width w of the short causal convolution in front of every GDN
 *    layer (the gdn.conv state section of "Adding a model", "The model layer:
 *    architecture registry and per-model state"), 1..4; 0 = none, and then a
 *    GDN layer's q, k, v are taken as already convolved.  With w > 0 a GDN
 *    layer's q, k, v inputs are the pre-conv channels; per channel the layer
 *    computes y = SiLU(sum_j W[c][j] x_{w-1-j}), x_r being the input r tokens
 *    back along the node's root path (the slot's conv tail before the root),
 *    then divides every q and k head by sqrt(sum of squares + 1e-6).  The
 *    post-conv values are rounded to io_dtype before the recurrence.
 *  gdn_conv_weight: device float32 [n_gdn][C][w] taps (tap w-1 multiplies the
 *    current token), C = 2 gdn_hk gdn_dk + gdn_hv gdn_dv channels ordered q, k,
 *    v, each head-major; 16-byte aligned.  Unused when gdn_conv = 0.
 */
typedef struct {
  int32_t n_layers;
  const uint8_t *layer_kind;
  int32_t gdn_hk, gdn_hv, gdn_dk, gdn_dv;
  int32_t attn_hq, attn_hkv, attn_d;
  int32_t io_dtype;
  float gdn_scale, attn_scale;
  int32_t max_nodes;
  int32_t gdn_conv;
  const float *gdn_conv_weight;
} hdt_model_desc;

/*
 * One slot: a sequence with its own recurrent state and K/V views ("Adding a
 * model", "The model layer: architecture registry and per-model state": state
 * sections copied whole, K and V views indexed by token position; "Parallel
 * requests": each slot has its own KV and recurrent state).  All device memory,
 * owned by the caller:
 *  gdn_state: float32 [n_gdn][gdn_hv][gdn_dv][gdn_dk]; element S[a][c] of a head
 *    (a over the key dim, c over the value dim) is at [c][a] (value-major).
 *  k_cache, v_cache: io_dtype [n_attn][attn_hkv][capacity][attn_d], row t =
 *    token position t.
 *  n_gdn / n_attn count the layers of each kind, in layer order.
 *  capacity: rows per head in the caches; a tree of n nodes needs
 *    length + n <= capacity.
 *  length: committed rows at creation.
 *  gdn_conv_state: io_dtype [n_gdn][w-1][C] (w = gdn_conv > 1): the pre-conv
 *    inputs of the last w-1 committed tokens, row w-2 the newest; commit_tree
 *    rolls the accepted path's rows in (bit copies).  16-byte aligned; unused
 *    (may be NULL) when gdn_conv <= 1.
 */
typedef struct {
  float *gdn_state;
  void *k_cache;
  void *v_cache;
  int64_t capacity;
  int64_t length;
  void *gdn_conv_state;
} hdt_slot_desc;

/*
 * Per-layer inputs and output of one tree, all device pointers in io_dtype,
 * n = the tree's node count:
 *  GDN layer:       q, k [n][gdn_hk][gdn_dk]; v [n][gdn_hv][gdn_dv] (pre-conv
 *                   and 16-byte aligned when gdn_conv > 0);
 *                   alpha, beta [n][gdn_hv] (decay and write strength, values in
 *                   (0,1)); o [n][gdn_hv][gdn_dv] out.
 *  attention layer: q [n][attn_hq][attn_d]; k, v [n][attn_hkv][attn_d] (the
 *                   tree's own rows, already rotated); alpha, beta unused;
 *                   o [n][attn_hq][attn_d] out.
 * Inputs are read during the pass only; the library copies what commit needs.
 */
typedef struct {
  const void *q, *k, *v, *alpha, *beta;
  void *o;
} hdt_layer_io;

/* One tree of a forward_tree call.  parent and io are HOST arrays (io has
 * n_layers entries). */
typedef struct {
  int32_t slot;
  int32_t n_nodes;
  const int32_t *parent;
  const hdt_layer_io *io;
} hdt_tree;

typedef struct hdt_engine hdt_engine;

/*
 * Create an engine over n_slots caller-owned slots: the one call per model load of
 * the flat C ABI in "How ignis serves a request" ("The shape of the process"), with
 * the model described by its layer kinds and head shapes ("Adding a model", "The
 * model layer: architecture registry and per-model state").  Validates every field;
 * allocates nothing on the device (scratch is allocated on the current HIP device at
 * the first call that launches work).  *out is NULL on failure.
 * Errors: HDT_E_INVALID (a field out of range), HDT_E_UNSUPPORTED (a shape the kernels
 * do not implement).
 */
hdt_status hdt_create(const hdt_model_desc *desc, int32_t n_slots, const hdt_slot_desc *slots,
                      hdt_engine **out);

/* Free the engine and its scratch (not the caller's buffers): the model-unload end of
 * the lifecycle in "How ignis serves a request" ("The shape of the process").  Waits
 * for the device first.  NULL is a no-op. */
void hdt_destroy(hdt_engine *eng);

/*
 * forward_tree ("Adding a model", step 4; "One request, end to end", 2.6): verify
 * n_trees trees (distinct slots, none with a pending round) in one pass through
 * every layer.  Per GDN layer, each value head advances its recurrent state
 * along every root-to-node path and writes S_i^T (s q_i) for every node; per
 * attention layer, every (node, q head) row attends to the committed rows and
 * its ancestors-or-self.  Writes each layer's o; stages each attention layer's
 * tree rows into the slot's cache rows [L, L+n) in tree-index order; keeps what
 * commit needs.  Committed state and rows below L are left unchanged.
 * Afterwards each slot has a pending round.  Several trees in one call give
 * every row the same bits as verifying each tree alone ("Parallel requests",
 * "On Flash-Next": the joint pass equals each lone verify bit for bit).
 * The call enqueues kernels only (no allocation, copy or fill once the engine's
 * scratch exists), so it may be captured into a HIP graph and replayed; a replay
 * repeats this round's pass at the same lengths.  The first launching call
 * allocates the scratch and must not be captured (HDT_E_ORDER).
 * Errors: HDT_E_INVALID, HDT_E_TREE, HDT_E_CAPACITY, HDT_E_ORDER, HDT_E_HIP.
 */
hdt_status hdt_forward_tree(hdt_engine *eng, int32_t n_trees, const hdt_tree *trees,
                            void *stream);

/*
 * A reusable graph of the verify pass, kept across rounds for a given set of tree sizes and
 * slots ("How ignis serves a request", 4 "Decode generates, one round for every lane": a
 * round replays a graph captured for its exact batch width; "Parallel requests", "What a
 * slot costs": a slot keeps its verify graphs).  hdt_graph_forward is hdt_forward_tree with
 * the round's kernels enqueued as one HIP graph launch on `stream`: the pass is captured on
 * the graph's own stream, and the instantiated graph is updated in place (kernel arguments
 * and grids) when the kernel sequence is the one it holds, else instantiated again.  The
 * results are hdt_forward_tree's bits, and so is the round's bookkeeping (a pending round
 * per slot, closed by commit or rollback).  Two instantiated graphs are used in turn and
 * each is updated only after its previous launch has finished (the host waits for that if
 * needed), so the host may prepare a round while the one before runs.  The first call on an
 * engine that has not yet run a forward allocates the engine's scratch first.
 * hdt_graph_stats counts instantiations and in-place updates.  A graph belongs to its
 * engine and must be destroyed before it; neither is thread-safe.
 * Errors: those of hdt_forward_tree.
 */
typedef struct hdt_graph hdt_graph;
hdt_status hdt_graph_create(hdt_engine *eng, hdt_graph **out);
hdt_status hdt_graph_forward(hdt_graph *g, int32_t n_trees, const hdt_tree *trees, void *stream);
hdt_status hdt_graph_stats(const hdt_graph *g, int64_t *instantiations, int64_t *updates);
void hdt_graph_destroy(hdt_graph *g);

/*
 * forward_tree that allocates nothing, for callers that cannot allocate: code under HIP
 * graph capture from the first call on, serving loops and harnesses that forbid
 * allocation.  The same pass and the same bits as hdt_forward_tree, but the round's scratch
 * (what commit needs of the pass, the attention partials, the conv staging) is carved from
 * a static array of the library, 48 MiB per device (HDT_STATIC_SCRATCH_BYTES), held until
 * the process ends; it makes no hipMalloc, hipHostMalloc, hipFree or event call.  A call
 * whose trees need more scratch than that (one slot of a 64-layer model at the 27B-like
 * shapes with max_nodes up to 32 fits) returns HDT_E_CAPACITY and changes nothing.
 * Every call on a device shares that device's array and it keeps the last call's
 * contents (nothing in it needs to start at zero).  A pending round made by this call
 * is closed by hdt_commit_tree, hdt_rollback_to or hdt_walk_commit as usual, but only
 * before the next hdt_forward_tree_noalloc call on the same device: after it those refuse
 * the round with HDT_E_ORDER (its scratch was reused) and hdt_rollback_to(length) drops it.
 * Calls that overlap in time on one device (other engines, other streams or threads)
 * race on the array.
 * Errors: those of hdt_forward_tree, and HDT_E_CAPACITY as above.
 */
#define HDT_STATIC_SCRATCH_BYTES (48ll << 20)
hdt_status hdt_forward_tree_noalloc(hdt_engine *eng, int32_t n_trees, const hdt_tree *trees,
                                    void *stream);

/* forward_block ("Adding a model", step 4 of "The adapter path in ten steps": the hot
 * verb that verifies a block of drafted tokens): forward_tree of one chain of n nodes
 * (parent[i] = i - 1), 1 <= n <= HDT_MAX_NODES.  Same errors as forward_tree. */
hdt_status hdt_forward_block(hdt_engine *eng, int32_t slot, int32_t n, const hdt_layer_io *io,
                             void *stream);

/*
 * forward_span: a prefill of T tokens ("One request, end to end", 2.5: the prompt
 * tokens past the resident prefix go through the model once), committed as it goes.
 * io has n_layers entries whose arrays hold T rows (the hdt_layer_io layouts with
 * n = T).  The span runs as consecutive chains of up to max_nodes tokens through the
 * tree kernels, each chain committed before the next, so every row and the final
 * state equal a token-by-token decode bit for bit.  With anchors set
 * (hdt_set_anchors), a chain also ends at every multiple of `every`, and the
 * recurrent state (and conv tails) at that position is copied to its anchor.
 * Needs no pending round; length + T <= capacity.  length += T.
 * Errors: HDT_E_INVALID, HDT_E_ORDER, HDT_E_CAPACITY, HDT_E_HIP.
 */
hdt_status hdt_forward_span(hdt_engine *eng, int32_t slot, int32_t T, const hdt_layer_io *io,
                            void *stream);

/*
 * forward_chunked: the same prefill as hdt_forward_span (T tokens after the slot's
 * committed ones, io of n_layers entries with T rows each, committed as it goes,
 * anchors filled), computed a chunk at a time on the matrix cores ("One request, end
 * to end", 2.5 "The caches decide where the prefill starts": the prompt past the
 * resident prefix goes through the model once, with state anchors; "How ignis serves
 * a request", 3 "Prefill reads the prompt", in chunks).
 *  GDN layers: with gdn_conv > 0, the short causal conv over the span's q, k, v rows
 *    after the layer's committed tail first (then the tail holds the span's last
 *    gdn_conv - 1 pre-conv rows); then the chunked (WY) form of the same recurrence
 *    over chunks of 64 tokens anchored at absolute positions (a multiple of 64); the
 *    state between chunks and the final state are float32.
 *  Attention layers: the span's k/v rows are written into the cache at [L, L + T),
 *    then each row (token t, q head j) attends causally to cache rows 0 .. L + t.
 * The span is cut into pieces of at most 2048 tokens (and at anchor positions) that
 * each pass through every layer in order.  Outputs, rows and state equal the
 * token-by-token recurrence up to rounding (outputs within the io precision), not bit
 * for bit: hdt_forward_span is the bit-exact chain mode.  Needs bf16 storage, GDN
 * heads of 128 by 128 and attn_d = 256 (else HDT_E_UNSUPPORTED);
 * alpha in (0, 1].  Buffers 16-byte aligned.  The first call allocates the
 * library's prefill scratch (not under graph capture).  Needs no pending round;
 * length + T <= capacity.  length += T.
 * Errors: HDT_E_INVALID, HDT_E_ORDER, HDT_E_CAPACITY, HDT_E_UNSUPPORTED, HDT_E_HIP.
 */
hdt_status hdt_forward_chunked(hdt_engine *eng, int32_t slot, int32_t T, const hdt_layer_io *io,
                               void *stream);

/*
 * State anchors of a slot ("One request, end to end", 2.5: recurrent-state anchors
 * every 1,024 tokens let a later turn resume inside the resident prefix).  Device
 * buffers owned by the caller: state float32 [n_max][n_gdn][gdn_hv][gdn_dv][gdn_dk]
 * (anchor k holds the state at position (k + 1) * every) and, when gdn_conv > 1,
 * conv in io_dtype [n_max][n_gdn][gdn_conv - 1][C] (else NULL).  every >= 1.
 * forward_span fills them; commit_tree and the accept walk do not.  A call replaces
 * the previous anchors of the slot (all marked empty); every = 0 removes them.
 * Errors: HDT_E_INVALID.
 */
hdt_status hdt_set_anchors(hdt_engine *eng, int32_t slot, int64_t every, int32_t n_max,
                           float *state, void *conv);

/* The highest position p <= n whose anchor holds a state, or -1 (none): where a later
 * turn can resume ("One request, end to end", 2.5: a prefix is reused up to its last
 * recurrent-state anchor).  Host only.  Errors: HDT_E_INVALID. */
hdt_status hdt_anchor_below(const hdt_engine *eng, int32_t slot, int64_t n, int64_t *out);

/*
 * commit_tree ("One request, end to end", 2.6: commit the accepted path's KV
 * rows and recurrent state): path is a HOST array of m >= 1 node indices with
 * path[0] = 0 and parent[path[d]] = path[d-1].  For every attention layer,
 * cache row L+d takes the pending row of path[d] (a bit copy); for every GDN
 * layer the committed state becomes the state of node path[m-1], with the same
 * bits the pass computed, and (gdn_conv > 1) the conv tail becomes the last w-1
 * rows of (old tail, path's pre-conv rows).  Then length += m and the pending
 * round ends.
 * Errors: HDT_E_INVALID, HDT_E_PATH, HDT_E_ORDER (no pending round), HDT_E_HIP.
 */
hdt_status hdt_commit_tree(hdt_engine *eng, int32_t slot, const int32_t *path, int32_t m,
                           void *stream);

/*
 * rollback_to(n) ("Adding a model", step 4 of "The adapter path in ten steps", a hot
 * verb; "The tests a new model must pass": a block verify followed by a rollback):
 * keep exactly n tokens.  n = length drops the pending round
 * (or does nothing when none is pending).  length < n <= length + c, c being
 * the pending tree's leading chain (nodes 0..c-1 with parent[i] = i-1), keeps
 * that chain prefix: the same as hdt_commit_tree with path 0..n-length-1.
 * n < length: when n is the position of a filled anchor (hdt_set_anchors,
 * hdt_anchor_below), the state and conv tails are copied back from it, the pending
 * round is dropped, length = n, and the anchors above n are emptied (the rows past
 * n will be written again); otherwise HDT_E_UNSUPPORTED.  Other n: HDT_E_INVALID.
 */
hdt_status hdt_rollback_to(hdt_engine *eng, int32_t slot, int64_t n, void *stream);

/*
 * Accept walk + commit on the device, with no host wait ("One request, end to end",
 * 2.6: the verified tree is walked with the model's own tokens, the longest agreeing
 * path plus one token of the model's own is kept, and that path is committed).
 *  draft: device int32 [n] token of each node of the slot's pending tree (draft[0],
 *    the root, is the model's own token from the last round and is not compared);
 *  target: device int32 [n], the model's own next token after each node (the argmax
 *    of its logits, computed by the caller);
 *  out: device int32 [2 + n] written by the walk: out[0] = m, out[1] = the bonus
 *    token, out[2 .. 2+m) = the accepted path.
 * Node i > 0 agrees when its parent agrees and draft[i] == target[parent[i]]; the
 * root agrees.  The path ends at the deepest agreeing node (the lowest index among
 * equals) and the bonus token is target[that node].  The path is then committed as
 * hdt_commit_tree would, reading it from `out` on the device.  The slot's new
 * length (length + m) is known to the host once the device has finished the walk:
 * every later call on the slot (hdt_kv_length included) first waits for that.
 * Buffers 4-byte aligned.  Not for graph capture.
 * Errors: HDT_E_INVALID, HDT_E_ORDER (no pending round), HDT_E_HIP.
 */
hdt_status hdt_walk_commit(hdt_engine *eng, int32_t slot, const int32_t *draft, const int32_t *target,
                           int32_t *out, void *stream);

/* kv.length ("Adding a model", step 4 of "The adapter path in ten steps"): committed
 * rows of a slot (host value; after hdt_walk_commit it waits for the device to finish
 * that walk).  Errors: HDT_E_INVALID, HDT_E_HIP. */
hdt_status hdt_kv_length(const hdt_engine *eng, int32_t slot, int64_t *out);

/* reset ("Adding a model", step 4 of "The adapter path in ten steps"): set a slot's
 * committed length (0..capacity) and drop any pending round; anchors above the new
 * length are emptied.  The caller owns the state and cache contents.
 * Errors: HDT_E_INVALID, HDT_E_HIP. */
hdt_status hdt_reset(hdt_engine *eng, int32_t slot, int64_t length);

/*
 * Tree metadata of one merged draft tree ("One request, end to end", 2.6: the drafts
 * are merged into one tree verified in one pass) on the host, as the kernels use it:
 * depth[n]; mask[n] with bit
 * j set when node j is an ancestor-or-self of node i; anc[n][HDT_MAX_NODES]
 * with anc[i][d] the ancestor of i at depth d (-1 beyond depth(i));
 * pos[n] = L + depth.  Any output may be NULL.  No engine, no device.
 * Errors: HDT_E_TREE.
 */
hdt_status hdt_tree_meta(int32_t n, const int32_t *parent, int64_t L, int32_t *depth,
                         uint64_t *mask, int32_t *anc, int64_t *pos);

/*
 * Attention split size of the row at `position` (0 <= position < capacity) of a
 * slot: the keys 0..position are cut into splits of this many positions anchored
 * at position 0, each reduced on its own and folded in ascending order.  With
 * bf16 storage it depends only on the position and the engine's shape (attn_hkv
 * and max_nodes: a tree of more than 96 query rows per kv head takes several row
 * groups per split): the smallest rung of 128, then s + max(32, s/32) rounded up
 * to 32, ... that cuts position + 1 keys into at most 256 / (attn_hkv row_groups)
 * splits.  With float32 storage it depends only on the slot's capacity.  Either
 * way a row's bits depend only on its inputs, never on how many of its keys were
 * committed.  Errors: HDT_E_INVALID.
 */
hdt_status hdt_split_size(const hdt_engine *eng, int32_t slot, int64_t position, int64_t *out);
/* (The split rule is how the kernels keep the rule of "Adding a model", step 4 of "The
 * adapter path in ten steps", that a verified row equals the decode step's row: a row's
 * reduction order follows from its own position.)  Host only. */

/*
 * Kernel timing for measurement (the per-device verify cost that StairCut prices its
 * cuts with, "One request, end to end", 2.6, is built from such timings).
 * hdt_profile(eng, 1) starts recording a HIP
 * event pair around every launch on the launch stream; hdt_profile_read waits
 * for the recorded events and returns, for kernel class `kind` (0 = GDN tree
 * walk, 1 = attention split pass, 2 = attention fold, 3 = commit, 4 = GDN conv,
 * 5 = accept walk, 6 = chunked-prefill GDN prep, 7 = its GDN scan, 8 = its attention,
 * 9 = its attention merge), the summed
 * milliseconds and the launch count since the last read; then clears them.
 */
hdt_status hdt_profile(hdt_engine *eng, int32_t enable);
hdt_status hdt_profile_read(hdt_engine *eng, int32_t kind, double *ms, int64_t *launches);

/*
 * State snapshot ("Adding a model", "The model layer: architecture registry and
 * per-model state": a model's cache state has sections copied whole and views sliced
 * by length, with nbytes, clone, restore and a signature that refuses a restore across
 * shapes).  The sections here are the recurrent state (gdn.S) and the conv tails
 * (gdn.conv); the views are the slot's K/V cache rows, which stay where they are.
 *
 * hdt_state_bytes: the size of a snapshot of this engine's shape (nbytes).
 *
 * hdt_state_copy(restore = 0) (clone): writes into `buf` (device memory owned by the
 * caller, 256-byte aligned, buf_bytes >= hdt_state_bytes) a 256-byte header holding the
 * engine's shape signature and the slot's committed length, then the state and conv
 * sections, enqueued on `stream`.  A pending round is left as it is (its rows are not
 * committed and are not part of the snapshot).
 *
 * hdt_state_copy(restore = 1): waits for `stream`, reads the header, and refuses
 * (HDT_E_INVALID, nothing changed) a buffer that holds no snapshot, a snapshot of an
 * engine of another shape, or one taken at more committed rows than the slot now holds
 * (the cache must still hold the rows below the snapshot's length).  Otherwise it copies
 * the sections back on `stream`, sets the slot's length to the snapshot's, drops any
 * pending round and empties the anchors above that length.  Not for graph capture.
 * Errors: HDT_E_INVALID, HDT_E_HIP.
 */
hdt_status hdt_state_bytes(const hdt_engine *eng, int64_t *out);
hdt_status hdt_state_copy(hdt_engine *eng, int32_t slot, void *buf, int64_t buf_bytes, int32_t restore,
                          void *stream);

/* Text of the last error on this engine ("" when none); never NULL.  The flat C ABI of
 * "How ignis serves a request" ("The shape of the process") lets no exception cross;
 * each call returns a status and this names the failed check.  Owned by the engine,
 * valid until its next call. */
const char *hdt_last_error(const hdt_engine *eng);

#ifdef __cplusplus
}
#endif

#endif /* HDT_H */
