// kv_attention.hip - one attention layer of the tree verify with bf16 storage, on
// the CDNA4 (gfx950) matrix cores.
//
// Each (node, q head) row attends to every committed row of its kv head and to
// the tree rows of its ancestors-or-self, node i sitting at position L + depth(i)
// ("One request, end to end", section 2.6: one forward pass verifies the merged
// tree; "Adding a model", "The model layer: architecture registry and per-model
// state": K and V are views indexed by token position).
//
// Two kernels per layer:
//  kv_split_kernel  streams the committed rows.  One workgroup takes one split of
//                   one kv head for every row of that head (up to kKvWaves * NB * 16
//                   rows), with kKvTile-key tiles of K and V going straight from HBM
//                   into a kKvStages-deep LDS ring (buffer_load ... lds), scores
//                   S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16, and
//                   an online softmax in base 2.  A split wholly below L leaves one
//                   normalised bf16 partial per row; the tiles of split L / split
//                   below tb0 = kKvTile * (L / kKvTile) leave their float32 state.
//  kv_tree_kernel   one workgroup per (kv head, node, quarter of the output columns):
//                   wave 0 continues that state through the tiles from tb0 to the
//                   node's position (rows at or past L are the node's ancestors,
//                   gathered into LDS by global_load_lds); waves 1-3 fold the
//                   row's split partials in ascending order meanwhile; then the two
//                   are combined and the output written.
//
// A row's result is a function of its query and of the key/value sequence by
// absolute position only (the verified row equals the decode step's row, "Adding
// a model", step 4 of "The adapter path in ten steps"):
//  - tiles and splits are anchored at absolute positions, and a row's split size is
//    a function of its own position; a tile is processed by the same instruction
//    sequence in both kernels, and an MFMA output column depends on its own row
//    only;
//  - masked slots hold a finite row (the node's own) and get probability 0;
//  - the running max moves only when a tile exceeds it by more than kLazyMax, a
//    rule that depends on the row's scores alone;
//  - every split but a row's last enters the fold as its normalised bf16 partial,
//    whichever kernel finished it.  The committed splits fold in chunks of
//    kFoldChunk (the chunk's max, then weighted sums in ascending split order; the
//    chunks merge in order), then the split finished in the tree pass if the node's
//    rows cross into the next split, then the last split's float32 state.
#include "common.h"

#pragma clang fp contract(off)

namespace hdt {
namespace {

// Probabilities stay below 2^kLazyMax: the running max moves only when a tile's max
// exceeds it by more than this (base-2 units).
constexpr float kLazyMax = 8.0f;

template <int D>
struct KvCfg {
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int HALF = kKvTile * ROWB;        // K (or V) part of a tile
  static constexpr int TILE = 2 * HALF;              // K then V
  static constexpr int LOADS = TILE / 1024;          // wave-wide 16-byte-per-lane loads per tile
  static constexpr int RPL = 1024 / ROWB;            // rows per wave-wide load
  static constexpr int KQ = D / 32;                  // k-steps of the score MFMA
  static constexpr int DB = D / 16;                  // 16-column blocks of a row
  static constexpr int QD = D / kKvQuarters;         // output columns per tree-pass block
  static constexpr int QDB = QD / 16;
  static_assert(LOADS % 8 == 0 && QD % 16 == 0 && 1024 % ROWB == 0, "tile shape");
};

// XOR swizzle of the 16-byte chunks of tile row `row`: keeps the score operand
// reads (16 keys at one chunk) and the transposed value reads (4 keys at two
// chunks) free of LDS bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 256) {
    return (2 * row) & 31;
  } else {
    return (row >> 1) & (KvCfg<D>::CPR - 1);
  }
}

template <int D>
__device__ __forceinline__ int chunk_off(int row, int c) {
  return row * KvCfg<D>::ROWB + ((c ^ swz<D>(row)) << 4);
}

// Online-softmax state of up to NB 16-row blocks of one wave.  Lane (g, n) holds
// row n of each block; acc[b][j][i] is output column 16 (db0 + j) + 4 g + i.
template <int D, int NB, int NDB>
struct KvRows {
  floatx4 acc[NB][NDB];
  float m[NB], l[NB];
  bf16x8 q[NB][D / 32];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < NDB; ++j) acc[b][j] = floatx4{0.f, 0.f, 0.f, 0.f};
      m[b] = -INFINITY;
      l[b] = 0.0f;
    }
  }
};

// Tile-invariant LDS byte offsets of this lane's operand reads within a tile: the
// score operand of key block 0 at k-step kk, and the low transposed value read of
// column block db0 + j.  Key block 1 and the high value read sit 16 rows further
// (the swizzle repeats every 16 rows), an immediate offset.
template <int D, int NDB>
struct KvLane {
  uint32_t ko[KvCfg<D>::KQ];
  uint32_t vo[NDB];
  __device__ __forceinline__ void init(int db0) {
    using C = KvCfg<D>;
    const int lane = threadIdx.x & 63, g = lane >> 4, ln = lane & 15;
#pragma unroll
    for (int kk = 0; kk < C::KQ; ++kk) ko[kk] = static_cast<uint32_t>(chunk_off<D>(ln, 4 * kk + g));
    const int r0 = 4 * g + (ln >> 2);
    const int half8 = 8 * (ln & 1);
#pragma unroll
    for (int j = 0; j < NDB; ++j) {
      const int c = 2 * (db0 + j) + ((ln & 3) >> 1);
      vo[j] = static_cast<uint32_t>(C::HALF + chunk_off<D>(r0, c) + half8);
    }
  }
};

// One tile (kKvTile keys from absolute position tb; K then V in `tile`, swizzled)
// for the NB row blocks of this wave, output columns [16 db0, 16 (db0 + NDB)) with
// the offsets of `ofs` (made for db0).
// MASK: keys past `pos` get probability 0.  Every block is computed (a block with
// no rows of its own holds copies of real queries and is discarded by the caller),
// so the instruction stream has no branches; all LDS reads of an operand are
// issued before the MFMAs that use them, and the value reads before the softmax.
template <int D, int NB, int NDB, bool MASK>
__device__ __forceinline__ void kv_tile(KvRows<D, NB, NDB> &st, uint32_t tile, const KvLane<D, NDB> &ofs,
                                        int64_t tb, int64_t pos, float c2) {
  using C = KvCfg<D>;
  constexpr int KB1 = 16 * C::ROWB;  // key block 1 / value rows 16..31
  constexpr int KQ = C::KQ;
  // the first MFMA waits for its reads while the rest stay in flight (the LDS
  // counter holds at most 15 outstanding reads)
  constexpr int KPRE = KQ > 7 ? 7 : KQ;
  const int lane = threadIdx.x & 63, g = lane >> 4;
  typedef __attribute__((address_space(3))) const bf16x8 *lds_b8;
  // ---- scores S^T = K Q^T: lane (g, n) gets keys 16 kb + 4 g + i of row n
  bf16x8 ka[2][KQ];
  // nothing of this wave's is outstanding on the LDS here; saying so lets the
  // waits below count only this tile's reads
  __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
  for (int kk = 0; kk < KPRE; ++kk) {
    const uint32_t a = tile + ofs.ko[kk];
    ka[0][kk] = *(lds_b8)(lds_ptr(a));
    ka[1][kk] = *(lds_b8)(lds_ptr(a + KB1));
  }
  __builtin_amdgcn_sched_barrier(0);
  // Even and odd k-steps accumulate separately (four independent MFMA chains per
  // block instead of two: one wave cannot issue a dependent MFMA until the previous
  // one is done), then the two halves are added.
  floatx4 s[NB][2], s2[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) s[b][0] = s[b][1] = s2[b][0] = s2[b][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) {
    if (kk + KPRE < KQ) {
      const uint32_t a = tile + ofs.ko[kk + KPRE];
      ka[0][kk + KPRE] = *(lds_b8)(lds_ptr(a));
      ka[1][kk + KPRE] = *(lds_b8)(lds_ptr(a + KB1));
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (kk & 1)
          s2[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][kk], st.q[b][kk], s2[b][kb], 0, 0, 0);
        else
          s[b][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][kk], st.q[b][kk], s[b][kb], 0, 0, 0);
      }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[b][kb] = s[b][kb] + s2[b][kb];
  // ---- value operands for O^T += V^T P^T.  The transposed read gives lane (g, m)
  // the values of keys 4 g + e (lo) and 16 + 4 g + e (hi), e = 0..3, at column
  // 16 db + m: the same key order as the probabilities below.
  bf16x8 va[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) {
    const uint32_t a = tile + ofs.vo[j];
    const shortx4 lo = ds_read_tr_at(a);
    const shortx4 hi = ds_read_tr_at(a + KB1);
    va[j] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                           lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  }
  // ---- online softmax, base 2, lazy max.  The running max is taken on the raw
  // scores (c2 > 0 keeps their order) and each exponent is one fused c2 s - m.
  bf16x8 pb[NB];
  float corr[NB];
  bool any_corr = false;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float z[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = s[b][kb][i];
        if constexpr (MASK) {
          if (tb + 16 * kb + 4 * g + i > pos) x = -INFINITY;
        }
        z[kb][i] = x;
        mt = fmaxf(mt, x);
      }
    mt = rows4_max(mt) * c2;
    const bool move = mt > st.m[b] + kLazyMax;  // always true on a row's first tile
    const float mn = move ? mt : st.m[b];
    corr[b] = (move && st.m[b] != -INFINITY) ? exp2_fast(st.m[b] - mn) : 1.0f;
    any_corr = any_corr || corr[b] != 1.0f;
    // probabilities rounded to bf16 in pairs; the row sum adds those rounded values
    // two at a time (a bf16 dot product with (1, 1), accumulated in float32)
    float lt = 0.0f;
    const bf16x2 ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const floatx2 e = {exp2_fast(fmaf(z[kb][i], c2, -mn)), exp2_fast(fmaf(z[kb][i + 1], c2, -mn))};
        const bf16x2 pp = __builtin_convertvector(e, bf16x2);
        lt = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, lt, false);
        pb[b][4 * kb + i] = pp[0];
        pb[b][4 * kb + i + 1] = pp[1];
      }
    lt = rows4_sum(lt);
    st.l[b] = st.l[b] * corr[b] + lt;
    st.m[b] = mn;
  }
  if (__any(any_corr)) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < NDB; ++j) st.acc[b][j] = st.acc[b][j] * corr[b];
  }
#pragma unroll
  for (int j = 0; j < NDB; ++j)
#pragma unroll
    for (int b = 0; b < NB; ++b)
      st.acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[j], pb[b], st.acc[b][j], 0, 0, 0);
}

// Normalised partial of 4 columns: acc / l rounded to bf16 (the float32 range, so any
// finite value row stays finite), packed.
__device__ __forceinline__ uint2 norm_part4(floatx4 acc, float inv_l) {
  uint2 r;
  r.x = static_cast<uint32_t>(bf16_bits(acc[0] * inv_l)) | (static_cast<uint32_t>(bf16_bits(acc[1] * inv_l)) << 16);
  r.y = static_cast<uint32_t>(bf16_bits(acc[2] * inv_l)) | (static_cast<uint32_t>(bf16_bits(acc[3] * inv_l)) << 16);
  return r;
}

__device__ __forceinline__ float part_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float part_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// A producer wave's share (IPW wave-wide loads) of the direct-to-LDS loads of a tile
// of one kv head, with NP producer waves.  Lane l of a wave-wide load lands at LDS
// (M0 + 16 l); the lane picks the global chunk that the swizzle puts there.  The
// loads are issued from inline assembly so that the compiler does not fence later
// LDS reads on them; the caller waits with wait_vm before the barrier that
// publishes the tile.  They are non-temporal (nt): each resident row is read once per
// pass, and a layer's K/V (about 270 MB at 65,536 tokens) is larger than the last-level
// cache.  With the hint a 65,536-token pass measured 49-50 us instead of 55-56 us per
// launch, and the commit after it 49 instead of 53 us.
template <int D, int NP>
struct KvDma {
  static constexpr int IPW = KvCfg<D>::LOADS / NP;
  static_assert(KvCfg<D>::LOADS % NP == 0, "loads per producer wave");
  uint32_t off[IPW];  // byte offset of this lane's chunk within the tile's rows
  int ins0;           // first wave-wide load of this wave (uniform)
  __device__ __forceinline__ void init(int pw) {
    using C = KvCfg<D>;
    ins0 = __builtin_amdgcn_readfirstlane(pw) * IPW;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int li = (ins0 + x) % (C::LOADS / 2);
      const int row = li * C::RPL + lane / C::CPR;
      const int cs = lane % C::CPR;
      off[x] = static_cast<uint32_t>(row * C::ROWB + ((cs ^ swz<D>(row)) << 4));
    }
  }
  // Rows [tb, tb + kKvTile) into `stage`.
  __device__ __forceinline__ void issue(unsigned char *stage, __amdgpu_buffer_rsrc_t kres,
                                        __amdgpu_buffer_rsrc_t vres, int64_t tb) const {
    using C = KvCfg<D>;
    const uint32_t base = static_cast<uint32_t>(tb * C::ROWB);
    const uint32_t lds = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char *)(stage)));
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
      const int ins = ins0 + x;
      const bool v = ins >= C::LOADS / 2;  // uniform over the wave
      asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen nt lds"
                   :
                   : "v"(base + off[x]), "s"(__builtin_amdgcn_readfirstlane(lds + ins * 1024)), "s"(v ? vres : kres)
                   : "memory", "m0");
    }
  }
};

// ============================================================================ split pass

// Byte offset of (row, column) in the bf16 partials of (kv head h, split s): rows
// of D values, so that the fold reads 16 contiguous bytes per 8 columns.
template <int D>
__device__ __forceinline__ int64_t part_off(const KvTree &T, int h, int s, int row, int col) {
  return (((static_cast<int64_t>(h) * T.nsplit_cap + s) * T.rows_cap + row) * D + col) * 2;
}

// W waves of which the first CW = W - PW compute (NB row blocks each) and the last
// PW only issue the tile loads (PW = 0: every wave issues its share of them).  The
// producer waves keep the load queue full without holding up the MFMA and softmax
// work of the others.
template <int D, int W, int NB, int PW>
__global__ __launch_bounds__(W * 64) void kv_split_kernel(const KvLaunch P) {
  using C = KvCfg<D>;
  constexpr int S = kKvStages;
  constexpr int CW = W - PW;              // computing waves
  constexpr int NP = PW > 0 ? PW : W;     // producer waves
  constexpr int IPW = KvDma<D, NP>::IPW;
  static_assert((S - 2) * IPW <= 63, "loads in flight per wave");
  __shared__ __align__(1024) unsigned char ring[S][C::TILE];
  // grid: x = item of the tree, y = tree
  const KvTree &T = P.t[blockIdx.y];
  scalar_touch(&T, sizeof(KvTree), &P.n_trees);
  // Workgroup x covers (kv head, split) pair p and row group rg: pairs go in runs of
  // 8, and the row groups of a run follow one another 8 apart, so that the row groups
  // of one split land on one XCD (workgroups are dealt to the 8 XCDs in turn) and
  // read its tiles through one L2.
  const int local = blockIdx.x;
  const int run = local / (8 * T.row_groups), rem = local % (8 * T.row_groups);
  const int rg = rem / 8, pair = run * 8 + rem % 8;
  if (pair >= P.hkv * T.a_splits) return;
  const int h = pair / T.a_splits, s = pair % T.a_splits;
  const bool carry = s == T.n_full;  // the tiles of split n_full below tb0
  const int G = P.hq / P.hkv;
  const int M = T.gn * G;  // rows of the group: (group node, q head)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, ln = lane & 15;
  const int split_tiles = T.split / kKvTile;
  const int ntiles = carry ? T.carry_tiles : split_tiles;
  const int64_t tile0 = static_cast<int64_t>(s) * split_tiles;
  // Row blocks of the item: [rblk0, rblk0 + nblk); wave w < CW takes blocks
  // rblk0 + NB w + k.  Waves past the rows do not compute.
  const int rblk0 = rg * CW * NB;
  const int nblk = min(CW * NB, (M + 15) / 16 - rblk0);
  const bool computes = wave < CW && wave * NB < nblk;
  const bool producer = PW == 0 || wave >= CW;  // uniform over the wave
  const int pw = PW == 0 ? wave : wave - CW;

  const unsigned char *kc = static_cast<const unsigned char *>(T.kc) + static_cast<int64_t>(h) * T.cap * C::ROWB;
  const unsigned char *vc = static_cast<const unsigned char *>(T.vc) + static_cast<int64_t>(h) * T.cap * C::ROWB;
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(kc, T.L * C::ROWB);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(vc, T.L * C::ROWB);

  // ---- prologue: the producers put tiles 0 .. S - 2 in flight while the computing
  // waves load their query rows straight into registers (rows past the tree's
  // repeat its last row); everyone waits for tile 0.
  KvDma<D, NP> dma;
  dma.init(pw);
  const int first = min(S - 1, ntiles);
  if (producer)
    for (int x = 0; x < first; ++x) dma.issue(ring[x], kres, vres, (tile0 + x) * kKvTile);
  KvRows<D, NB, C::DB> st;
  KvLane<D, C::DB> ofs;
  ofs.init(0);
  if (computes) {
    const unsigned char *qb = static_cast<const unsigned char *>(T.q);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int r = min(16 * (rblk0 + NB * wave + k) + ln, M - 1);
      const int gi = r / G;
      const int node = static_cast<int8_t>(
          (reinterpret_cast<const uint32_t *>(T.nodes)[gi >> 2] >> (8 * (gi & 3))) & 0xFFu);
      const unsigned char *qr = qb + (static_cast<int64_t>(node) * P.hq + h * G + r % G) * C::ROWB;
#pragma unroll
      for (int kk = 0; kk < C::KQ; ++kk) st.q[k][kk] = *reinterpret_cast<const bf16x8 *>(qr + (4 * kk + g) * 16);
    }
  }
  if (producer) {
    switch (first - 1) {  // tiles 1 .. first - 1 stay in flight
      case 3: wait_vm<3 * IPW>(); break;
      case 2: wait_vm<2 * IPW>(); break;
      case 1: wait_vm<IPW>(); break;
      default: wait_vm<0>(); break;
    }
  } else {
    wait_vm<0>();  // the query rows
  }
  bare_barrier();  // tile 0 is in LDS
  st.reset();
  const uint32_t ring0 = lds_addr(ring[0]);
  int stage = 0;  // tt % S
  for (int tt = 0; tt < ntiles; ++tt) {
    if (tt > 0) {
      // tiles tt .. tt + ahead are in flight; wait for tile tt
      const int ahead = min(S - 2, ntiles - 1 - tt);
      if (ahead >= 3) {
        wait_vm<3 * IPW>();
      } else if (ahead == 2) {
        wait_vm<2 * IPW>();
      } else if (ahead == 1) {
        wait_vm<IPW>();
      } else {
        wait_vm<0>();
      }
      bare_barrier();  // tile tt landed for every wave; tile tt - 1 is no longer read
    }
    if (producer && tt + S - 1 < ntiles)
      dma.issue(ring[stage == 0 ? S - 1 : stage - 1], kres, vres, (tile0 + tt + S - 1) * kKvTile);
    if (computes) kv_tile<D, NB, C::DB, false>(st, ring0 + stage * C::TILE, ofs, 0, 0, P.c2);
    stage = stage == S - 1 ? 0 : stage + 1;
  }
  // ---- epilogue.  The partials go out as whole rows: each wave writes its block's
  // normalised bf16 values into its own padded region of the (now idle) ring, then
  // stores them back 16 contiguous bytes per lane, two rows per wave-wide store.
  // The stores are non-temporal: every workgroup writes its partials at about the same
  // time, at the end of the pass, and the tree pass reads them once.
  constexpr int SROW = C::ROWB + 16;  // padded row: the 16 rows of a column group hit distinct banks
  static_assert(CW * 16 * SROW <= S * C::TILE, "staging area");
  bare_barrier();  // every wave is past its last tile
  if (!computes) return;
  unsigned char *stage_w = &ring[0][0] + wave * 16 * SROW;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int blk = rblk0 + NB * wave + k;
    const int row = 16 * blk + ln;
    if (!carry) {
      const float inv_l = 1.0f / st.l[k];
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        *reinterpret_cast<uint2 *>(stage_w + ln * SROW + (16 * db + 4 * g) * 2) = norm_part4(st.acc[k][db], inv_l);
      if (g == 0 && row < M) {
        const int64_t prow = (static_cast<int64_t>(h) * T.nsplit_cap + s) * T.rows_cap + row;
        __builtin_nontemporal_store(floatx2{st.m[k], st.l[k]}, reinterpret_cast<floatx2 *>(T.part_ml + prow * 2));
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the wave's staged rows are in LDS
      unsigned char *po = static_cast<unsigned char *>(T.part_o);
#pragma unroll
      for (int i = 0; i < 16 * C::CPR / 64; ++i) {
        const int x = 64 * i + lane, rl = x / C::CPR, cc = x % C::CPR;
        const uint4 v = *reinterpret_cast<const uint4 *>(stage_w + rl * SROW + cc * 16);
        if (16 * blk + rl < M)
          __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<u32x4 *>(po + part_off<D>(T, h, s, 16 * blk + rl, cc * 8)));
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // read back before the next block reuses the region
    } else if (row < M) {
      const int64_t crow = static_cast<int64_t>(h) * T.rows_cap + row;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        *reinterpret_cast<floatx4 *>(T.carry_acc + crow * D + 16 * db + 4 * g) = st.acc[k][db];
      if (g == 0) *reinterpret_cast<float2 *>(T.carry_ml + crow * 2) = make_float2(st.m[k], st.l[k]);
    }
  }
}

// ============================================================================ tree pass

// Running softmax state of one row over 8 output columns: max (base 2), sum, and
// the weighted column sums relative to that max.
struct Fold8 {
  float m, l;
  float x[8];
};

__device__ __forceinline__ void fold8_empty(Fold8 &f) {
  f.m = -INFINITY;
  f.l = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.x[e] = 0.0f;
}

// f <- f (+) y for states relative to their own maxima.  Symmetric in f and y bit
// for bit (products and sums of the same two terms), so lanes that swap operands
// agree.  Neither may be empty.
__device__ __forceinline__ void fold8_merge(Fold8 &f, const Fold8 &y) {
  const float mn = fmaxf(f.m, y.m);
  const float a = exp2_fast(f.m - mn), b = exp2_fast(y.m - mn);
  f.l = f.l * a + y.l * b;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.x[e] = f.x[e] * a + y.x[e] * b;
  f.m = mn;
}

// The same state as held by the lane 16 (SWAP16) or 32 lanes away.
template <bool SWAP16>
__device__ __forceinline__ Fold8 fold8_partner(const Fold8 &f) {
  Fold8 y;
  auto pick = [](float v) {
    const auto r = SWAP16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
                          : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    // r[0] and r[1] are this lane's value and the partner's, in lane order
    const bool upper = SWAP16 ? ((threadIdx.x >> 4) & 1) : ((threadIdx.x >> 5) & 1);
    return __uint_as_float(upper ? r[0] : r[1]);
  };
  y.m = pick(f.m);
  y.l = pick(f.l);
#pragma unroll
  for (int e = 0; e < 8; ++e) y.x[e] = pick(f.x[e]);
  return y;
}

constexpr int kFoldChunk = 16;  // split partials in flight per fold lane

// MAX_TILES: the most kKvTile-key tiles from tb0 to a node's position over the launch's
// nodes (the host picks it).  Two tiles (a node within 2 kKvTile - 1 keys of tb0, as in
// every tree of depth < kKvTile) leave room for two workgroups on a CU; three cover any
// tree (kKvTile - 1 committed rows past tb0 and depth up to kMaxNodes - 1).
template <int D, int MAX_TILES>
__global__ __launch_bounds__(kKvThreads) void kv_tree_kernel(const KvLaunch P) {
  using C = KvCfg<D>;
  constexpr int QD = C::QD, QDB = C::QDB, QO = QD / 8;  // 8-column groups per quarter
  static_assert(MAX_TILES == 2 || MAX_TILES == 3, "tree tiles");
  static_assert((kKvTile - 1 + kMaxNodes - 1) / kKvTile + 1 <= 3, "three tiles cover any tree");
  __shared__ __align__(1024) unsigned char tiles[MAX_TILES][C::TILE];
  __shared__ __align__(16) float x_o[16][QD];   // finished split n_full (crossing), bf16 values
  __shared__ float x_ml[16][2];
  __shared__ __align__(16) float f_acc[16][QD];  // the row's last split, float32 state
  __shared__ float f_ml[16][2];
  // grid: x = (kv head, node of the group, column quarter) of the tree, y = tree
  const KvTree &T = P.t[blockIdx.y];
  scalar_touch(&T, sizeof(KvTree), &P.n_trees);
  const int local = blockIdx.x;
  if (local >= P.hkv * T.gn * kKvQuarters) return;
  const int qd = local % kKvQuarters, rest = local / kKvQuarters;
  const int gi = rest % T.gn, h = rest / T.gn;  // gi: the node's index within the group
  const int node = static_cast<int8_t>(
      (reinterpret_cast<const uint32_t *>(T.nodes)[gi >> 2] >> (8 * (gi & 3))) & 0xFFu);
  const int G = P.hq / P.hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, ln = lane & 15;
  // depth by a scalar load of the 32-bit word that holds it (the tree arrays are
  // bytes; a byte load from the argument block would be a vector load)
  const int dep = static_cast<int8_t>(
      (reinterpret_cast<const uint32_t *>(T.depth)[node >> 2] >> (8 * (node & 3))) & 0xFFu);
  const int64_t L = T.L, pos = L + dep;
  const int64_t tb0 = (L / kKvTile) * kKvTile;
  const int ntree = static_cast<int>((pos / kKvTile) * kKvTile - tb0) / kKvTile + 1;
  const bool crossing = pos / T.split > T.n_full;  // at most one boundary: split > 94
  const unsigned char *kt = static_cast<const unsigned char *>(T.kt);
  const unsigned char *vt = static_cast<const unsigned char *>(T.vt);
  const unsigned char *kc = static_cast<const unsigned char *>(T.kc) + static_cast<int64_t>(h) * T.cap * C::ROWB;
  const unsigned char *vc = static_cast<const unsigned char *>(T.vc) + static_cast<int64_t>(h) * T.cap * C::ROWB;

  if (wave == 0) {
    // ---- ancestors first (scalar walk over the parent array held in a VGPR):
    // lane d holds the node's ancestor at depth d
    // the parent array as uniform words (scalar loads from the launch block), spread
    // over the lanes: lane i holds parent[i]
    const uint32_t *pw = reinterpret_cast<const uint32_t *>(T.parent);
    const int pl = min(lane, T.n - 1);
    uint32_t par_w = 0;
#pragma unroll
    for (int i = 0; i < kMaxNodes / 4; ++i) par_w = (pl >> 2) == i ? pw[i] : par_w;
    const int par_v = static_cast<int8_t>((par_w >> (8 * (pl & 3))) & 0xFFu);
    int anc_v = node;
    {
      int x = node;
      for (int d = dep; d >= 0; --d) {
        anc_v = lane == d ? x : anc_v;
        x = __builtin_amdgcn_readlane(par_v, max(x, 0));
      }
    }
    // ---- the queries and the carried state of split n_full, in flight with the
    // gather below (lanes past the node's q heads read a real row and are
    // discarded; without a carry the loads read the buffer and are dropped)
    KvRows<D, 1, QDB> st;
    KvLane<D, QDB> ofs;
    ofs.init(qd * QDB);
    const int jr = min(ln, G - 1);
    {
      const unsigned char *qrow =
          static_cast<const unsigned char *>(T.q) + (static_cast<int64_t>(node) * P.hq + h * G + jr) * C::ROWB;
#pragma unroll
      for (int kk = 0; kk < C::KQ; ++kk) st.q[0][kk] = *reinterpret_cast<const bf16x8 *>(qrow + (32 * kk + 8 * g) * 2);
    }
    const int64_t crow = static_cast<int64_t>(h) * T.rows_cap + gi * G + jr;
    const float2 cml = *reinterpret_cast<const float2 *>(T.carry_ml + crow * 2);
    floatx4 cacc[QDB];
#pragma unroll
    for (int j = 0; j < QDB; ++j)
      cacc[j] = *reinterpret_cast<const floatx4 *>(T.carry_acc + crow * D + 16 * (qd * QDB + j) + 4 * g);
    // ---- gather the node's tiles into LDS: committed rows from tb0 below L, then
    // the ancestors' tree rows up to the node's own (position pos).  Only those rows
    // are loaded (a wave-wide load covers RPL rows; a part-filled last one takes the
    // node's own row); the masked value rows past them are zeroed so that their
    // zero probabilities multiply finite values.  Rows are counted from tb0 in
    // 32-bit; lane d of trow_v holds the byte offset of the tree row at depth d.  The
    // RPL rows of a load have uniform depths, so their tree rows come from readlane.
    const int lres = static_cast<int>(L - tb0);  // committed rows in the first tile
    const int nreal = lres + dep + 1;            // rows tb0 .. pos
    const int trow_v = ((lane <= dep ? anc_v : node) * P.hkv + h) * C::ROWB;
    const unsigned char *kres0 = kc + tb0 * C::ROWB;
    const unsigned char *vres0 = vc + tb0 * C::ROWB;
    const int rr = lane / C::CPR, cs = lane % C::CPR;
    for (int tt = 0; tt < ntree; ++tt) {
      const int nl = (min(kKvTile, nreal - kKvTile * tt) + C::RPL - 1) / C::RPL;  // loads per half
      for (int x = nl * 64 + lane; x < C::LOADS / 2 * 64; x += 64)
        *reinterpret_cast<uint4 *>(tiles[tt] + C::HALF + 16 * x) = make_uint4(0, 0, 0, 0);
      for (int li = 0; li < nl; ++li) {
        const int row = li * C::RPL + rr;  // row within the tile
        const int rbase = kKvTile * tt + li * C::RPL;
        int toff = 0;
#pragma unroll
        for (int q = 0; q < C::RPL; ++q) {
          const int dq = min(max(rbase + q - lres, 0), 63);  // uniform
          const int tq = __builtin_amdgcn_readlane(trow_v, dq);
          toff = rr == q ? tq : toff;
        }
        const int rel = rbase + rr;
        const int off_c = (cs ^ swz<D>(row)) << 4;
        const bool res = rel < lres;
        const unsigned char *ksrc = (res ? kres0 + rel * C::ROWB : kt + toff) + off_c;
        const unsigned char *vsrc = (res ? vres0 + rel * C::ROWB : vt + toff) + off_c;
        __builtin_amdgcn_global_load_lds(
            ksrc, (__attribute__((address_space(3))) void *)(tiles[tt] + li * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            vsrc, (__attribute__((address_space(3))) void *)(tiles[tt] + C::HALF + li * 1024), 16, 0, 0);
      }
    }
    st.reset();
    if (T.carry_tiles > 0) {
      st.m[0] = cml.x;
      st.l[0] = cml.y;
#pragma unroll
      for (int j = 0; j < QDB; ++j) st.acc[0][j] = cacc[j];
    }
    wait_vm<0>();  // the gathered tiles are in LDS
    for (int tt = 0; tt < ntree; ++tt) {
      const int64_t tb = tb0 + static_cast<int64_t>(kKvTile) * tt;
      if (tt > 0 && tb % T.split == 0) {
        // split n_full ends here: it enters the fold as a normalised partial
        if (ln < G) {
          const float inv_l = 1.0f / st.l[0];
#pragma unroll
          for (int j = 0; j < QDB; ++j) {
            const uint2 hv = norm_part4(st.acc[0][j], inv_l);
            float *dst = &x_o[ln][16 * j + 4 * g];
            dst[0] = part_lo(hv.x);
            dst[1] = part_hi(hv.x);
            dst[2] = part_lo(hv.y);
            dst[3] = part_hi(hv.y);
          }
          if (g == 0) {
            x_ml[ln][0] = st.m[0];
            x_ml[ln][1] = st.l[0];
          }
        }
        st.reset();
      }
      kv_tile<D, 1, QDB, true>(st, lds_addr(tiles[tt]), ofs, tb, pos, P.c2);
    }
    if (ln < G) {
#pragma unroll
      for (int j = 0; j < QDB; ++j) *reinterpret_cast<floatx4 *>(&f_acc[ln][16 * j + 4 * g]) = st.acc[0][j];
      if (g == 0) {
        f_ml[ln][0] = st.m[0];
        f_ml[ln][1] = st.l[0];
      }
    }
  }

  // ---- waves 1..3: the pending rows, then the fold of the split partials
  if (wave == 1 && qd == 0) {
    // this node's tree rows go to the cache's pending row L + node
    for (int c = lane; c < 2 * C::CPR; c += 64) {
      const int which = c / C::CPR, cc = c % C::CPR;
      const uint4 x = *reinterpret_cast<const uint4 *>((which ? vt : kt) +
                                                       (static_cast<int64_t>(node) * P.hkv + h) * C::ROWB + cc * 16);
      unsigned char *dst = static_cast<unsigned char *>(which ? T.vc : T.kc) +
                           (static_cast<int64_t>(h) * T.cap + L + node) * C::ROWB + cc * 16;
      *reinterpret_cast<uint4 *>(dst) = x;
    }
  }
  // The row's splits before its last (the committed ones, then split n_full if the
  // node's rows cross into the next split: n_nl in all) fold in four ranges of
  // consecutive splits, one per 16-lane row of a fold wave; lane (sq, it) of fold
  // wave w takes item (w - 1) * 16 + it = (q head, 8-column group) and range sq.
  // A range folds in chunks of kFoldChunk (the chunk's max, then weighted sums in
  // ascending split order; chunks merge in order).  The ranges then merge as
  // (0 (+) 1) (+) (2 (+) 3), then the last split's float32 state.
  const int n_nl = T.n_full + (crossing ? 1 : 0);
  const int per = (n_nl + 3) / 4;
  const int sq = lane >> 4, it = (wave - 1) * 16 + (lane & 15);
  const int items = G * QO;
  const bool fold_lane = wave > 0 && it < items;
  const int r = min(it / QO, G - 1), co = it % QO;
  const int R = gi * G + r;
  const int col = qd * QD + 8 * co;
  const int s_lo = min(sq * per, n_nl), s_hi = min(s_lo + per, n_nl);
  Fold8 acc8;
  fold8_empty(acc8);
  float2 mlv[kFoldChunk];
  uint4 ov[kFoldChunk];
  auto load_chunk = [&](int c0, int nm) {  // loads past the memory splits repeat the last one
#pragma unroll
    for (int j = 0; j < kFoldChunk; ++j) {
      const int sj = c0 + max(0, min(j, nm - 1));
      const int64_t prow = (static_cast<int64_t>(h) * T.nsplit_cap + sj) * T.rows_cap + R;
      mlv[j] = *reinterpret_cast<const float2 *>(T.part_ml + prow * 2);
      ov[j] = *reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(T.part_o) +
                                               part_off<D>(T, h, sj, R, col));
    }
  };
  // fold splits [c0, c0 + ns) of the loaded chunk; index jx (if >= 0) is the
  // crossing partial, taken from LDS
  auto fold_chunk = [&](int ns, int jx) {
    float mc = -INFINITY;
#pragma unroll
    for (int j = 0; j < kFoldChunk; ++j)
      if (j < ns) mc = fmaxf(mc, j == jx ? x_ml[r][0] : mlv[j].x);
    Fold8 ch;
    fold8_empty(ch);
    ch.m = mc;
#pragma unroll
    for (int j = 0; j < kFoldChunk; ++j) {
      if (j < ns) {
        const bool x = j == jx;
        const float w = (x ? x_ml[r][1] : mlv[j].y) * exp2_fast((x ? x_ml[r][0] : mlv[j].x) - mc);
        float o[8];
        if (x) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = x_o[r][8 * co + e];
        } else {
          o[0] = part_lo(ov[j].x);
          o[1] = part_hi(ov[j].x);
          o[2] = part_lo(ov[j].y);
          o[3] = part_hi(ov[j].y);
          o[4] = part_lo(ov[j].z);
          o[5] = part_hi(ov[j].z);
          o[6] = part_lo(ov[j].w);
          o[7] = part_hi(ov[j].w);
        }
        ch.l = ch.l + w;
#pragma unroll
        for (int e = 0; e < 8; ++e) ch.x[e] = ch.x[e] + w * o[e];
      }
    }
    if (acc8.m == -INFINITY && acc8.l == 0.0f) {
      acc8 = ch;
    } else {
      fold8_merge(acc8, ch);
    }
  };
  // chunks of this range wholly in memory fold now; a chunk that holds the
  // crossing partial waits for wave 0
  int c_defer = -1, ns_defer = 0;
  if (fold_lane) {
    for (int c0 = s_lo; c0 < s_hi; c0 += kFoldChunk) {
      const int ns = min(kFoldChunk, s_hi - c0);
      const int nm = min(ns, T.n_full - c0);
      load_chunk(c0, nm);
      if (nm < ns) {  // holds split n_full, finished by wave 0
        c_defer = c0;
        ns_defer = ns;
        break;
      }
      fold_chunk(ns, -1);
    }
  }
  __syncthreads();
  if (wave > 0) {
    if (fold_lane && c_defer >= 0) fold_chunk(ns_defer, T.n_full - c_defer);
    // merge the four ranges: (0 (+) 1) (+) (2 (+) 3); empty ranges (more lanes
    // than splits) contribute nothing
    const bool has = s_lo < s_hi;
    {
      Fold8 y = fold8_partner<true>(acc8);
      const bool yhas = __shfl_xor(static_cast<int>(has), 16) != 0;
      if (has && yhas) {
        if ((lane >> 4) & 1) { Fold8 lo = y; fold8_merge(lo, acc8); acc8 = lo; } else { fold8_merge(acc8, y); }
      } else if (yhas) {
        acc8 = y;
      }
    }
    const bool has2 = has || (__shfl_xor(static_cast<int>(has), 16) != 0);
    {
      Fold8 y = fold8_partner<false>(acc8);
      const bool yhas = __shfl_xor(static_cast<int>(has2), 32) != 0;
      if (has2 && yhas) {
        if ((lane >> 5) & 1) { Fold8 lo = y; fold8_merge(lo, acc8); acc8 = lo; } else { fold8_merge(acc8, y); }
      } else if (yhas) {
        acc8 = y;
      }
    }
    if (fold_lane && sq == 0) {
      Fold8 last;
      last.m = f_ml[r][0];
      last.l = f_ml[r][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) last.x[e] = f_acc[r][8 * co + e];
      if (n_nl > 0) {
        fold8_merge(acc8, last);
      } else {
        acc8 = last;
      }
      const float inv = 1.0f / acc8.l;
      uint4 w;
      w.x = static_cast<uint32_t>(bf16_bits(acc8.x[0] * inv)) | (static_cast<uint32_t>(bf16_bits(acc8.x[1] * inv)) << 16);
      w.y = static_cast<uint32_t>(bf16_bits(acc8.x[2] * inv)) | (static_cast<uint32_t>(bf16_bits(acc8.x[3] * inv)) << 16);
      w.z = static_cast<uint32_t>(bf16_bits(acc8.x[4] * inv)) | (static_cast<uint32_t>(bf16_bits(acc8.x[5] * inv)) << 16);
      w.w = static_cast<uint32_t>(bf16_bits(acc8.x[6] * inv)) | (static_cast<uint32_t>(bf16_bits(acc8.x[7] * inv)) << 16);
      *reinterpret_cast<uint4 *>(static_cast<unsigned char *>(T.o) +
                                 ((static_cast<int64_t>(node) * P.hq + h * G + r) * D + col) * 2) = w;
    }
  }
}

}  // namespace

hipError_t launch_kv_split(const KvLaunch &a, int D, int max_items, hipStream_t s, KernelEvents ev) {
  const dim3 grid(max_items, a.n_trees);
  static_assert(kKvRowsPerItem == 6 * 16, "six computing waves of one block");
  if (D == 256) {
    hipExtLaunchKernelGGL((kv_split_kernel<256, 8, 1, 2>), grid, dim3(8 * 64), 0, s, ev.start, ev.stop, 0, a);
  } else if (D == 64) {
    hipExtLaunchKernelGGL((kv_split_kernel<64, 8, 1, 2>), grid, dim3(8 * 64), 0, s, ev.start, ev.stop, 0, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kv_tree(const KvLaunch &a, int D, int max_items, int tiles, hipStream_t s, KernelEvents ev) {
  const dim3 grid(max_items, a.n_trees);
  if (tiles < 1 || tiles > 3) return hipErrorInvalidValue;
#define HDT_TREE(DD, NT) \
  hipExtLaunchKernelGGL((kv_tree_kernel<DD, NT>), grid, dim3(kKvThreads), 0, s, ev.start, ev.stop, 0, a)
  if (D == 256) {
    if (tiles <= 2) HDT_TREE(256, 2); else HDT_TREE(256, 3);
  } else if (D == 64) {
    if (tiles <= 2) HDT_TREE(64, 2); else HDT_TREE(64, 3);
  } else {
    return hipErrorInvalidValue;
  }
#undef HDT_TREE
  return hipGetLastError();
}

}  // namespace hdt
