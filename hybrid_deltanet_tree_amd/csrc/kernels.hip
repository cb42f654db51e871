// kernels.hip - tree-verify kernels for CDNA4 (gfx950).
//
//  gdn_tree_kernel    one Gated DeltaNet layer over a tree: every value head
//                     advances its recurrent state along every root-to-node path
//                     ("Adding a model", "What is still specific to Qwen3.8":
//                     state heads of 128 by 128; the step is the published gated
//                     delta rule).
//  attn_split_kernel  one attention layer with float32 storage (the small
//                     parity configuration): ancestor-masked GQA over the
//                     committed rows plus the tree's own rows ("One request, end
//                     to end", 2.6), as per-split partial softmax results.
//                     bf16 storage runs the kernels of kv_attention.hip.
//  attn_fold_kernel   folds a row's split partials in ascending split order.
//  commit_kernel      commit_tree: replays the accepted path's rank-1 steps into
//                     every GDN layer's committed state, gathers the path's
//                     pending K/V rows into place ("One request, end to end", 2.6)
//                     and rolls the path's pre-conv rows into the conv tails.
//
// Bit-exactness (a verified row equals the decode step's row, "Adding a model",
// step 4 of "The adapter path in ten steps"): every value a row gets is a
// function of that row's inputs alone.
//  - GDN: one step function (decay, k^T S with a fixed lane reduction, rank-1
//    write, S q with the same reduction) serves tree nodes, decode steps, the
//    replays that restore a branch point, and commit.  The write is
//    fmaf(k, u, alpha * P) everywhere, so a replay or commit reproduces the
//    pass's state bit for bit.
//  - Attention: tiles of kTile keys and splits of `split` keys are anchored at
//    absolute positions; each tile is reduced by the same MFMA sequence whatever
//    other rows share the instruction; masked key slots hold exact zeros; splits
//    fold in ascending order.
#include "common.h"

#include <mutex>

#pragma clang fp contract(off)

namespace hdt {
namespace {

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits
// (each stage adds the same two partials in either order).
__device__ __forceinline__ float rowsum16(float x) {
  x = x + dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x = x + dpp<0x141>(x);  // row_half_mirror
  x = x + dpp<0x140>(x);  // row_mirror
  return x;
}

// ============================================================================ GDN

// LDS layout of the GDN walk: k[n+1][dk] and s*q[n+1][dk] (float); per node
// {alpha, beta, k . s q, parent} (float4) [n+1]; v[n+1][16], u[n][16], o[n][16]
// (float); depth[n] and parent[n] (int); then the kept states [n_saves][16][dk]
// (float); then save[n] and, when some tree of the launch replays a root path,
// anc[n][64] (int8).  Row n of the operand arrays is never
// written: the walk's operand load after the last node reads it and drops it.
__host__ __device__ constexpr size_t gdn_lds_floats(int dk, int n) {
  return static_cast<size_t>(n + 1) * (2 * dk + 4 + kGdnCols) + static_cast<size_t>(n) * 2 * kGdnCols +
         ((2 * n + 3) & ~3);
}

// Sum of x[a] * y[a] over a lane's R elements in a fixed order: even and odd
// elements in two fused chains, then their sum.
template <int R>
__device__ __forceinline__ float lane_dot(const float *x, const float *y) {
  float s0 = x[0] * y[0], s1 = x[1] * y[1];
#pragma unroll
  for (int a = 2; a < R; a += 2) {
    s0 = fmaf(x[a], y[a], s0);
    s1 = fmaf(x[a + 1], y[a + 1], s1);
  }
  return s0 + s1;
}

template <int R>
__device__ __forceinline__ void lds_row(const float *src, float *dst) {
#pragma unroll
  for (int a = 0; a < R; a += 4) {
    const float4 x = *reinterpret_cast<const float4 *>(src + a);
    dst[a] = x.x;
    dst[a + 1] = x.y;
    dst[a + 2] = x.z;
    dst[a + 3] = x.w;
  }
}

template <bool BF>
__device__ __forceinline__ void unpack16(const uint4 &c, float *out) {
  if constexpr (BF) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    out[0] = __uint_as_float(c.x);
    out[1] = __uint_as_float(c.y);
    out[2] = __uint_as_float(c.z);
    out[3] = __uint_as_float(c.w);
  }
}

// Sum over the LPC lanes that hold one value column (16: a DPP row; 32: two
// adjacent rows, joined by a row swap).  Every lane of the column gets the same
// bits: each stage adds the same two partials in either order.
template <int LPC>
__device__ __forceinline__ float colsum(float x) {
  static_assert(LPC == 16 || LPC == 32, "lanes per column");
  x = rowsum16(x);
  if constexpr (LPC == 32) {
    // with both operands x, the two results hold this row's and the partner row's
    // value (in an order that depends on the row): their sum is the same in both
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// Two interleaved colsum reductions.
template <int LPC>
__device__ __forceinline__ void colsum2(float &a, float &b) {
  a = a + dpp<0xB1>(a);
  b = b + dpp<0xB1>(b);
  a = a + dpp<0x4E>(a);
  b = b + dpp<0x4E>(b);
  a = a + dpp<0x141>(a);
  b = b + dpp<0x141>(b);
  a = a + dpp<0x140>(a);
  b = b + dpp<0x140>(b);
  if constexpr (LPC == 32) {
    const auto ra = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    const auto rb = __builtin_amdgcn_permlane16_swap(__float_as_uint(b), __float_as_uint(b), false, false);
    a = __uint_as_float(ra[0]) + __uint_as_float(ra[1]);
    b = __uint_as_float(rb[0]) + __uint_as_float(rb[1]);
  }
}

// Sum over the N consecutive lanes (8, 16 or 32) that hold one node's chunks: the first
// 3 or 4 butterfly stages of a DPP row, joined across two rows for 32.  Every lane of the
// group gets the same bits.
template <int N>
__device__ __forceinline__ float groupsum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "lanes per node");
  x = x + dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x = x + dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x = x + dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x = x + dpp<0x140>(x);  // row_mirror
  if constexpr (N == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// One node's operands, in the registers of a lane: its key rows and s*q rows,
// {alpha, beta, k . s q, parent} and the value of the lane's column.
template <int R>
struct GdnNode {
  float k[R], q[R];
  float4 sc;
  float v;
};

template <bool BF, int DK>
__global__ __launch_bounds__(gdn_threads(DK)) void gdn_tree_kernel(const GdnLaunch P) {
  constexpr int LPC = kGdnLanes;             // lanes per value column
  constexpr int R = DK / LPC;                // key rows per lane
  constexpr int CPW = 64 / LPC;              // value columns per wave
  constexpr int NT = gdn_threads(DK);        // kGdnCols / CPW waves
  static_assert(NT == kGdnCols / CPW * 64, "workgroup shape");
  constexpr int ESZ = BF ? 2 : 4;
  constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
  constexpr int CPR = DK / EPC;              // chunks per q/k row
  constexpr int MAXC = (kMaxNodes * CPR + NT - 1) / NT;
  constexpr int VCH = kGdnCols / EPC;        // chunks of one node's 16 value columns
  extern __shared__ __align__(16) float g_lds[];
  // grid: x = (v head, column group), y = tree
  const GdnTree &T = P.t[blockIdx.y];
  scalar_touch(&T, sizeof(GdnTree), &P.n_trees);
  // which nodes restore their parent's state first (the parent is not the node just
  // finished) and which keep theirs for later siblings, tested per node as scalar
  // bits; the opaque copies keep their loads here, waited on once, out of the walk
  uint64_t restore_mask = T.restore_mask, keep_mask = T.keep_mask;
  asm volatile("" : "+s"(restore_mask), "+s"(keep_mask));
  const int n = T.n;
  const int nm = P.n_max;
  float *kf = g_lds;
  float *qs = kf + (nm + 1) * DK;
  float4 *nsc = reinterpret_cast<float4 *>(qs + (nm + 1) * DK);
  float *vl = reinterpret_cast<float *>(nsc + nm + 1);
  float *ul = vl + (nm + 1) * kGdnCols;
  float *ol = ul + nm * kGdnCols;
  int *dep = reinterpret_cast<int *>(ol + nm * kGdnCols);  // depth[n], then parent[n]
  float *kept = reinterpret_cast<float *>(dep + ((2 * nm + 3) & ~3));  // 16-byte aligned
  int8_t *savel = reinterpret_cast<int8_t *>(kept + P.n_saves * kGdnCols * DK);
  int8_t *anc = savel + nm;  // allocated when P.any_anc (touched only when T.need_anc)

  const int cgroups = P.dv / kGdnCols;
  const int local = blockIdx.x;
  const int h = local / cgroups, cg = local % cgroups;
  const int ratio = P.hv / P.hk, qh = h / ratio;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lc = wave * CPW + lane / LPC;  // value column within the workgroup
  const int g = lane % LPC;                // key rows [g*R, g*R+R)
  const int col = cg * kGdnCols + lc;

  // ---- issue every load of the prologue before using any of them (tree first)
  int par_i = -1, dep_i = 0, save_i = -1;
  if (tid < n) {
    par_i = T.parent[tid];
    dep_i = T.depth[tid];
    save_i = T.save[tid];
  }
  float base[R];
  lds_row<R>(T.state + (static_cast<int64_t>(h) * P.dv + col) * DK + g * R, base);
  const unsigned char *kb = static_cast<const unsigned char *>(T.k);
  const unsigned char *qb = static_cast<const unsigned char *>(T.q);
  uint4 kc[MAXC], qc[MAXC];
  const int nch = n * CPR;
#pragma unroll
  for (int x = 0; x < MAXC; ++x) {
    const int c = tid + x * NT;
    if (c < nch) {
      const int i = c / CPR, cc = c % CPR;
      const int64_t off = (static_cast<int64_t>(i) * P.hk + qh) * DK * ESZ + cc * 16;
      kc[x] = *reinterpret_cast<const uint4 *>(kb + off);
      qc[x] = *reinterpret_cast<const uint4 *>(qb + off);
    }
  }
  uint4 vc = make_uint4(0, 0, 0, 0);
  if (tid < n * VCH) {
    const int i = tid / VCH, cc = tid % VCH;
    vc = *reinterpret_cast<const uint4 *>(
        static_cast<const unsigned char *>(T.v) +
        ((static_cast<int64_t>(i) * P.hv + h) * P.dv + cg * kGdnCols) * ESZ + cc * 16);
  }
  io_t<BF> araw{}, braw{};
  if (tid < n) {
    araw = static_cast<const io_t<BF> *>(T.alpha)[static_cast<int64_t>(tid) * P.hv + h];
    braw = static_cast<const io_t<BF> *>(T.beta)[static_cast<int64_t>(tid) * P.hv + h];
  }

  // ---- tree metadata (ancestor table walked in LDS) and LDS staging
  if (tid < n) {
    dep[tid] = dep_i;
    dep[nm + tid] = par_i;
    savel[tid] = static_cast<int8_t>(save_i);
  }
  lds_barrier();
  if (T.need_anc && tid < n) {
    int x = tid;
    for (int k = dep_i; k >= 0; --k) {
      anc[tid * kMaxNodes + k] = static_cast<int8_t>(x);
      x = dep[nm + x];
    }
  }
  // k . s q of every node (it does not depend on the state), taken here: a node's CPR
  // chunks sit on CPR consecutive lanes, so an in-lane dot and a CPR-lane sum give it
  const bool keep_k = (cg == 0) && (h % ratio == 0);
#pragma unroll
  for (int x = 0; x < MAXC; ++x) {
    // a wave whose first chunk lies past the last node has none in this or a later round
    if (x * NT + __builtin_amdgcn_readfirstlane(tid) >= nch) break;
    const int c = tid + x * NT;
    const int i = c / CPR, cc = c % CPR;
    float kq = 0.0f;
    if (c < nch) {
      float kv[EPC], qv[EPC];
      unpack16<BF>(kc[x], kv);
      unpack16<BF>(qc[x], qv);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        qv[e] = P.scale * qv[e];
        kf[i * DK + cc * EPC + e] = kv[e];
        qs[i * DK + cc * EPC + e] = qv[e];
      }
      kq = lane_dot<EPC>(kv, qv);
      if (keep_k)  // commit replays the accepted path with these exact k bits
        *reinterpret_cast<uint4 *>(static_cast<unsigned char *>(T.k_pend) +
                                   (static_cast<int64_t>(i) * P.hk + qh) * DK * ESZ + cc * 16) = kc[x];
    }
    kq = groupsum<CPR>(kq);  // every lane takes part: the lanes past the nodes add zeros
    if (c < nch && cc == 0) nsc[i].z = kq;
  }
  if (tid < n * VCH) {
    const int i = tid / VCH, cc = tid % VCH;
    float vv[EPC];
    unpack16<BF>(vc, vv);
#pragma unroll
    for (int e = 0; e < EPC; ++e) vl[i * kGdnCols + cc * EPC + e] = vv[e];
  }
  if (tid < n) {
    float a, b;
    if constexpr (BF) {
      a = __uint_as_float(static_cast<uint32_t>(araw) << 16);
      b = __uint_as_float(static_cast<uint32_t>(braw) << 16);
    } else {
      a = araw;
      b = braw;
    }
    nsc[tid].x = a;  // .z, k . s q, is written by the staging above
    nsc[tid].y = b;
    // parent, the node's own kept slot, the parent's kept slot (-1: none), one byte each
    const int psave = par_i >= 0 ? static_cast<int>(savel[par_i]) : -1;
    nsc[tid].w = __int_as_float((par_i & 0xFF) | ((save_i & 0xFF) << 8) | ((psave & 0xFF) << 16));
    if (cg == 0) static_cast<io_t<BF> *>(T.a_pend)[static_cast<int64_t>(tid) * P.hv + h] = araw;
  }
  __syncthreads();

  // ---- walk the nodes in index order (parents first).  Per node, from the
  // parent's state P:  A = alpha P;  r = k^T A;  u = beta (v - r);  S = A + k u^T;
  // o = S^T (s q) taken as A^T (s q) + u (k . s q), so the readout does not wait
  // for the state write.  Every dot product is a lane_dot then a colsum.  The
  // loop is unrolled twice so the next node's operands load into the other set.
  float cur[R];
#pragma unroll
  for (int a = 0; a < R; ++a) cur[a] = base[a];
  // this lane's operands of the next node to load, one node further per load (the
  // load after the last node reads the spare row n); its u and o slots, one node
  // further per step
  const float *k_at = kf + g * R, *q_at = qs + g * R, *v_at = vl + lc;
  const float4 *sc_at = nsc;
  float *u_at = ul + lc, *o_at = ol + lc;
  auto load_node = [&](GdnNode<R> &x) {
    lds_row<R>(k_at, x.k);
    lds_row<R>(q_at, x.q);
    x.sc = *sc_at;
    x.v = *v_at;
    k_at += DK;
    q_at += DK;
    sc_at += 1;
    v_at += kGdnCols;
  };
  auto restore = [&](int p, int sl) {
    // the parent's state: kept in LDS (slot sl >= 0), or replayed from the committed
    // state along its root path with the same rank-1 write as the step below
    if (sl >= 0) {
      lds_row<R>(kept + (sl * kGdnCols + lc) * DK + g * R, cur);
      return;
    }
#pragma unroll
    for (int a = 0; a < R; ++a) cur[a] = base[a];
    if (p < 0) return;
    const int dp = dep[p];
    const int8_t *path = anc + p * kMaxNodes;
    int j = path[0];
    float kj[R];
    lds_row<R>(kf + j * DK + g * R, kj);
    float aj = nsc[j].x, uj = ul[j * kGdnCols + lc];
    for (int d = 0; d <= dp; ++d) {
      float kk[R];
#pragma unroll
      for (int a = 0; a < R; ++a) kk[a] = kj[a];
      const float ak = aj, uk = uj;
      if (d < dp) {
        j = path[d + 1];
        lds_row<R>(kf + j * DK + g * R, kj);
        aj = nsc[j].x;
        uj = ul[j * kGdnCols + lc];
      }
#pragma unroll
      for (int a = 0; a < R; ++a) cur[a] = fmaf(kk[a], uk, ak * cur[a]);
    }
  };
  // the parent's state into `cur` when it is not the node just finished
  auto prepare = [&](int i, const GdnNode<R> &x) {
    if ((restore_mask >> i) & 1) {
      const int w = __builtin_amdgcn_readfirstlane(__float_as_int(x.sc.w));
      restore(static_cast<int8_t>(w & 0xFF), static_cast<int8_t>((w >> 16) & 0xFF));
    }
  };
  auto step = [&](int i, const GdnNode<R> &x) {
    float A[R];
#pragma unroll
    for (int a = 0; a < R; ++a) A[a] = x.sc.x * cur[a];
    float r = lane_dot<R>(A, x.k);
    float oa = lane_dot<R>(A, x.q);
    colsum2<LPC>(r, oa);
    const float u = x.sc.y * (x.v - r);
#pragma unroll
    for (int a = 0; a < R; ++a) cur[a] = fmaf(x.k[a], u, A[a]);
    // every lane of the column stores the same bits (no branch)
    *u_at = u;
    *o_at = fmaf(u, x.sc.z, oa);
    u_at += kGdnCols;
    o_at += kGdnCols;
    if ((keep_mask >> i) & 1) {
      const int keep = static_cast<int8_t>((__builtin_amdgcn_readfirstlane(__float_as_int(x.sc.w)) >> 8) & 0xFF);
#pragma unroll
      for (int a = 0; a < R; a += 4)
        *reinterpret_cast<float4 *>(kept + (keep * kGdnCols + lc) * DK + g * R + a) =
            make_float4(cur[a], cur[a + 1], cur[a + 2], cur[a + 3]);
    }
  };
  // Per node: wait for its operands (loaded during the previous node), restore
  // the parent's state if needed, issue the next node's loads into the other
  // register set, then compute with no LDS read outstanding that the node needs.
  // The load after the last node reads the spare row, so the loads are unconditional.  LDS
  // operations of a wave complete in order, so the operands are in once at most
  // the previous node's two u / o stores are outstanding (its state copy, when
  // kept, only makes the wait longer).
  GdnNode<R> na, nb;
  load_node(na);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  for (int i = 0; i < n; i += 2) {
    __builtin_amdgcn_s_waitcnt(0xC27F);  // lgkmcnt(2)
    prepare(i, na);
    __builtin_amdgcn_sched_barrier(0);
    load_node(nb);
    __builtin_amdgcn_sched_barrier(0);
    step(i, na);
    if (i + 1 >= n) break;
    __builtin_amdgcn_s_waitcnt(0xC27F);
    prepare(i + 1, nb);
    __builtin_amdgcn_sched_barrier(0);
    load_node(na);
    __builtin_amdgcn_sched_barrier(0);
    step(i + 1, nb);
  }
  __syncthreads();
  for (int e = tid; e < n * kGdnCols; e += NT) {
    const int i = e / kGdnCols, c = e % kGdnCols;
    const int64_t idx = (static_cast<int64_t>(i) * P.hv + h) * P.dv + cg * kGdnCols + c;
    st_io<BF>(T.o, idx, ol[e]);
    T.u_pend[idx] = ul[e];
  }
  if (T.commit_state) {
    // a chain committed whole (a prefill span): `cur` is the last node's state, the
    // same bits a commit replay of the chain would write; each lane owns its slice
    float *dst = T.commit_state + (static_cast<int64_t>(h) * P.dv + col) * DK + g * R;
#pragma unroll
    for (int a = 0; a < R; a += 4)
      *reinterpret_cast<float4 *>(dst + a) = make_float4(cur[a], cur[a + 1], cur[a + 2], cur[a + 3]);
  }
}

// ============================================================================ attention

template <bool BF, int D>
struct AttnCfg {
  static constexpr int ESZ = BF ? 2 : 4;
  static constexpr int KQ = BF ? D / 32 : D / 4;  // k-steps of the score MFMA
  static constexpr int DB = D / 16;               // 16-wide value blocks
  static constexpr int ROWB = D * ESZ;            // bytes per cache row
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  // LDS tile: bf16 keys [64][D] (16-byte chunks XOR-swizzled by key), bf16 values
  // transposed [D][64] (8-byte chunks XOR-swizzled by d); f32 keys [64][D+1],
  // f32 values [64][D].
  static constexpr int K_BYTES = BF ? 64 * D * 2 : 64 * (D + 1) * 4;
  static constexpr int V_BYTES = BF ? D * 64 * 2 : 64 * D * 4;
  static constexpr int TILE_BYTES = K_BYTES + V_BYTES;
  static constexpr int KSW = (CPR > 16 ? 16 : CPR) - 1;
  // register staging of one tile
  static constexpr int NK = 64 * CPR;                        // key chunks
  static constexpr int KPT = (NK + kAttnThreads - 1) / kAttnThreads;
  static constexpr int NV = BF ? 16 * (D / 8) : 64 * CPR;    // bf16: 4 keys x 8 d units
  static constexpr int VPT = (NV + kAttnThreads - 1) / kAttnThreads;
  static constexpr int VCH = BF ? 4 : 1;                     // chunks per value unit
};

template <bool BF, int D>
struct TileStage {
  using C = AttnCfg<BF, D>;
  uint4 k[C::KPT];
  uint4 v[C::VPT][C::VCH];

  // Rows [tb, tb+64) of one head; rows at or past `lim` read as zeros.
  __device__ __forceinline__ void load(const unsigned char *kh, const unsigned char *vh,
                                       int64_t tb, int64_t lim) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int x = 0; x < C::KPT; ++x) {
      const int c = tid + x * kAttnThreads;
      const int key = c / C::CPR, cc = c % C::CPR;
      const int64_t pos = tb + key;
      if (c < C::NK && pos < lim)
        k[x] = *reinterpret_cast<const uint4 *>(kh + pos * C::ROWB + cc * 16);
      else
        k[x] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < C::VPT; ++x) {
      const int u = tid + x * kAttnThreads;
      if constexpr (BF) {
        const int kq = u % 16, dc = u / 16;  // keys 4kq..4kq+3, d 8dc..8dc+7
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int64_t pos = tb + 4 * kq + y;
          if (u < C::NV && pos < lim)
            v[x][y] = *reinterpret_cast<const uint4 *>(vh + pos * C::ROWB + dc * 16);
          else
            v[x][y] = make_uint4(0, 0, 0, 0);
        }
      } else {
        const int key = u / C::CPR, cc = u % C::CPR;
        const int64_t pos = tb + key;
        if (u < C::NV && pos < lim)
          v[x][0] = *reinterpret_cast<const uint4 *>(vh + pos * C::ROWB + cc * 16);
        else
          v[x][0] = make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(unsigned char *lk, unsigned char *lv) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int x = 0; x < C::KPT; ++x) {
      const int c = tid + x * kAttnThreads;
      if (c >= C::NK) continue;
      const int key = c / C::CPR, cc = c % C::CPR;
      if constexpr (BF) {
        *reinterpret_cast<uint4 *>(lk + key * C::ROWB + ((cc ^ (key & C::KSW)) * 16)) = k[x];
      } else {
        float *dst = reinterpret_cast<float *>(lk) + key * (D + 1) + cc * 4;
        dst[0] = __uint_as_float(k[x].x);
        dst[1] = __uint_as_float(k[x].y);
        dst[2] = __uint_as_float(k[x].z);
        dst[3] = __uint_as_float(k[x].w);
      }
    }
#pragma unroll
    for (int x = 0; x < C::VPT; ++x) {
      const int u = tid + x * kAttnThreads;
      if (u >= C::NV) continue;
      if constexpr (BF) {
        const int kq = u % 16, dc = u / 16;
        const uint32_t w[4][4] = {{v[x][0].x, v[x][0].y, v[x][0].z, v[x][0].w},
                                  {v[x][1].x, v[x][1].y, v[x][1].z, v[x][1].w},
                                  {v[x][2].x, v[x][2].y, v[x][2].z, v[x][2].w},
                                  {v[x][3].x, v[x][3].y, v[x][3].z, v[x][3].w}};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // d = 8dc + 2e (low halves) and 8dc + 2e + 1 (high halves) of keys 4kq..4kq+3
          const int d0 = 8 * dc + 2 * e, d1 = d0 + 1;
          uint2 lo, hi;
          lo.x = (w[0][e] & 0xFFFFu) | (w[1][e] << 16);
          lo.y = (w[2][e] & 0xFFFFu) | (w[3][e] << 16);
          hi.x = (w[0][e] >> 16) | (w[1][e] & 0xFFFF0000u);
          hi.y = (w[2][e] >> 16) | (w[3][e] & 0xFFFF0000u);
          *reinterpret_cast<uint2 *>(lv + d0 * 128 + ((kq ^ (d0 & 15)) * 8)) = lo;
          *reinterpret_cast<uint2 *>(lv + d1 * 128 + ((kq ^ (d1 & 15)) * 8)) = hi;
        }
      } else {
        const int key = u / C::CPR, cc = u % C::CPR;
        *reinterpret_cast<uint4 *>(lv + key * C::ROWB + cc * 16) = v[x][0];
      }
    }
  }
};

// Online-softmax state of the 16 rows of one wave.  Lane (g, n) holds row n;
// acc[db][i] is output element d = 16 db + 4 g + i of that row.
template <int D>
struct RowState {
  floatx4 acc[D / 16];
  float m, l;
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) acc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.0f;
  }
};

// One tile of kTile keys at absolute position tb, already in LDS, for the 16 rows
// of this wave.  MASK: keys past `pos` (the wave's node position) are masked; the
// tile builder left exact zeros in their K and V slots.
template <bool BF, int D, bool MASK>
__device__ __forceinline__ void attn_tile(RowState<D> &st, const void *qreg,
                                          const unsigned char *lk, const unsigned char *lv,
                                          int64_t tb, int64_t pos, float c2) {
  using C = AttnCfg<BF, D>;
  const int lane = threadIdx.x & 63, g = lane >> 4, ln = lane & 15;
  floatx4 s[4];
  // ---- scores S^T = K Q^T: lane (g, n) gets keys 16 kb + 4 g + i of row n
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int key = 16 * kb + ln;  // A-operand key of this lane
#pragma unroll
    for (int kk = 0; kk < C::KQ; ++kk) {
      if constexpr (BF) {
        const bf16x8 *qb = static_cast<const bf16x8 *>(qreg);
        const int cc = 4 * kk + g;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8 *>(lk + key * C::ROWB + ((cc ^ (key & C::KSW)) * 16));
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[kk], s[kb], 0, 0, 0);
      } else {
        const float *qf = static_cast<const float *>(qreg);
        const float a = reinterpret_cast<const float *>(lk)[key * (D + 1) + 4 * kk + g];
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf[kk], s[kb], 0, 0, 0);
      }
    }
  }
  // ---- online softmax in base 2
  float z[4][4];
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = s[kb][i] * c2;
      if constexpr (MASK) {
        if (tb + 16 * kb + 4 * g + i > pos) x = -INFINITY;
      }
      z[kb][i] = x;
      mt = fmaxf(mt, x);
    }
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float mn = fmaxf(st.m, mt);
  const float corr = exp2_fast(st.m - mn);
  float lt = 0.0f;
  float p[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float e = exp2_fast(z[kb][i] - mn);
      if constexpr (BF) e = static_cast<float>(static_cast<__bf16>(e));
      p[kb][i] = e;
      lt = lt + e;
    }
  lt = lt + __shfl_xor(lt, 16);
  lt = lt + __shfl_xor(lt, 32);
  st.l = st.l * corr + lt;
  st.m = mn;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) st.acc[db] = st.acc[db] * corr;

  // ---- O^T += V^T P^T
  if constexpr (BF) {
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      bf16x8 b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = static_cast<__bf16>(p[2 * kk2][i]);
        b[4 + i] = static_cast<__bf16>(p[2 * kk2 + 1][i]);
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int d = 16 * db + ln;
        const uint2 lo =
            *reinterpret_cast<const uint2 *>(lv + d * 128 + (((8 * kk2 + g) ^ (d & 15)) * 8));
        const uint2 hi =
            *reinterpret_cast<const uint2 *>(lv + d * 128 + (((8 * kk2 + 4 + g) ^ (d & 15)) * 8));
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, st.acc[db], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int d = 16 * db + ln;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = reinterpret_cast<const float *>(lv)[(16 * kb + 4 * g + i) * D + d];
          st.acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[kb][i], st.acc[db], 0, 0, 0);
        }
    }
  }
}

// Rewrite the LDS tile rows at positions [max(L, tb), tb + kTile) for one node:
// position L + d holds the node's ancestor at depth d while d <= depth, zeros after.
// Rows below L (committed) are left as loaded.
template <bool BF, int D>
__device__ __forceinline__ void build_node_rows(unsigned char *lk, unsigned char *lv,
                                                const unsigned char *kt, const unsigned char *vt,
                                                int hkv, int h, const int8_t *anc, int depth,
                                                int64_t tb, int64_t L) {
  using C = AttnCfg<BF, D>;
  const int k0 = static_cast<int>(L > tb ? L - tb : 0);  // first key slot at or past L
  const int nk = kTile - k0;
  const int tid = threadIdx.x;
  // keys: 16-byte chunks
  for (int c = tid; c < nk * C::CPR; c += kAttnThreads) {
    const int key = k0 + c / C::CPR, cc = c % C::CPR;
    const int64_t d = tb + key - L;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (d <= depth)
      x = *reinterpret_cast<const uint4 *>(
          kt + (static_cast<int64_t>(anc[d]) * hkv + h) * C::ROWB + cc * 16);
    if constexpr (BF) {
      *reinterpret_cast<uint4 *>(lk + key * C::ROWB + ((cc ^ (key & C::KSW)) * 16)) = x;
    } else {
      float *dst = reinterpret_cast<float *>(lk) + key * (D + 1) + cc * 4;
      dst[0] = __uint_as_float(x.x);
      dst[1] = __uint_as_float(x.y);
      dst[2] = __uint_as_float(x.z);
      dst[3] = __uint_as_float(x.w);
    }
  }
  // values
  if constexpr (BF) {
    for (int c = tid; c < nk * D; c += kAttnThreads) {
      const int key = k0 + c / D, dd = c % D;
      const int64_t d = tb + key - L;
      uint16_t x = 0;
      if (d <= depth)
        x = reinterpret_cast<const uint16_t *>(vt)[(static_cast<int64_t>(anc[d]) * hkv + h) * D + dd];
      reinterpret_cast<uint16_t *>(lv)[dd * 64 + (((key >> 2) ^ (dd & 15)) * 4) + (key & 3)] = x;
    }
  } else {
    for (int c = tid; c < nk * C::CPR; c += kAttnThreads) {
      const int key = k0 + c / C::CPR, cc = c % C::CPR;
      const int64_t d = tb + key - L;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (d <= depth)
        x = *reinterpret_cast<const uint4 *>(
            vt + (static_cast<int64_t>(anc[d]) * hkv + h) * C::ROWB + cc * 16);
      *reinterpret_cast<uint4 *>(lv + key * C::ROWB + cc * 16) = x;
    }
  }
}

// Q operand of one wave: lane (g, n) holds row n; rows past `rows` are zero.
template <bool BF, int D>
struct QRegs {
  using C = AttnCfg<BF, D>;
  typename std::conditional<BF, bf16x8, float>::type q[C::KQ];
  // row_ptr: start of row n's D elements (nullptr for a padding row)
  __device__ __forceinline__ void load(const void *row_ptr) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kk = 0; kk < C::KQ; ++kk) {
      if constexpr (BF) {
        if (row_ptr)
          q[kk] = *reinterpret_cast<const bf16x8 *>(static_cast<const uint16_t *>(row_ptr) +
                                                    32 * kk + 8 * g);
        else
          q[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
      } else {
        q[kk] = row_ptr ? static_cast<const float *>(row_ptr)[4 * kk + g] : 0.0f;
      }
    }
  }
};

template <int D>
__device__ __forceinline__ void write_partial(const RowState<D> &st, float *acc_row, float *ml_row) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    *reinterpret_cast<floatx4 *>(acc_row + 16 * db + 4 * g) = st.acc[db];
  if (g == 0) {
    ml_row[0] = st.m;
    ml_row[1] = st.l;
  }
}

// Shared item: kv head h, committed split s, row group rg; every (node, q head)
// row of the group sees every key of the split.
template <bool BF, int D>
__device__ __forceinline__ void attn_shared_item(const AttnLaunch &P, const AttnTree &T, int it,
                                              unsigned char *lk, unsigned char *lv) {
  using C = AttnCfg<BF, D>;
  const int G = P.hq / P.hkv;
  const int M = T.n * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15;
  const int split_tiles = T.split / kTile;
  const int rg = it % T.row_groups;
  const int rest = it / T.row_groups;
  const int s = rest % T.n_shared;
  const int h = rest / T.n_shared;
  const int r = (rg * kAttnWaves + wave) * 16 + ln;  // this lane's row
  const bool wave_on = (rg * kAttnWaves + wave) * 16 < M;
  RowState<D> st;
  QRegs<BF, D> qr;
  TileStage<BF, D> stage;
  const void *qrow = nullptr;
  if (r < M) {
    const int node = r / G, j = h * G + r % G;
    qrow = static_cast<const unsigned char *>(T.q) +
           (static_cast<int64_t>(node) * P.hq + j) * C::ROWB;
  }
  qr.load(qrow);
  st.reset();
  const unsigned char *kh = static_cast<const unsigned char *>(T.kc) +
                            static_cast<int64_t>(h) * T.cap * C::ROWB;
  const unsigned char *vh = static_cast<const unsigned char *>(T.vc) +
                            static_cast<int64_t>(h) * T.cap * C::ROWB;
  const int64_t t0 = static_cast<int64_t>(s) * split_tiles;
  stage.load(kh, vh, t0 * kTile, T.L);
  for (int tt = 0; tt < split_tiles; ++tt) {
    __syncthreads();
    stage.store(lk, lv);
    __syncthreads();
    if (tt + 1 < split_tiles) stage.load(kh, vh, (t0 + tt + 1) * kTile, T.L);
    if (wave_on) attn_tile<BF, D, false>(st, qr.q, lk, lv, (t0 + tt) * kTile, 0, P.c2);
  }
  if (r < M) {
    const int64_t prow = (static_cast<int64_t>(h) * T.nsplit_cap + s) * T.rows_cap + r;
    write_partial<D>(st, T.part_acc + prow * D, T.part_ml + prow * 2);
  }
}

// Tail item: kv head h, nodes ng*8 .. ng*8+7 (one per wave); every position from
// the first split not wholly below L up to each node's own position.  Tiles wholly
// below L are shared by the group's waves; a tile holding positions >= L is rebuilt
// in LDS for one node at a time (its ancestors, zeros past its position) and run
// by that node's wave alone.
template <bool BF, int D>
__device__ __forceinline__ void attn_tail_item(const AttnLaunch &P, const AttnTree &T, int item,
                                               unsigned char *a_lds) {
  using C = AttnCfg<BF, D>;
  unsigned char *lk = a_lds;
  unsigned char *lv = a_lds + C::K_BYTES;
  const int G = P.hq / P.hkv;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15;
  const int split_tiles = T.split / kTile;
  const int ngroups = (T.n + kAttnWaves - 1) / kAttnWaves;
  const int h = item / ngroups, ng = item % ngroups;
  const int node = ng * kAttnWaves + wave;
  const bool node_on = node < T.n;
  int8_t *anc_all = reinterpret_cast<int8_t *>(a_lds + C::TILE_BYTES);
  const unsigned char *kt = static_cast<const unsigned char *>(T.kt);
  const unsigned char *vt = static_cast<const unsigned char *>(T.vt);

  // Group 0 stages the tree rows into the cache's pending rows [L, L+n), in
  // tree-index order (commit gathers the accepted ones from there).
  if (ng == 0) {
    unsigned char *kcd = static_cast<unsigned char *>(T.kc) +
                         (static_cast<int64_t>(h) * T.cap + T.L) * C::ROWB;
    unsigned char *vcd = static_cast<unsigned char *>(T.vc) +
                         (static_cast<int64_t>(h) * T.cap + T.L) * C::ROWB;
    for (int c = tid; c < T.n * C::CPR; c += kAttnThreads) {
      const int i = c / C::CPR, cc = c % C::CPR;
      const int64_t src = (static_cast<int64_t>(i) * P.hkv + h) * C::ROWB + cc * 16;
      *reinterpret_cast<uint4 *>(kcd + static_cast<int64_t>(i) * C::ROWB + cc * 16) =
          *reinterpret_cast<const uint4 *>(kt + src);
      *reinterpret_cast<uint4 *>(vcd + static_cast<int64_t>(i) * C::ROWB + cc * 16) =
          *reinterpret_cast<const uint4 *>(vt + src);
    }
  }
  // Ancestor table of every node of the group, by depth (parents walked in LDS).
  int8_t *par_l = anc_all + kAttnWaves * kMaxNodes;
  if (tid < T.n) par_l[tid] = T.parent[tid];
  __syncthreads();
  if (tid < kAttnWaves) {
    const int x0 = ng * kAttnWaves + tid;
    if (x0 < T.n) {
      int x = x0;
      for (int d = T.depth[x0]; d >= 0; --d) {
        anc_all[tid * kMaxNodes + d] = static_cast<int8_t>(x);
        x = par_l[x];
      }
    }
  }
  int64_t pos_max = 0;
  for (int w = 0; w < kAttnWaves; ++w) {
    const int x = ng * kAttnWaves + w;
    if (x < T.n) pos_max = max(pos_max, T.L + static_cast<int64_t>(T.depth[x]));
  }
  const int64_t pos = node_on ? T.L + T.depth[node] : 0;
  RowState<D> st;
  QRegs<BF, D> qr;
  TileStage<BF, D> stage;
  const void *qrow = nullptr;
  if (node_on && ln < G)
    qrow = static_cast<const unsigned char *>(T.q) +
           (static_cast<int64_t>(node) * P.hq + h * G + ln) * C::ROWB;
  qr.load(qrow);
  st.reset();

  const unsigned char *kh = static_cast<const unsigned char *>(T.kc) +
                            static_cast<int64_t>(h) * T.cap * C::ROWB;
  const unsigned char *vh = static_cast<const unsigned char *>(T.vc) +
                            static_cast<int64_t>(h) * T.cap * C::ROWB;
  const int64_t t_first = static_cast<int64_t>(T.n_shared) * split_tiles;
  const int64_t t_last = pos_max / kTile;
  const int64_t my_last = pos / kTile;
  stage.load(kh, vh, t_first * kTile, T.L);
  for (int64_t tt = t_first; tt <= t_last; ++tt) {
    const int64_t tb = tt * kTile;
    __syncthreads();
    stage.store(lk, lv);
    __syncthreads();
    if (tt + 1 <= t_last) stage.load(kh, vh, (tt + 1) * kTile, T.L);
    if (tb + kTile <= T.L) {
      if (node_on && tt <= my_last) attn_tile<BF, D, false>(st, qr.q, lk, lv, tb, 0, P.c2);
    } else {
      for (int w = 0; w < kAttnWaves; ++w) {
        const int x = ng * kAttnWaves + w;
        if (x >= T.n || tt > (T.L + T.depth[x]) / kTile) continue;  // uniform over the group
        build_node_rows<BF, D>(lk, lv, kt, vt, P.hkv, h, anc_all + w * kMaxNodes, T.depth[x],
                               tb, T.L);
        __syncthreads();
        if (wave == w) attn_tile<BF, D, true>(st, qr.q, lk, lv, tb, pos, P.c2);
        __syncthreads();
      }
    }
    if (node_on && tt <= my_last) {
      const bool split_end = ((tt + 1) % split_tiles) == 0;
      if (split_end || tt == my_last) {
        if (ln < G) {
          const int s = static_cast<int>(tt / split_tiles);
          const int64_t prow =
              (static_cast<int64_t>(h) * T.nsplit_cap + s) * T.rows_cap + node * G + ln;
          write_partial<D>(st, T.part_acc + prow * D, T.part_ml + prow * 2);
        }
        st.reset();
      }
    }
  }
}

template <bool BF, int D>
__global__ __launch_bounds__(kAttnThreads) void attn_split_kernel(const AttnLaunch P) {
  using C = AttnCfg<BF, D>;
  extern __shared__ __align__(16) unsigned char a_lds[];
  const int bid = blockIdx.x;
  int t = 0;
  while (t + 1 < P.n_trees && bid >= P.t[t + 1].item_begin) ++t;
  const AttnTree &T = P.t[t];
  const int item = bid - T.item_begin;
  if (item >= T.n_tail_items)
    attn_shared_item<BF, D>(P, T, item - T.n_tail_items, a_lds, a_lds + C::K_BYTES);
  else
    attn_tail_item<BF, D>(P, T, item, a_lds);
}

// Fold the split partials of one (node, q head) row.  The row's S splits are cut
// into kFoldWaves contiguous ranges; each wave folds its range in ascending order
// (kFoldBatch loads in flight), then the range results are folded in ascending
// order.  The structure depends only on S, i.e. on the row's position.
constexpr int kFoldWaves = kFoldThreads / 64;
constexpr int kFoldBatch = 8;

struct FoldAcc {
  float m, l;
  __device__ __forceinline__ void add(float ms, float ls, float *acc, const float *x, int E) {
    const float mn = fmaxf(m, ms);
    const float a = exp2_fast(m - mn), b = exp2_fast(ms - mn);
    l = l * a + ls * b;
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * a + x[e] * b;
    m = mn;
  }
};

template <bool BF, int D>
__global__ __launch_bounds__(kFoldThreads) void attn_fold_kernel(const FoldLaunch P) {
  constexpr int E = D / 64;  // elements per lane
  __shared__ float w_ml[kFoldWaves][2];
  __shared__ __align__(16) float w_acc[kFoldWaves][D];
  const int bid = blockIdx.x;
  int t = 0;
  while (t + 1 < P.n_trees && bid >= P.t[t + 1].row_begin) ++t;
  const FoldTree &T = P.t[t];
  const int local = bid - T.row_begin;
  const int node = local / P.hq, j = local % P.hq;
  const int G = P.hq / P.hkv, h = j / G;
  const int r = node * G + (j - h * G);
  const int64_t pos = T.L + T.depth[node];
  const int S = static_cast<int>(pos / T.split) + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per = (S + kFoldWaves - 1) / kFoldWaves;
  const int lo = min(S, wave * per), hi = min(S, lo + per);
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  FoldAcc f{-INFINITY, 0.0f};
  const int64_t row0 = static_cast<int64_t>(h) * T.nsplit_cap * T.rows_cap + r;
  for (int s0 = lo; s0 < hi; s0 += kFoldBatch) {
    float ms[kFoldBatch], ls[kFoldBatch], x[kFoldBatch][E];
#pragma unroll
    for (int b = 0; b < kFoldBatch; ++b) {
      if (s0 + b < hi) {
        const int64_t prow = row0 + static_cast<int64_t>(s0 + b) * T.rows_cap;
        ms[b] = T.part_ml[prow * 2];
        ls[b] = T.part_ml[prow * 2 + 1];
        const float *pa = T.part_acc + prow * D + lane * E;
        if constexpr (E == 4) {
          const float4 v = *reinterpret_cast<const float4 *>(pa);
          x[b][0] = v.x;
          x[b][1] = v.y;
          x[b][2] = v.z;
          x[b][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) x[b][e] = pa[e];
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kFoldBatch; ++b)
      if (s0 + b < hi) f.add(ms[b], ls[b], acc, x[b], E);
  }
  if (lane == 0) {
    w_ml[wave][0] = f.m;
    w_ml[wave][1] = f.l;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) w_acc[wave][lane * E + e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
  float out[E];
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = 0.0f;
  FoldAcc tot{-INFINITY, 0.0f};
  for (int w = 0; w < kFoldWaves; ++w) {
    const int lw = min(S, w * per);
    if (lw >= min(S, lw + per)) continue;  // empty range
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = w_acc[w][lane * E + e];
    tot.add(w_ml[w][0], w_ml[w][1], out, x, E);
  }
  const int64_t o0 = (static_cast<int64_t>(node) * P.hq + j) * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) st_io<BF>(T.o, o0 + e, out[e] / tot.l);
}

// ============================================================================ commit

// The accepted path: from the launch block, or (after the accept walk) from the
// walk's output in device memory, {m, bonus token, path[m]}.
// A device path is read in one round trip: m by every lane, and lane j's copy of
// path[j] (j < the tree's node count, P.m); entry d is then read from lane d.
struct CommitPath {
  const int8_t *host;
  int m;
  int pv;
  bool dev;
  // d is uniform over the wave
  __device__ __forceinline__ int operator[](int d) const {
    return dev ? __builtin_amdgcn_readlane(pv, d) : host[d];
  }
};

__device__ __forceinline__ CommitPath load_path(const CommitLaunch &P, int lane) {
  if (!P.dev_out) return CommitPath{P.path, P.m, 0, false};
  const int mv = P.dev_out[0];
  const int pv = P.dev_out[2 + min(lane, P.m - 1)];
  return CommitPath{P.path, __builtin_amdgcn_readfirstlane(mv), pv, true};
}

template <bool BF, int DK>
__global__ __launch_bounds__(kGdnThreads) void commit_kernel(const CommitLaunch P) {
  constexpr int R = DK / 16;
  constexpr int ESZ = BF ? 2 : 4;
  constexpr int KW = R * ESZ / 4;    // 32-bit words of a lane's k slice (2, 4 or 8)
  constexpr int B = 4;               // path steps whose operands are in flight together
  const int bid = blockIdx.x, tid = threadIdx.x;
  if (bid < P.gdn_blocks) {
    // Committed state of one (GDN layer, value head, NC groups of 16 columns): replay
    // the accepted path's rank-1 steps fmaf(k, u, alpha * S) with the bits the pass
    // used, so the result equals the pass's state of the path's last node.  A lane
    // holds the same 8 key rows of NC columns 16 apart, which share its k and alpha
    // loads, so every lane keeps NC state slices in flight.
    constexpr int NC = kCommitCols;
    const int cgroups = P.dv / (kGdnCols * NC);
    const int per_layer = P.hv * cgroups;
    const int lg = bid / per_layer, local = bid % per_layer;
    const int h = local / cgroups, cg = local % cgroups;
    const int qh = h / (P.hv / P.hk);
    const int wave = tid >> 6, lane = tid & 63;
    const int col0 = cg * kGdnCols * NC + wave * 4 + (lane >> 4);
    const int g = lane & 15;
    float *sp0 = P.state + ((static_cast<int64_t>(lg) * P.hv + h) * P.dv + col0) * DK + g * R;
    float cur[NC][R];
#pragma unroll
    for (int j = 0; j < NC; ++j) lds_row<R>(sp0 + j * kGdnCols * DK, cur[j]);  // in flight first
    const CommitPath path = load_path(P, lane);
    const int64_t lbase = static_cast<int64_t>(lg) * P.max_nodes;
    for (int d0 = 0; d0 < path.m; d0 += B) {
      uint32_t kw[B][KW];
      float u[B][NC];
      io_t<BF> araw[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (d0 + b < path.m) {
          const int64_t nb = lbase + path[d0 + b];
          const unsigned char *kp = static_cast<const unsigned char *>(P.k_pend) +
                                    ((nb * P.hk + qh) * DK + g * R) * ESZ;
          if constexpr (KW % 4 == 0) {
#pragma unroll
            for (int c = 0; c < KW; c += 4) {
              const uint4 x = *reinterpret_cast<const uint4 *>(kp + 4 * c);
              kw[b][c] = x.x;
              kw[b][c + 1] = x.y;
              kw[b][c + 2] = x.z;
              kw[b][c + 3] = x.w;
            }
          } else {
            const uint2 x = *reinterpret_cast<const uint2 *>(kp);
            kw[b][0] = x.x;
            kw[b][1] = x.y;
          }
#pragma unroll
          for (int j = 0; j < NC; ++j) u[b][j] = P.u_pend[(nb * P.hv + h) * P.dv + col0 + j * kGdnCols];
          araw[b] = static_cast<const io_t<BF> *>(P.a_pend)[nb * P.hv + h];
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        if (d0 + b < path.m) {
          float kj[R];
#pragma unroll
          for (int a = 0; a < R; ++a) {
            if constexpr (BF)
              kj[a] = __uint_as_float((a & 1) ? (kw[b][a / 2] & 0xFFFF0000u) : (kw[b][a / 2] << 16));
            else
              kj[a] = __uint_as_float(kw[b][a]);
          }
          float al;
          if constexpr (BF)
            al = __uint_as_float(static_cast<uint32_t>(araw[b]) << 16);
          else
            al = araw[b];
#pragma unroll
          for (int j = 0; j < NC; ++j)
#pragma unroll
            for (int a = 0; a < R; ++a) cur[j][a] = fmaf(kj[a], u[b][j], al * cur[j][a]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
      for (int a = 0; a < R; a += 4)
        *reinterpret_cast<float4 *>(sp0 + j * kGdnCols * DK + a) =
            make_float4(cur[j][a], cur[j][a + 1], cur[j][a + 2], cur[j][a + 3]);
    return;
  }
  if (bid >= P.gdn_blocks + P.kv_blocks) {
    // Conv tail of one GDN layer, 16 bytes of channels per thread: the new tail is
    // the last width-1 rows of (old tail, the path's pre-conv rows), bit copies.
    // A thread reads every source of its channels before it writes any row.
    const CommitPath path = load_path(P, tid & 63);  // every lane, before any returns
    const int cb = bid - P.gdn_blocks - P.kv_blocks;
    const int lg = cb / P.conv_blocks_per_layer;
    const int64_t row_bytes = static_cast<int64_t>(P.conv_C) * (BF ? 2 : 4);
    const int64_t byte = (static_cast<int64_t>(cb % P.conv_blocks_per_layer) * kGdnThreads + tid) * 16;
    if (byte >= row_bytes) return;
    const int keep = P.conv_width - 1;
    unsigned char *tail = static_cast<unsigned char *>(P.conv_state) + lg * keep * row_bytes + byte;
    const unsigned char *xp = static_cast<const unsigned char *>(P.x_pend) +
                              static_cast<int64_t>(lg) * P.max_nodes * row_bytes + byte;
    static_assert(kConvMaxWidth - 1 == 3, "three tail rows at most");
    auto source = [&](int r) {  // row r of the new tail: (old tail rows, path rows)[m + r]
      const int src = path.m + r;
      return src < keep ? *reinterpret_cast<const uint4 *>(tail + src * row_bytes)
                        : *reinterpret_cast<const uint4 *>(xp + static_cast<int64_t>(path[src - keep]) * row_bytes);
    };
    const uint4 r0 = source(0);
    const uint4 r1 = keep > 1 ? source(1) : r0;
    const uint4 r2 = keep > 2 ? source(2) : r0;
    *reinterpret_cast<uint4 *>(tail) = r0;
    if (keep > 1) *reinterpret_cast<uint4 *>(tail + row_bytes) = r1;
    if (keep > 2) *reinterpret_cast<uint4 *>(tail + 2 * row_bytes) = r2;
    return;
  }
  // K/V gather: row L+d <- row L+path[d] of one (attention layer, kv head).
  // Rows are staged through LDS because a destination row may be another
  // destination's source.
  extern __shared__ __align__(16) uint4 c_lds[];
  __shared__ int path_s[kMaxNodes];  // the path, for lanes that index it per lane
  const CommitPath path = load_path(P, tid & 63);
  if (tid < kMaxNodes) path_s[tid] = tid < path.m ? (path.dev ? path.pv : P.path[tid]) : 0;
  __syncthreads();
  const int kb = bid - P.gdn_blocks;
  const int la = kb / P.hkv, hh = kb % P.hkv;
  const int esz = BF ? 2 : 4;
  const int cpr = P.D * esz / 16;
  for (int which = 0; which < 2; ++which) {
    unsigned char *base = static_cast<unsigned char *>(which == 0 ? P.kc : P.vc) +
                          ((static_cast<int64_t>(la) * P.hkv + hh) * P.cap + P.L) * P.D * esz;
    for (int c = tid; c < path.m * cpr; c += kGdnThreads) {
      const int d = c / cpr, cc = c % cpr;
      c_lds[c] = *reinterpret_cast<const uint4 *>(base + static_cast<int64_t>(path_s[d]) * P.D * esz +
                                                  cc * 16);
    }
    __syncthreads();
    for (int c = tid; c < path.m * cpr; c += kGdnThreads) {
      const int d = c / cpr, cc = c % cpr;
      *reinterpret_cast<uint4 *>(base + static_cast<int64_t>(d) * P.D * esz + cc * 16) = c_lds[c];
    }
    __syncthreads();
  }
}

// ============================================================================ accept walk

// One wave: lane i is node i.  Node i > 0 agrees when draft[i] equals the model's own
// token after its parent and every ancestor agrees (its ancestor mask holds no
// disagreeing node).  The deepest agreeing node, the lowest index among equals,
// ends the path; its ancestors-or-self in index order are the path (parents have
// lower indices); the bonus token is the model's own token after it.
__global__ __launch_bounds__(64) void walk_kernel(const WalkLaunch W) {
  const int lane = threadIdx.x;
  const bool real = lane < W.n;
  const int me = real ? lane : 0;
  const uint64_t anc = W.anc[me];
  const int par = lane > 0 && real ? 63 - __builtin_clzll(anc & ~(1ull << lane)) : 0;
  const bool match = real && (lane == 0 || W.draft[lane] == W.target[par]);
  const uint64_t ok = __ballot(match);
  const bool agrees = real && (anc & ~ok) == 0;
  const int depth = __popcll(anc) - 1;
  int key = agrees ? depth * 64 + (63 - lane) : -1;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) key = max(key, __shfl_xor(key, m));
  const int x = 63 - (key & 63);  // key >= 0: the root always agrees
  const uint64_t path = W.anc[x];
  const int m = __popcll(path);
  if (lane < 64 && ((path >> lane) & 1)) W.out[2 + __popcll(path & ((1ull << lane) - 1))] = lane;
  if (lane == 0) {
    W.out[0] = m;
    W.out[1] = W.target[x];
  }
}

// The header of a state snapshot, from the kernel arguments: eight 64-bit words.
__global__ __launch_bounds__(64) void snapshot_header_kernel(const SnapshotHeader H, uint64_t *dst) {
  const uint64_t w[8] = {H.magic, H.signature, static_cast<uint64_t>(H.length), static_cast<uint64_t>(H.state_bytes),
                         static_cast<uint64_t>(H.conv_bytes), 0, 0, 0};
  const int t = threadIdx.x;
  if (t < 8) dst[t] = w[t];
}

template <typename K>
hipError_t set_lds(K kernel, size_t bytes) {
  // Raised once per kernel to the largest dynamic LDS any launch asks for (the 160 KiB
  // of a workgroup less the kernel's static LDS), at the first launch: later launches,
  // graph capture included, then make no attribute call.
  static const hipError_t once = [kernel] {
    hipFuncAttributes attr{};
    hipError_t r = hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(kernel));
    if (r != hipSuccess) return r;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               kMaxDynamicLds - static_cast<int>(attr.sharedSizeBytes));
  }();
  (void)bytes;
  return once;
}

}  // namespace

size_t gdn_lds_bytes(int dk, int n_max, int n_saves, int anc) {
  return (gdn_lds_floats(dk, n_max) + static_cast<size_t>(n_saves) * kGdnCols * dk) * sizeof(float) +
         static_cast<size_t>(n_max) * (anc ? kMaxNodes + 1 : 1);
}

size_t attn_lds_bytes(int D, int bf16, int n_max) {
  (void)n_max;
  if (bf16) return 0;  // the kv_* kernels use static LDS only
  return AttnCfg<false, 64>::TILE_BYTES + kAttnWaves * kMaxNodes + kMaxNodes;
}

int attn_rows_per_item(int) { return kAttnWaves * 16; }
int attn_nodes_per_tail(int) { return kAttnWaves; }

size_t commit_lds_bytes(int D, int bf16, int m) {
  return static_cast<size_t>(m) * D * (bf16 ? 2 : 4);
}

hipError_t launch_gdn_tree(const GdnLaunch &a, int dk, int bf16, hipStream_t s, KernelEvents ev) {
  const dim3 blocks(a.hv * (a.dv / kGdnCols), a.n_trees);
  const size_t lds = gdn_lds_bytes(dk, a.n_max, a.n_saves, a.any_anc);
#define HDT_GDN(BF, DK)                                                                   \
  do {                                                                                    \
    (void)set_lds(gdn_tree_kernel<BF, DK>, lds);                                                \
    hipExtLaunchKernelGGL((gdn_tree_kernel<BF, DK>), blocks, dim3(gdn_threads(DK)), lds, s,  \
                          ev.start, ev.stop, 0, a);                                               \
  } while (0)
  if (bf16) {
    if (dk == 128) HDT_GDN(true, 128); else HDT_GDN(true, 64);
  } else {
    if (dk == 128) HDT_GDN(false, 128); else HDT_GDN(false, 64);
  }
#undef HDT_GDN
  return hipGetLastError();
}

hipError_t launch_attn_split(const AttnLaunch &a, int D, int bf16, int n_blocks, hipStream_t s,
                             KernelEvents ev) {
  if (bf16 || D != 64) return hipErrorInvalidValue;  // bf16 storage runs the kv_* kernels
  const size_t lds = attn_lds_bytes(D, bf16, a.n_max);
  (void)set_lds(attn_split_kernel<false, 64>, lds);
  hipExtLaunchKernelGGL((attn_split_kernel<false, 64>), dim3(n_blocks), dim3(kAttnThreads), lds, s,
                        ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_attn_fold(const FoldLaunch &a, int D, int bf16, int n_blocks, hipStream_t s,
                            KernelEvents ev) {
  if (bf16 || D != 64) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL((attn_fold_kernel<false, 64>), dim3(n_blocks), dim3(kFoldThreads), 0, s,
                        ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_walk(const WalkLaunch &a, hipStream_t s, KernelEvents ev) {
  hipExtLaunchKernelGGL(walk_kernel, dim3(1), dim3(64), 0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

// The scratch of hdt_forward_tree_noalloc: one file-scope device array, one copy on every
// device the library runs on.  In host code its name is a host-side stand-in, never a
// device address: only the address hipGetSymbolAddress returns on a device is passed to
// kernels or copies.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch_address(void **out) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void *addr[kDevices] = {};
  int dev = 0;
  hipError_t r = hipGetDevice(&dev);
  if (r != hipSuccess) return r;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // first use on this device, with it current
    void *p = nullptr;
    r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess) return r;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_snapshot_header(const SnapshotHeader &h, void *dst, hipStream_t s) {
  hipLaunchKernelGGL(snapshot_header_kernel, dim3(1), dim3(64), 0, s, h, static_cast<uint64_t *>(dst));
  return hipGetLastError();
}

hipError_t launch_commit(const CommitLaunch &a, int dk, int bf16, int n_blocks, hipStream_t s,
                         KernelEvents ev) {
  const size_t lds = commit_lds_bytes(a.D, bf16, a.m);
#define HDT_COMMIT(BF, DK)                                                                 \
  do {                                                                                     \
    (void)set_lds(commit_kernel<BF, DK>, lds);                                                   \
    hipExtLaunchKernelGGL((commit_kernel<BF, DK>), dim3(n_blocks), dim3(kGdnThreads), lds, s,     \
                          ev.start, ev.stop, 0, a);                                                \
  } while (0)
  if (bf16) {
    if (dk == 128) HDT_COMMIT(true, 128); else HDT_COMMIT(true, 64);
  } else {
    if (dk == 128) HDT_COMMIT(false, 128); else HDT_COMMIT(false, 64);
  }
#undef HDT_COMMIT
  return hipGetLastError();
}

}  // namespace hdt
