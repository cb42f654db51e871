// prefill.hip - the chunked prefill of a span of T tokens on the CDNA4 (gfx950)
// matrix cores.
//
// A prompt's tokens past the resident prefix go through the model once, in spans
// ("One request, end to end", 2.5 "The caches decide where the prefill starts";
// "How ignis serves a request", 3 "Prefill reads the prompt").  Unlike a tree verify,
// a span is one chain, so each layer can work on whole chunks of it at once:
//
//  GDN layers: the chunked (WY) form of the gated delta rule.  Within a chunk of C
//  tokens with cumulative decays g_i = a_1 ... a_i, the recurrence
//    S_i = a_i S_{i-1} + k_i u_i^T,  u_i = b_i (v_i - a_i S_{i-1}^T k_i),  o_i = S_i^T (s q_i)
//  unrolls to a unit lower-triangular system for the corrections u:
//    (I + A) U = diag(b) V - diag(b g) K S_0,   A_ij = b_i (g_i / g_j) k_i.k_j  (j < i),
//  so U = U~ - W S_0 with U~ = (I + A)^-1 diag(b) V and W = (I + A)^-1 diag(b g) K, and
//    O = diag(s g) Q S_0 + Mq U,   Mq_ij = s (g_i / g_j) q_i.k_j  (j <= i),
//    S_C = g_C S_0 + K^T diag(g_C / g) U.
//  gdn_wy_prep_kernel builds A, Mq, U~ and W for every (chunk, head) at once: they do
//  not depend on the state.  gdn_wy_scan_kernel then carries the state across the
//  chunks of a head, one 16-column slice of it per workgroup.  Decay ratios are taken
//  as 2^(G_i - G_j) of the base-2 log cumsum G, never as a quotient.
//
//  Attention layers: the span's K/V rows are copied into the cache first; each query
//  row (token t, q head j) then attends to cache rows 0 .. L + t, the causal limit.
//  attn_prefill_kernel streams 32-key tiles of K and V from HBM into an LDS ring
//  (buffer_load ... lds) for 128 query rows of one kv head, four waves of 32 rows, on
//  v_mfma_f32_32x32x16_bf16 with an online softmax in base 2.  Long contexts are cut
//  into key splits whose partials attn_prefill_fold_kernel merges.
//
// The chunked sums differ from the token-by-token recurrence in rounding only: a
// prefilled row matches the decode step's row to within the io precision, not bit
// for bit (the bit-exact prefill is hdt_forward_span's chain mode).
#include <cmath>

#include "common.h"

#pragma clang fp contract(off)

namespace hdt {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx4 mfma16(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x16, lane layout (gfx950): the A operand of lane l holds row l % 32, k = 8 (l / 32)
// + j; the B operand of lane l holds column l % 32, k = 8 (l / 32) + j; the result of lane
// l holds column l % 32 and, in register r, row 8 (r / 4) + 4 (l / 32) + r % 4.
__device__ __forceinline__ floatx16 mfma32(const bf16x8 &a, const bf16x8 &b, const floatx16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc *= c for an accumulator the matrix cores keep in AGPRs.  The value passes through
// a VGPR eight registers at a time inside one asm block, so the compiler keeps the
// accumulator where the MFMAs want it instead of copying all of it to VGPRs on every
// tile in case the (rare) rescale runs.  Each read, multiply and write is eight
// instructions from the one it depends on.
__device__ __forceinline__ void scale_agpr8(float &x0, float &x1, float &x2, float &x3, float &x4, float &x5,
                                            float &x6, float &x7, float c) {
  float t0, t1, t2, t3, t4, t5, t6, t7;
  asm volatile(
      "v_accvgpr_read_b32 %8, %0\n\tv_accvgpr_read_b32 %9, %1\n\t"
      "v_accvgpr_read_b32 %10, %2\n\tv_accvgpr_read_b32 %11, %3\n\t"
      "v_accvgpr_read_b32 %12, %4\n\tv_accvgpr_read_b32 %13, %5\n\t"
      "v_accvgpr_read_b32 %14, %6\n\tv_accvgpr_read_b32 %15, %7\n\t"
      "v_mul_f32 %8, %16, %8\n\tv_mul_f32 %9, %16, %9\n\t"
      "v_mul_f32 %10, %16, %10\n\tv_mul_f32 %11, %16, %11\n\t"
      "v_mul_f32 %12, %16, %12\n\tv_mul_f32 %13, %16, %13\n\t"
      "v_mul_f32 %14, %16, %14\n\tv_mul_f32 %15, %16, %15\n\t"
      "v_accvgpr_write_b32 %0, %8\n\tv_accvgpr_write_b32 %1, %9\n\t"
      "v_accvgpr_write_b32 %2, %10\n\tv_accvgpr_write_b32 %3, %11\n\t"
      "v_accvgpr_write_b32 %4, %12\n\tv_accvgpr_write_b32 %5, %13\n\t"
      "v_accvgpr_write_b32 %6, %14\n\tv_accvgpr_write_b32 %7, %15"
      : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "+a"(x4), "+a"(x5), "+a"(x6), "+a"(x7),
        "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(c));
}
__device__ __forceinline__ void scale_acc(floatx16 &a, float c) {
  float x[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = a[e];
  scale_agpr8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7], c);
  scale_agpr8(x[8], x[9], x[10], x[11], x[12], x[13], x[14], x[15], c);
#pragma unroll
  for (int e = 0; e < 16; ++e) a[e] = x[e];
}

// A float32 value as the sum of two bf16 values (hi = x rounded, lo = the rest rounded):
// products of two such pairs keep the three larger partial products, so a bf16 matrix
// core multiplies float32 operands to about 2^-16 relative.
__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  const __bf16 h = static_cast<__bf16>(x);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x - static_cast<float>(h)));
}

// Four float32 values as bf16 pairs (hi, lo), packed as MFMA operands.
__device__ __forceinline__ void split4(const floatx4 &x, shortx4 &hi, shortx4 &lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint16_t h, l;
    split_bf16(x[e], h, l);
    hi[e] = static_cast<short>(h);
    lo[e] = static_cast<short>(l);
  }
}

// 16x16x16: the A operand of lane l holds row l % 16, k = 4 (l / 16) + e; the B operand
// column l % 16, k = 4 (l / 16) + e; the result rows 4 (l / 16) + r of column l % 16.
__device__ __forceinline__ floatx4 mfma16k16(const shortx4 &a, const shortx4 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ float bf(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// ============================================================================ GDN prep
//
// One workgroup per (chunk, v head), four waves.  Rows past the chunk's tokens are
// zero (k = q = v = 0, b = 0, a = 1): they leave U~, W and every sum unchanged.

template <int DK, int DV>
struct WyPrepLds {
  static constexpr int KP = DK + 8;  // padded rows: 16 consecutive rows hit distinct banks
  static constexpr int VP = DV + 8;
  uint16_t k[kWyChunk][KP];
  uint16_t q[kWyChunk][KP];
  uint16_t v[kWyChunk][VP];
  float a[kWyChunk][kWyChunk + 4];  // A_ij (j < i), zero elsewhere
  float t[4][16][20];               // inverses of the four diagonal blocks of I + A
  float G[kWyChunk];                // base-2 log of the cumulative decay
  float b[kWyChunk];
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void gdn_wy_prep_kernel(const WyPrep P) {
  static_assert(DK + DV == 256, "one substitution column per thread");
  constexpr int C = kWyChunk;
  __shared__ __align__(16) WyPrepLds<DK, DV> sm;
  const int ch = blockIdx.x, h = blockIdx.y;
  const int ratio = P.hv / P.hk, gk = h / ratio;
  const int t0 = max(0, C * ch - P.off), t1 = min(P.T, C * (ch + 1) - P.off), n = t1 - t0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // ---- gates and the log-decay cumsum (wave 0; an inclusive scan over the lanes)
  if (wave == 0) {
    const int i = lane;
    float lg = 0.0f, be = 0.0f;
    if (i < n) {
      const int64_t gi = static_cast<int64_t>(t0 + i) * P.hv + h;
      lg = log2f(ld_io<true>(P.alpha, gi));
      be = ld_io<true>(P.beta, gi);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(lg, d, 64);
      if (lane >= d) lg += o;
    }
    sm.G[i] = lg;
    sm.b[i] = be;
  }
  // ---- K, Q (q/k head gk) and V (v head h) rows into LDS, zero past the chunk
  {
    constexpr int KC = DK / 8, VC = DV / 8;  // 16-byte chunks per row
    const unsigned char *kb = static_cast<const unsigned char *>(P.k);
    const unsigned char *qb = static_cast<const unsigned char *>(P.q);
    const unsigned char *vb = static_cast<const unsigned char *>(P.v);
    for (int x = tid; x < C * KC; x += 256) {
      const int i = x / KC, c = x % KC;
      uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
      if (i < n) {
        const int64_t off = ((static_cast<int64_t>(t0 + i) * P.hk + gk) * DK + 8 * c) * 2;
        kv = *reinterpret_cast<const uint4 *>(kb + off);
        qv = *reinterpret_cast<const uint4 *>(qb + off);
      }
      *reinterpret_cast<uint4 *>(&sm.k[i][8 * c]) = kv;
      *reinterpret_cast<uint4 *>(&sm.q[i][8 * c]) = qv;
    }
    for (int x = tid; x < C * VC; x += 256) {
      const int i = x / VC, c = x % VC;
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (i < n) vv = *reinterpret_cast<const uint4 *>(vb + ((static_cast<int64_t>(t0 + i) * P.hv + h) * DV + 8 * c) * 2);
      *reinterpret_cast<uint4 *>(&sm.v[i][8 * c]) = vv;
    }
  }
  __syncthreads();

  // ---- Gram matrices K K^T and Q K^T on the matrix cores: wave w takes rows
  // [16 w, 16 w + 16) and all four 16-column blocks.  A lane's result register r is
  // row 16 w + 4 (l / 16) + r, column 16 cb + l % 16.
  const int ln = lane & 15, qd = lane >> 4;
  {
    floatx4 kk[4], qk[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) kk[cb] = qk[cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DK / 32; ++s) {
      const bf16x8 ak = ld8(&sm.k[16 * wave + ln][32 * s + 8 * qd]);
      const bf16x8 aq = ld8(&sm.q[16 * wave + ln][32 * s + 8 * qd]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const bf16x8 bk = ld8(&sm.k[16 * cb + ln][32 * s + 8 * qd]);
        kk[cb] = mfma16(ak, bk, kk[cb]);
        qk[cb] = mfma16(aq, bk, qk[cb]);
      }
    }
    const size_t mq0 = (static_cast<size_t>(ch) * P.hv + h) * C * C;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int j = 16 * cb + ln;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * wave + 4 * qd + r;
        const float dec = j <= i ? exp2f(sm.G[i] - sm.G[j]) : 0.0f;
        sm.a[i][j] = j < i ? sm.b[i] * dec * kk[cb][r] : 0.0f;
        uint16_t hi, lo;
        split_bf16(j <= i ? P.scale * dec * qk[cb][r] : 0.0f, hi, lo);
        P.mq_hi[mq0 + i * C + j] = hi;
        P.mq_lo[mq0 + i * C + j] = lo;
      }
    }
  }
  __syncthreads();

  // ---- (I + A) X = B by blocks of 16 rows.  The diagonal blocks' inverses
  // T_k = (I + A_kk)^-1 come first (wave 0, one column of one block per lane, plain
  // substitution); then, for row blocks k = 0..3 in turn,
  //   X_k = T_k (B_k - sum_{j < k} A_kj X_j)
  // on the matrix cores with float32 operands split into bf16 pairs.  The right-hand
  // sides are diag(b) V (columns [0, DV), giving U~) and diag(b g) K (columns
  // [DV, DV + DK), giving W); wave w takes columns [64 w, 64 w + 64), four blocks of
  // 16.  The 16x16x16 result layout (lane l: rows 4 (l / 16) + r, column l % 16) is
  // also its B operand layout, so a solved block feeds the next products directly.
  if (wave == 0) {
    const int kb = lane >> 4, c = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == c ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < i; ++j) acc = acc - sm.a[16 * kb + i][16 * kb + j] * x[j];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.t[kb][i][c] = x[i];
  }
  __syncthreads();
  {
    floatx4 X[4][4];  // [row block][column block]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // A_kj and T_k as A operands: row 16 k + l % 16, columns 4 (l / 16) .. + 3
      shortx4 ah[4], al[4], th, tl;
#pragma unroll
      for (int j = 0; j < k; ++j) split4(*reinterpret_cast<const floatx4 *>(&sm.a[16 * k + ln][16 * j + 4 * qd]), ah[j], al[j]);
      split4(*reinterpret_cast<const floatx4 *>(&sm.t[k][ln][4 * qd]), th, tl);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int c = 64 * wave + 16 * cb + ln;  // this lane's right-hand column
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < k; ++j) {
          shortx4 xh, xl;
          split4(X[j][cb], xh, xl);
          acc = mfma16k16(ah[j], xh, acc);
          acc = mfma16k16(ah[j], xl, acc);
          acc = mfma16k16(al[j], xh, acc);
        }
        floatx4 rr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * k + 4 * qd + r;
          const float bi = c < DV ? bf(sm.v[i][c]) : exp2f(sm.G[i]) * bf(sm.k[i][c - DV]);
          rr[r] = sm.b[i] * bi - acc[r];
        }
        shortx4 rh, rl;
        split4(rr, rh, rl);
        floatx4 xk = floatx4{0.f, 0.f, 0.f, 0.f};
        xk = mfma16k16(th, rh, xk);
        xk = mfma16k16(th, rl, xk);
        xk = mfma16k16(tl, rh, xk);
        X[k][cb] = xk;
      }
    }
    const size_t blk = static_cast<size_t>(ch) * P.hv + h;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int c = 64 * wave + 16 * cb + ln;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * k + 4 * qd + r;
          if (c < DV) {
            P.ut[(blk * C + i) * DV + c] = X[k][cb][r];
          } else {
            uint16_t hi, lo;
            split_bf16(X[k][cb][r], hi, lo);
            P.w_hi[(blk * C + i) * DK + c - DV] = hi;
            P.w_lo[(blk * C + i) * DK + c - DV] = lo;
          }
        }
    }
  }
  // ---- decays, and (once per q/k head) Q and K^T of the chunk for the scan
  if (tid < C) {
    const int i = tid;
    float *g = P.g + (static_cast<size_t>(ch) * P.hv + h) * 3 * C;
    const float Gn = sm.G[n - 1];
    g[i] = P.scale * exp2f(sm.G[i]);
    g[C + i] = i < n ? exp2f(Gn - sm.G[i]) : 0.0f;
    if (i == 0) g[2 * C] = exp2f(Gn);
  }
  if (h % ratio == 0) {
    const size_t blk = static_cast<size_t>(ch) * P.hk + gk;
    uint16_t *qc = P.qc + blk * C * DK;
    for (int x = tid; x < C * DK / 8; x += 256) {
      const int i = x / (DK / 8), c = x % (DK / 8);
      *reinterpret_cast<uint4 *>(qc + i * DK + 8 * c) = *reinterpret_cast<const uint4 *>(&sm.q[i][8 * c]);
    }
    uint16_t *kt = P.kt + blk * DK * C;
    for (int x = tid; x < DK * C / 8; x += 256) {
      const int d = x / (C / 8), i0 = 8 * (x % (C / 8));
      uint16_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = sm.k[i0 + e][d];
      *reinterpret_cast<uint4 *>(kt + d * C + i0) = *reinterpret_cast<const uint4 *>(w);
    }
  }
}

// ============================================================================ GDN scan
//
// One workgroup per (v head, 16 value columns), four waves; the state slice S[:, c0 ..
// c0 + 16) lives in registers: wave w holds key dims [DK/4 w, DK/4 (w + 1)), lane l
// the column c0 + l % 16 and, in s[rb][r], dim DK/4 w + 16 rb + 4 (l / 16) + r (the
// result layout of the state update).  Per chunk:
//   U = U~ - W S           wave w: tokens [16 w, 16 w + 16)
//   O = diag(s g) Q S + Mq U
//   S = g_C S + K^T (diag(g_C / g) U)
// with S, U and diag(g_C / g) U passed between waves through LDS as bf16 pairs.

template <int DK>
struct WyOps {
  static constexpr int RB = DK / 64;
  bf16x8 wh[DK / 32], wl[DK / 32], q[DK / 32];  // A operands: rows 16 w + l % 16
  bf16x8 mh[2], ml[2];                          // Mq rows 16 w + l % 16, tokens 32 s + 8 (l / 16)
  bf16x8 kt[RB][2];                             // K^T rows (dims), tokens 32 s + 8 (l / 16)
  float ut[4], gq[4], gk[4], gC;
};

template <int DK, int DV>
__device__ __forceinline__ void wy_load(WyOps<DK> &o, const WyScan &P, int ch, int h, int gk, int c0) {
  constexpr int C = kWyChunk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  const size_t blk = static_cast<size_t>(ch) * P.hv + h, kblk = static_cast<size_t>(ch) * P.hk + gk;
  const int row = 16 * wave + ln;
#pragma unroll
  for (int s = 0; s < DK / 32; ++s) {
    o.wh[s] = ld8(P.w_hi + (blk * C + row) * DK + 32 * s + 8 * qd);
    o.wl[s] = ld8(P.w_lo + (blk * C + row) * DK + 32 * s + 8 * qd);
    o.q[s] = ld8(P.qc + (kblk * C + row) * DK + 32 * s + 8 * qd);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    o.mh[s] = ld8(P.mq_hi + (blk * C + row) * C + 32 * s + 8 * qd);
    o.ml[s] = ld8(P.mq_lo + (blk * C + row) * C + 32 * s + 8 * qd);
  }
#pragma unroll
  for (int rb = 0; rb < WyOps<DK>::RB; ++rb)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      o.kt[rb][s] = ld8(P.kt + (kblk * DK + DK / 4 * wave + 16 * rb + ln) * C + 32 * s + 8 * qd);
  const float *g = P.g + blk * 3 * C;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * wave + 4 * qd + r;
    o.ut[r] = P.ut[(blk * C + i) * DV + c0 + ln];
    o.gq[r] = g[i];
    o.gk[r] = g[C + i];
  }
  o.gC = g[2 * C];
}

template <int DK, int DV>
__global__ __launch_bounds__(256) void gdn_wy_scan_kernel(const WyScan P) {
  constexpr int C = kWyChunk;
  constexpr int RB = DK / 64;
  constexpr int SP = DK + 8, UP = C + 8;  // padded LDS rows
  __shared__ __align__(16) uint16_t s_hi[16][SP], s_lo[16][SP];
  __shared__ __align__(16) uint16_t u_hi[16][UP], u_lo[16][UP], w_hi[16][UP], w_lo[16][UP];
  const int h = blockIdx.x, c0 = 16 * blockIdx.y;
  const int gk = h / (P.hv / P.hk);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, ln = lane & 15, qd = lane >> 4;
  float *st = P.state + (static_cast<size_t>(h) * DV + c0 + ln) * DK;
  floatx4 s[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) s[rb] = *reinterpret_cast<const floatx4 *>(st + DK / 4 * wave + 16 * rb + 4 * qd);
  // one chunk with the operands `cur`; the next chunk's operands load into the other
  // set meanwhile (two sets used in turn: no register copy waits for a load)
  auto step = [&](const WyOps<DK> &cur, int ch) {
    const int t0 = max(0, C * ch - P.off), n = min(P.T, C * (ch + 1) - P.off) - t0;
    // ---- publish S as [column][dim] bf16 pairs
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint16_t hi[4], lo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) split_bf16(s[rb][r], hi[r], lo[r]);
      const int d = DK / 4 * wave + 16 * rb + 4 * qd;
      *reinterpret_cast<uint2 *>(&s_hi[ln][d]) = *reinterpret_cast<const uint2 *>(hi);
      *reinterpret_cast<uint2 *>(&s_lo[ln][d]) = *reinterpret_cast<const uint2 *>(lo);
    }
    lds_barrier();  // the next chunk's operand loads stay in flight
    // ---- W S and Q S for tokens [16 w, 16 w + 16)
    floatx4 ws = floatx4{0.f, 0.f, 0.f, 0.f}, qs = ws;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
      const bf16x8 bh = ld8(&s_hi[ln][32 * kk + 8 * qd]);
      const bf16x8 bl = ld8(&s_lo[ln][32 * kk + 8 * qd]);
      ws = mfma16(cur.wh[kk], bh, ws);
      ws = mfma16(cur.wh[kk], bl, ws);
      ws = mfma16(cur.wl[kk], bh, ws);
      qs = mfma16(cur.q[kk], bh, qs);
      qs = mfma16(cur.q[kk], bl, qs);
    }
    floatx4 o;
    {
      uint16_t uh[4], ul[4], vh[4], vl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = cur.ut[r] - ws[r];
        o[r] = cur.gq[r] * qs[r];
        split_bf16(u, uh[r], ul[r]);
        split_bf16(cur.gk[r] * u, vh[r], vl[r]);
      }
      const int t = 16 * wave + 4 * qd;
      *reinterpret_cast<uint2 *>(&u_hi[ln][t]) = *reinterpret_cast<const uint2 *>(uh);
      *reinterpret_cast<uint2 *>(&u_lo[ln][t]) = *reinterpret_cast<const uint2 *>(ul);
      *reinterpret_cast<uint2 *>(&w_hi[ln][t]) = *reinterpret_cast<const uint2 *>(vh);
      *reinterpret_cast<uint2 *>(&w_lo[ln][t]) = *reinterpret_cast<const uint2 *>(vl);
    }
    lds_barrier();  // the next chunk's operand loads stay in flight
    // ---- O += Mq U, written for the chunk's tokens
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 bh = ld8(&u_hi[ln][32 * kk + 8 * qd]);
      const bf16x8 bl = ld8(&u_lo[ln][32 * kk + 8 * qd]);
      o = mfma16(cur.mh[kk], bh, o);
      o = mfma16(cur.mh[kk], bl, o);
      o = mfma16(cur.ml[kk], bh, o);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * wave + 4 * qd + r;
      if (i < n)
        static_cast<uint16_t *>(P.o)[(static_cast<int64_t>(t0 + i) * P.hv + h) * DV + c0 + ln] = bf16_bits(o[r]);
    }
    // ---- S = g_C S + K^T (diag(g_C / g) U)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      floatx4 a = s[rb] * cur.gC;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 bh = ld8(&w_hi[ln][32 * kk + 8 * qd]);
        const bf16x8 bl = ld8(&w_lo[ln][32 * kk + 8 * qd]);
        a = mfma16(cur.kt[rb][kk], bh, a);
        a = mfma16(cur.kt[rb][kk], bl, a);
      }
      s[rb] = a;
    }
  };
  WyOps<DK> opa, opb;
  wy_load<DK, DV>(opa, P, 0, h, gk, c0);
  for (int ch = 0; ch < P.n_chunks; ch += 2) {
    if (ch + 1 < P.n_chunks) wy_load<DK, DV>(opb, P, ch + 1, h, gk, c0);
    step(opa, ch);
    if (ch + 1 >= P.n_chunks) break;
    if (ch + 2 < P.n_chunks) wy_load<DK, DV>(opa, P, ch + 2, h, gk, c0);
    step(opb, ch + 1);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) *reinterpret_cast<floatx4 *>(st + DK / 4 * wave + 16 * rb + 4 * qd) = s[rb];
}

// ============================================================================ attention

template <int D>
struct PfCfg {
  static constexpr int ROWB = D * 2;         // bytes per row
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  static constexpr int HALF = kKvTile * ROWB;
  static constexpr int TILE = 2 * HALF;      // K then V
  static constexpr int LOADS = TILE / 1024;  // wave-wide 16-byte-per-lane loads per tile
  static constexpr int RPL = 1024 / ROWB;    // rows per wave-wide load
  static constexpr int KQ = D / 16;          // k-steps of the score MFMA
  static constexpr int DB = D / 32;          // 32-column blocks of a row
  static_assert(D == 256 && kKvTile == 32, "tile shape");
};

// XOR swizzle of the 16-byte chunks of tile row `row`.  gfx950's LDS serves a
// ds_read_b128 32 lanes (512 bytes, every bank once) at a time, so a read is free of bank
// conflicts when its 32 lanes hit distinct 16-byte units modulo 32.  The score operand
// reads take 32 rows at one chunk, so the swizzle is a bijection of the 32 rows; a
// transposed value read takes rows 8 s .. 8 s + 7 at four consecutive chunks, so the low
// three row bits move the chunk's upper bits and the next two its lower ones.  The
// swizzle repeats every 32 rows: 16 rows further, chunk bit 1 flips.
__device__ __forceinline__ int pf_swz(int row) { return ((row & 7) << 2) | ((row >> 3) & 3); }
template <int D>
__device__ __forceinline__ int pf_off(int row, int c) {
  return row * PfCfg<D>::ROWB + ((c ^ pf_swz(row)) << 4);
}

// Online-softmax state of one 32-row block: lane l holds query row l % 32 (lanes l and
// l ^ 32 hold the same row and the same bits); acc[j][r] is output column 32 j +
// 8 (r / 4) + 4 (l / 32) + r % 4; q[kk] the row's d = 16 kk + 8 (l / 32) .. + 7.
template <int D>
struct PfRows {
  floatx16 acc[D / 32];
  float m, l;
  bf16x8 q[D / 16];
};

// Tile-invariant LDS offsets of this lane's operand reads: ko[kk] the score operand
// (key row l % 32, d chunk 2 kk + l / 32); vo[j][r] the transposed value reads of
// column block j for keys 4 h + e (r = 0) and 8 + 4 h + e (r = 1) of the first 16 keys
// (the second 16 sit 16 rows further, at the offset with bit 5 flipped: pf_swz).  In each 16-lane group lane p addresses row
// 4 h + p / 4 (+ 8 r) at columns 32 j + 16 ((l / 16) % 2) + 4 (p % 4), so the group's
// transposed read gives lane p column 32 j + 16 ((l / 16) % 2) + p of the four rows.
template <int D>
struct PfLane {
  uint32_t ko[D / 16];
  uint32_t vo[D / 32][2];
  __device__ __forceinline__ void init() {
    using C = PfCfg<D>;
    const int lane = threadIdx.x & 63, h = lane >> 5, p = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
    for (int kk = 0; kk < C::KQ; ++kk) ko[kk] = static_cast<uint32_t>(pf_off<D>(lane & 31, 2 * kk + h));
#pragma unroll
    for (int j = 0; j < C::DB; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = 8 * r + 4 * h + (p >> 2);
        const int byte = (32 * j + 16 * half + 4 * (p & 3)) * 2;
        vo[j][r] = static_cast<uint32_t>(C::HALF + row * C::ROWB + (((byte >> 4) ^ pf_swz(row)) << 4) + (byte & 15));
      }
  }
};

// Probabilities stay below 2^kPfLazy: the running max moves only when a tile's max
// exceeds it by more than this (base-2 units).
constexpr float kPfLazy = 8.0f;

// Scores S^T = K Q^T of one tile (its K half at `tile`) for this wave's 32 rows.
// Register r holds key 8 (r / 4) + 4 (l / 32) + r % 4 of the lane's row.  One
// accumulation chain: a dependent 32x32x16 MFMA issues about 8 cycles later than an
// independent one, and a second chain would hold 16 more registers.
template <int D>
__device__ __forceinline__ floatx16 pf_scores(const PfRows<D> &st, uint32_t tile, const PfLane<D> &ofs) {
  constexpr int KQ = PfCfg<D>::KQ;
  typedef __attribute__((address_space(3))) const bf16x8 *lds_b8;
  bf16x8 ka[KQ];
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) ka[kk] = *(lds_b8)(lds_ptr(tile + ofs.ko[kk]));
  floatx16 sc = floatx16{};
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) sc = mfma32(ka[kk], st.q[kk], sc);
  return sc;
}

// One step of the pipelined tile loop: the online softmax of tile t's scores `s`
// (keys from absolute position tb) and its value product (V half at `tv`), with the
// score MFMAs of tile t + 1 (K half at `tk`) interleaved into the softmax so that the
// matrix cores and the vector ALU work at once; returns tile t + 1's scores.  The
// probability operand of the value MFMA for keys 16 s .. 16 s + 15 is registers 8 s ..
// 8 s + 7, which the transposed value reads match key for key.  MASK: keys past the
// lane's `pos` get probability 0; a row with no key yet keeps m = -inf, l = 0, acc = 0.
template <int D, bool MASK>
__device__ __forceinline__ floatx16 pf_step(PfRows<D> &st, const floatx16 &s, uint32_t tk, uint32_t tv,
                                            const PfLane<D> &ofs, int64_t tb, int64_t pos, float c2) {
  using C = PfCfg<D>;
  constexpr int DB = C::DB;
  constexpr int KB16 = 16 * C::ROWB;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  bf16x8 va[DB][2];
#pragma unroll
  for (int j = 0; j < DB; ++j)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // the stage base is 32 KiB aligned, so flipping bit 5 of the sum flips it in the
      // offset; taken per tile, it costs no register across the loop
      const shortx4 lo = ds_read_tr_at(kb ? ((tv + ofs.vo[j][0]) ^ 32u) + KB16 : tv + ofs.vo[j][0]);
      const shortx4 hi = ds_read_tr_at(kb ? ((tv + ofs.vo[j][1]) ^ 32u) + KB16 : tv + ofs.vo[j][1]);
      va[j][kb] = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                                 lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
  const floatx16 sn = pf_scores<D>(st, tk, ofs);
  float z[16];
  float mt = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = s[r];
    if constexpr (MASK) {
      if (tb + 8 * (r >> 2) + 4 * h + (r & 3) > pos) x = -INFINITY;
    }
    z[r] = x;
    mt = fmaxf(mt, x);
  }
  mt = pair_max(mt) * c2;
  const bool move = mt > st.m + kPfLazy;  // true on a row's first tile with a key
  const float mn = move ? mt : st.m;
  const float corr = (move && st.m != -INFINITY) ? exp2_fast(st.m - mn) : 1.0f;
  const float mref = mn == -INFINITY ? 0.0f : mn;  // no key yet: every z is -inf
  float lt = 0.0f;
  const bf16x2 ones2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  bf16x8 pb[2];
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const floatx2 e = {exp2_fast(fmaf(z[r], c2, -mref)), exp2_fast(fmaf(z[r + 1], c2, -mref))};
    const bf16x2 pp = __builtin_convertvector(e, bf16x2);
    lt = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, lt, false);
    pb[r >> 3][r & 7] = pp[0];
    pb[r >> 3][(r & 7) + 1] = pp[1];
  }
  lt = pair_sum(lt);
  st.l = st.l * corr + lt;
  st.m = mn;
  // the LDS reads first, then each score MFMA followed by a share of the softmax
#pragma unroll
  for (int i = 0; i < C::KQ; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five VALU instructions
  }
  if (__any(corr != 1.0f)) {
#pragma unroll
    for (int j = 0; j < DB; ++j) scale_acc(st.acc[j], corr);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int j = 0; j < DB; ++j) st.acc[j] = mfma32(va[j][kb], pb[kb], st.acc[j]);
  return sn;
}

// This wave's quarter of the direct-to-LDS loads of a tile: wave w issues loads
// [LOADS/4 w, LOADS/4 (w + 1)) (K rows for w < 2, V rows for w >= 2).  Lane l of a
// wave-wide load lands at LDS (M0 + 16 l) and picks the global chunk the swizzle puts
// there.  Issued from inline assembly so the compiler does not fence later LDS reads
// on them; the caller waits with wait_vm before the barrier that publishes the tile.
template <int D>
struct PfDma {
  using C = PfCfg<D>;
  static constexpr int N = C::LOADS / 4;
  uint32_t off[N];
  int ins0;
  __device__ __forceinline__ void init(int wave) {
    ins0 = __builtin_amdgcn_readfirstlane(wave) * N;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int li = (ins0 + x) % (C::LOADS / 2);
      const int row = li * C::RPL + lane / C::CPR;
      off[x] = static_cast<uint32_t>(pf_off<D>(row, lane % C::CPR));
    }
  }
  __device__ __forceinline__ void issue(unsigned char *stage, __amdgpu_buffer_rsrc_t kres,
                                        __amdgpu_buffer_rsrc_t vres, int64_t tb) const {
    const uint32_t base = static_cast<uint32_t>(tb * C::ROWB);
    const uint32_t lds = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char *)(stage)));
#pragma unroll
    for (int x = 0; x < N; ++x) {
      const int ins = ins0 + x;
      const bool v = ins >= C::LOADS / 2;  // uniform over the wave
      asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                   :
                   : "v"(base + off[x]), "s"(__builtin_amdgcn_readfirstlane(lds + ins * 1024)), "s"(v ? vres : kres)
                   : "memory", "m0");
    }
  }
};

// Workgroup b covers item j(b): the items of XCD x (b = x mod 8) are the contiguous
// range [x items/8, (x + 1) items/8) of the order (kv head, split, row tile), so the
// row tiles that read the same keys run on one XCD and share its L2.
template <int D>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const PfAttn P) {
  using C = PfCfg<D>;
  constexpr int S = kPfStages;
  constexpr int IPW = PfDma<D>::N;
  static_assert(S >= 3 && (S - 2) * IPW <= 63, "tiles t and t + 1 resident; loads in flight per wave");
  __shared__ __align__(1024) unsigned char ring[S][C::TILE];
  const int b = blockIdx.x;
  const int item = (b % 8) * (P.items / 8) + b / 8;
  const int per_head = P.nsplit * P.row_tiles;
  const int h = item / per_head;
  if (h >= P.hkv) return;  // padding items
  const int sp = (item % per_head) / P.row_tiles, rt = item % P.row_tiles;
  const int G = P.hq / P.hkv;
  const int M = P.T * G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // rows of the tile and their last keys
  const int rlast = min(M - 1, kPfRows * rt + kPfRows - 1);
  const int64_t k0 = static_cast<int64_t>(sp) * P.split;
  const int64_t k1 = min(k0 + P.split, P.L + rlast / G + 1);  // keys [k0, k1) of this item
  if (k0 >= k1) return;  // every row of the tile ends before this split
  const int ntiles = static_cast<int>((k1 - k0 + kKvTile - 1) / kKvTile);
  const int r0 = kPfRows * rt + 32 * wave;          // this wave's first row
  const int r = min(r0 + (lane & 31), M - 1);       // this lane's row (past the rows: a copy)
  const int64_t pos = P.L + r / G;                   // its last key
  const int64_t pos_min = P.L + min(r0, M - 1) / G;  // the wave's smallest last key

  const unsigned char *kc = static_cast<const unsigned char *>(P.kc) + static_cast<int64_t>(h) * P.cap * C::ROWB;
  const unsigned char *vc = static_cast<const unsigned char *>(P.vc) + static_cast<int64_t>(h) * P.cap * C::ROWB;
  const int64_t valid = P.L + P.T;  // rows past the span read as zeros
  const __amdgpu_buffer_rsrc_t kres = make_rsrc(kc, valid * C::ROWB);
  const __amdgpu_buffer_rsrc_t vres = make_rsrc(vc, valid * C::ROWB);

  PfDma<D> dma;
  dma.init(wave);
  const int first = min(S - 1, ntiles);
  for (int x = 0; x < first; ++x) dma.issue(ring[x], kres, vres, k0 + static_cast<int64_t>(x) * kKvTile);
  PfRows<D> st;
  PfLane<D> ofs;
  ofs.init();
  {
    const int t = r / G, j = h * G + r % G;
    const unsigned char *qr = static_cast<const unsigned char *>(P.q) + (static_cast<int64_t>(t) * P.hq + j) * C::ROWB;
#pragma unroll
    for (int kk = 0; kk < C::KQ; ++kk) st.q[kk] = *reinterpret_cast<const bf16x8 *>(qr + (16 * kk + 8 * (lane >> 5)) * 2);
  }
  wait_vm<0>();  // the query rows and the first tiles
  bare_barrier();
#pragma unroll
  for (int j = 0; j < C::DB; ++j) st.acc[j] = floatx16{};
  st.m = -INFINITY;
  st.l = 0.0f;
  const uint32_t ring0 = lds_addr(ring[0]);
  // Tile t's softmax and value product run in iteration t together with tile t + 1's
  // scores, so tiles t and t + 1 are in LDS during it; the iteration's barrier frees the
  // stage of tile t - 1 for tile t + S - 1.  The last iteration scores a stale stage and
  // drops the result.
  floatx16 sc = pf_scores<D>(st, ring0, ofs);
  int stage = 0;
  for (int tt = 0; tt < ntiles; ++tt) {
    if (tt > 0) {
      // tiles up to min(tt + S - 2, ntiles - 1) are issued; wait for tile tt + 1
      const int ahead = min(S - 3, ntiles - 2 - tt);
      static_assert(S <= 5, "at most two tiles ahead of the one waited for");
      if (ahead >= 2) {
        wait_vm<2 * IPW>();
      } else if (ahead == 1) {
        wait_vm<IPW>();
      } else if (ahead == 0) {
        wait_vm<0>();
      }
      bare_barrier();  // tile tt + 1 landed for every wave; tile tt - 1 is no longer read
    }
    if (tt + S - 1 < ntiles)
      dma.issue(ring[stage == 0 ? S - 1 : stage - 1], kres, vres, k0 + static_cast<int64_t>(tt + S - 1) * kKvTile);
    const int nstage = stage == S - 1 ? 0 : stage + 1;
    const int64_t tb = k0 + static_cast<int64_t>(tt) * kKvTile;
    const uint32_t tk = ring0 + nstage * C::TILE, tv = ring0 + stage * C::TILE;
    if (tb + kKvTile - 1 > pos_min)
      sc = pf_step<D, true>(st, sc, tk, tv, ofs, tb, pos, P.c2);
    else
      sc = pf_step<D, false>(st, sc, tk, tv, ofs, tb, pos, P.c2);
    stage = nstage;
  }
  // ---- out: lane l holds row r0 + l % 32, columns 32 j + 8 b + 4 (l / 32) + e
  if (r0 + (lane & 31) >= M) return;
  const int hh = lane >> 5;
  if (P.nsplit == 1) {
    const float inv = 1.0f / st.l;
    const int t = r / G, j = h * G + r % G;
    uint16_t *o = static_cast<uint16_t *>(P.o) + (static_cast<int64_t>(t) * P.hq + j) * D;
#pragma unroll
    for (int j2 = 0; j2 < C::DB; ++j2)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        uint16_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = bf16_bits(st.acc[j2][4 * b4 + e] * inv);
        *reinterpret_cast<uint2 *>(o + 32 * j2 + 8 * b4 + 4 * hh) = *reinterpret_cast<const uint2 *>(w);
      }
  } else {
    const int64_t prow = (static_cast<int64_t>(h) * P.nsplit + sp) * P.rows_cap + r;
    float *pa = P.part_acc + prow * D;
#pragma unroll
    for (int j2 = 0; j2 < C::DB; ++j2)
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4)
        *reinterpret_cast<floatx4 *>(pa + 32 * j2 + 8 * b4 + 4 * hh) =
            floatx4{st.acc[j2][4 * b4], st.acc[j2][4 * b4 + 1], st.acc[j2][4 * b4 + 2], st.acc[j2][4 * b4 + 3]};
    if (hh == 0) *reinterpret_cast<floatx2 *>(P.part_ml + prow * 2) = floatx2{st.m, st.l};
  }
}

// Merge of a row's split partials: splits 0 .. (L + t) / split hold its keys.  One
// 64-lane group per (kv head, row), four columns a lane.
template <int D>
__global__ __launch_bounds__(256) void attn_prefill_fold_kernel(const PfAttn P) {
  const int G = P.hq / P.hkv, M = P.T * G;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (x >= static_cast<int64_t>(P.hkv) * M) return;
  const int h = static_cast<int>(x / M), r = static_cast<int>(x % M);
  const int t = r / G, lane = threadIdx.x & 63;
  const int ns = min(P.nsplit, static_cast<int>((P.L + t) / P.split) + 1);
  const int64_t base = static_cast<int64_t>(h) * P.nsplit * P.rows_cap + r;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, P.part_ml[(base + static_cast<int64_t>(s) * P.rows_cap) * 2]);
  float den = 0.0f;
  floatx4 num = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const int64_t prow = base + static_cast<int64_t>(s) * P.rows_cap;
    const float m = P.part_ml[prow * 2], l = P.part_ml[prow * 2 + 1];
    if (l == 0.0f) continue;
    const float w = exp2_fast(m - mx);
    den += w * l;
    num += w * *reinterpret_cast<const floatx4 *>(P.part_acc + prow * D + 4 * lane);
  }
  const float inv = 1.0f / den;
  uint16_t w4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = bf16_bits(num[e] * inv);
  uint16_t *o = static_cast<uint16_t *>(P.o) + (static_cast<int64_t>(t) * P.hq + h * G + r % G) * D;
  *reinterpret_cast<uint2 *>(o + 4 * lane) = *reinterpret_cast<const uint2 *>(w4);
}

// The span's K and V rows into the caches at [L, L + T): 16 bytes a thread.
template <int D>
__global__ __launch_bounds__(256) void pf_copy_kernel(const PfCopy P) {
  constexpr int CPR = D / 8;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per = static_cast<int64_t>(P.T) * P.hkv * CPR;
  if (x >= 2 * per) return;
  const bool isv = x >= per;
  const int64_t y = isv ? x - per : x;
  const int c = static_cast<int>(y % CPR);
  const int64_t row = y / CPR;  // t hkv + head
  const int hd = static_cast<int>(row % P.hkv);
  const int64_t t = row / P.hkv;
  const uint4 val = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(isv ? P.v : P.k) + row * D + 8 * c);
  uint16_t *dst = static_cast<uint16_t *>(isv ? P.vc : P.kc) + (static_cast<int64_t>(hd) * P.cap + P.L + t) * D + 8 * c;
  *reinterpret_cast<uint4 *>(dst) = val;
}

}  // namespace

hipError_t launch_wy_prep(const WyPrep &a, int dk, hipStream_t s, KernelEvents ev) {
  if (dk != 128) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL((gdn_wy_prep_kernel<128, 128>), dim3(a.n_chunks, a.hv), dim3(256), 0, s, ev.start,
                        ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_wy_scan(const WyScan &a, int dk, hipStream_t s, KernelEvents ev) {
  if (dk != 128) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL((gdn_wy_scan_kernel<128, 128>), dim3(a.hv, 128 / 16), dim3(256), 0, s, ev.start,
                        ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_pf_copy(const PfCopy &a, int D, hipStream_t s) {
  if (D != 256) return hipErrorInvalidValue;
  const int64_t n = 2 * static_cast<int64_t>(a.T) * a.hkv * (D / 8);
  hipLaunchKernelGGL((pf_copy_kernel<256>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_attn(const PfAttn &a, int D, hipStream_t s, KernelEvents ev) {
  if (D != 256 || a.items % 8 != 0) return hipErrorInvalidValue;
  hipExtLaunchKernelGGL((attn_prefill_kernel<256>), dim3(a.items), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_pf_fold(const PfAttn &a, int D, hipStream_t s, KernelEvents ev) {
  if (D != 256) return hipErrorInvalidValue;
  const int64_t rows = static_cast<int64_t>(a.hkv) * a.T * (a.hq / a.hkv);
  hipExtLaunchKernelGGL((attn_prefill_fold_kernel<256>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256),
                        0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace hdt
