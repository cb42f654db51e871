// conv.hip - the short causal convolution in front of a Gated DeltaNet layer, over a
// draft tree (the gdn.conv state section of "Adding a model", "The model layer:
// architecture registry and per-model state": a GDN layer keeps a conv tail beside
// its recurrent state).
//
//  gdn_conv_kernel  per (channel chunk, node, tree): a depthwise causal
//                   convolution of `width` taps along the node's root path, then
//                   SiLU, then the L2 norm of every q and k head (the published
//                   Gated DeltaNet block).  Taps older than the root read the
//                   slot's committed tail.  The post-conv q, k, v go to the
//                   engine's scratch, where the GDN walk reads them; the node's
//                   own pre-conv row is kept for commit, which rolls it into the
//                   tail.
//
// Layout: one thread owns 16 bytes of channels (8 bf16 or 4 float32) of one node
// row, so every load and store is a 16-byte vector and a wave covers 512 (bf16)
// or 256 (float32) consecutive channels.  A q or k head of dk channels is dk/8 or
// dk/4 consecutive lanes of one wave; its sum of squares is an xor butterfly over
// those lanes, which leaves the same bits in every lane.
//
// Bit-exactness (a verified row equals the decode row, "Adding a model", step 4
// of "The adapter path in ten steps"): a node's outputs are a function of its
// width input rows and the taps alone.  A decode step reads the same rows from
// the tail that commit wrote there as bit copies, so it computes the same values.
#include "common.h"

#pragma clang fp contract(off)

namespace hdt {
namespace {

// 16 bytes of an io-dtype row widened to float.
template <bool BF>
__device__ __forceinline__ void load_chunk(const void *base, int64_t elem, float *x, uint4 &raw) {
  raw = *reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(base) +
                                         elem * (BF ? 2 : 4));
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
}

template <bool BF>
__device__ __forceinline__ void store_chunk(void *base, int64_t elem, const float *y) {
  uint4 out;
  if constexpr (BF) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(bf16_bits(y[2 * i])) |
             (static_cast<uint32_t>(bf16_bits(y[2 * i + 1])) << 16);
    out = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    out = make_uint4(__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                     __float_as_uint(y[3]));
  }
  *reinterpret_cast<uint4 *>(static_cast<unsigned char *>(base) + elem * (BF ? 2 : 4)) = out;
}

template <bool BF, int W>
__global__ __launch_bounds__(kConvThreads) void gdn_conv_kernel(const ConvLaunch P) {
  constexpr int CPT = BF ? 8 : 4;
  const ConvTree &T = P.t[blockIdx.z];
  const int node = blockIdx.y;
  if (node >= T.n) return;
  const int CQ = P.hk * P.dk;
  const int C = 2 * CQ + P.hv * P.dv;
  const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * CPT;
  if (c0 >= C) return;

  // where channel c0 of a node row lives: q, k or v, and the element offset in it
  const void *in;
  void *out;
  int64_t row_len, col;
  if (c0 < CQ) {
    in = T.q, out = T.qo, row_len = CQ, col = c0;
  } else if (c0 < 2 * CQ) {
    in = T.k, out = T.ko, row_len = CQ, col = c0 - CQ;
  } else {
    in = T.v, out = T.vo, row_len = static_cast<int64_t>(P.hv) * P.dv, col = c0 - 2 * CQ;
  }

  // tap j reads the input r = W-1-j steps above the node: an ancestor while
  // r <= depth, else tail row (W-1) - (r - depth)
  const int d = T.depth[node];
  const void *src[W];
  int64_t off[W];
  {
    int a = node;
#pragma unroll
    for (int r = 0; r < W; ++r) {
      if (r > 0 && r <= d) a = T.parent[a];
      if (r <= d) {
        src[W - 1 - r] = in;
        off[W - 1 - r] = a * row_len + col;
      } else {
        src[W - 1 - r] = T.tail;
        off[W - 1 - r] = static_cast<int64_t>((W - 1) - (r - d)) * C + c0;
      }
    }
  }
  float x[W][CPT];
  uint4 own;
#pragma unroll
  for (int j = 0; j < W; ++j) {
    uint4 raw;
    load_chunk<BF>(src[j], off[j], x[j], raw);
    if (j == W - 1) own = raw;
  }
  float wt[CPT * W];
  {
    const float4 *wp = reinterpret_cast<const float4 *>(P.weight + static_cast<int64_t>(c0) * W);
#pragma unroll
    for (int i = 0; i < CPT * W / 4; ++i) {
      const float4 f = wp[i];
      wt[4 * i] = f.x, wt[4 * i + 1] = f.y, wt[4 * i + 2] = f.z, wt[4 * i + 3] = f.w;
    }
  }
  // the node's own pre-conv row, for the tail commit
  *reinterpret_cast<uint4 *>(static_cast<unsigned char *>(T.x_pend) +
                             (static_cast<int64_t>(node) * C + c0) * (BF ? 2 : 4)) = own;

  float y[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < W; ++j) acc = fmaf(wt[e * W + j], x[j][e], acc);
    y[e] = acc / (1.0f + __expf(-acc));  // SiLU
  }
  if (c0 < 2 * CQ) {
    // L2 norm of the head: dk / CPT lanes, aligned within the wave
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) ss = fmaf(y[e], y[e], ss);
    const int lanes = P.dk / CPT;
    for (int m = 1; m < lanes; m <<= 1) ss = ss + __shfl_xor(ss, m);
    const float inv = rsqrtf(ss + P.eps);
#pragma unroll
    for (int e = 0; e < CPT; ++e) y[e] = y[e] * inv;
  }
  store_chunk<BF>(out, static_cast<int64_t>(node) * row_len + col, y);
}

// The conv over a prefill span: token t of the span is a chain node at depth t, so tap
// j reads span row t - r (r = W-1-j) while r <= t, else tail row (W-1) - (r - t); the
// arithmetic is gdn_conv_kernel's.  A thread takes kPfConvTokens consecutive tokens of
// its 16 bytes of channels and slides the W-row window down them, so each input row is
// loaded once per run.  Grid: x = channel block, y = run of tokens.
constexpr int kPfConvTokens = 8;

template <bool BF, int W>
__global__ __launch_bounds__(kPfConvThreads) void pf_conv_kernel(const PfConv P) {
  constexpr int CPT = BF ? 8 : 4;
  const int t0 = blockIdx.y * kPfConvTokens;
  const int CQ = P.hk * P.dk;
  const int C = 2 * CQ + P.hv * P.dv;
  const int c0 = (blockIdx.x * kPfConvThreads + threadIdx.x) * CPT;
  if (t0 >= P.T || c0 >= C) return;
  const void *in;
  void *out;
  int64_t row_len, col;
  if (c0 < CQ) {
    in = P.q, out = P.qo, row_len = CQ, col = c0;
  } else if (c0 < 2 * CQ) {
    in = P.k, out = P.ko, row_len = CQ, col = c0 - CQ;
  } else {
    in = P.v, out = P.vo, row_len = static_cast<int64_t>(P.hv) * P.dv, col = c0 - 2 * CQ;
  }
  // row s of (tail, span): span row s >= 0, else tail row (W-1) + s
  auto load_row = [&](int srow, float *x) {
    uint4 raw;
    if (srow >= 0) {
      load_chunk<BF>(in, static_cast<int64_t>(srow) * row_len + col, x, raw);
    } else {
      load_chunk<BF>(P.tail, static_cast<int64_t>((W - 1) + srow) * C + c0, x, raw);
    }
  };
  float wt[CPT * W];
  {
    const float4 *wp = reinterpret_cast<const float4 *>(P.weight + static_cast<int64_t>(c0) * W);
#pragma unroll
    for (int i = 0; i < CPT * W / 4; ++i) {
      const float4 f = wp[i];
      wt[4 * i] = f.x, wt[4 * i + 1] = f.y, wt[4 * i + 2] = f.z, wt[4 * i + 3] = f.w;
    }
  }
  float x[W][CPT];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) load_row(t0 - (W - 1) + j, x[j]);
  const int n = min(kPfConvTokens, P.T - t0);
  for (int i = 0; i < n; ++i) {
    const int t = t0 + i;
    load_row(t, x[W - 1]);
    float y[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < W; ++j) acc = fmaf(wt[e * W + j], x[j][e], acc);
      y[e] = acc / (1.0f + __expf(-acc));  // SiLU
    }
    if (c0 < 2 * CQ) {
      float ss = 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) ss = fmaf(y[e], y[e], ss);
      const int lanes = P.dk / CPT;
      for (int m = 1; m < lanes; m <<= 1) ss = ss + __shfl_xor(ss, m);
      const float inv = rsqrtf(ss + P.eps);
#pragma unroll
      for (int e = 0; e < CPT; ++e) y[e] = y[e] * inv;
    }
    store_chunk<BF>(out, static_cast<int64_t>(t) * row_len + col, y);
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
      for (int e = 0; e < CPT; ++e) x[j][e] = x[j + 1][e];
  }
}

// The tail after the span: its last W - 1 rows of (old tail, span rows).  Row i takes
// combined row T + i; each thread moves its 16 bytes of channels in ascending i, so a
// tail row is read (T + i > i) before it is overwritten.  Runs after pf_conv_kernel.
template <bool BF>
__global__ __launch_bounds__(kPfConvThreads) void pf_conv_tail_kernel(const PfConv P) {
  constexpr int CPT = BF ? 8 : 4;
  const int CQ = P.hk * P.dk;
  const int C = 2 * CQ + P.hv * P.dv;
  const int c0 = (blockIdx.x * kPfConvThreads + threadIdx.x) * CPT;
  if (c0 >= C) return;
  const void *in;
  int64_t row_len, col;
  if (c0 < CQ) {
    in = P.q, row_len = CQ, col = c0;
  } else if (c0 < 2 * CQ) {
    in = P.k, row_len = CQ, col = c0 - CQ;
  } else {
    in = P.v, row_len = static_cast<int64_t>(P.hv) * P.dv, col = c0 - 2 * CQ;
  }
  constexpr int ESZ = BF ? 2 : 4;
  unsigned char *tail = static_cast<unsigned char *>(P.tail);
  for (int i = 0; i < P.width - 1; ++i) {
    const int k = P.T + i;  // row of (old tail, span)
    const uint4 x = k < P.width - 1
                        ? *reinterpret_cast<const uint4 *>(tail + (static_cast<int64_t>(k) * C + c0) * ESZ)
                        : *reinterpret_cast<const uint4 *>(static_cast<const unsigned char *>(in) +
                                                           (static_cast<int64_t>(k - (P.width - 1)) * row_len + col) * ESZ);
    *reinterpret_cast<uint4 *>(tail + (static_cast<int64_t>(i) * C + c0) * ESZ) = x;
  }
}

}  // namespace

hipError_t launch_gdn_conv(const ConvLaunch &a, int bf16, hipStream_t s, KernelEvents ev) {
  const int C = 2 * a.hk * a.dk + a.hv * a.dv;
  const int cpt = conv_channels_per_thread(bf16);
  const dim3 grid((C / cpt + kConvThreads - 1) / kConvThreads, a.n_max, a.n_trees);
#define HDT_CONV(BF, W)                                                                       \
  hipExtLaunchKernelGGL((gdn_conv_kernel<BF, W>), grid, dim3(kConvThreads), 0, s, ev.start,  \
                        ev.stop, 0, a)
#define HDT_CONV_W(BF)                                                                        \
  switch (a.width) {                                                                          \
    case 1: HDT_CONV(BF, 1); break;                                                           \
    case 2: HDT_CONV(BF, 2); break;                                                           \
    case 3: HDT_CONV(BF, 3); break;                                                           \
    case 4: HDT_CONV(BF, 4); break;                                                           \
    default: return hipErrorInvalidValue;                                                     \
  }
  if (bf16) {
    HDT_CONV_W(true)
  } else {
    HDT_CONV_W(false)
  }
#undef HDT_CONV_W
#undef HDT_CONV
  return hipGetLastError();
}

hipError_t launch_pf_conv(const PfConv &a, int bf16, hipStream_t s, KernelEvents ev) {
  const int C = 2 * a.hk * a.dk + a.hv * a.dv;
  const int cpt = conv_channels_per_thread(bf16);
  const dim3 grid((C / cpt + kPfConvThreads - 1) / kPfConvThreads, (a.T + kPfConvTokens - 1) / kPfConvTokens);
#define HDT_PFCONV(BF, W)                                                                     \
  hipExtLaunchKernelGGL((pf_conv_kernel<BF, W>), grid, dim3(kPfConvThreads), 0, s, ev.start,   \
                        ev.stop, 0, a)
#define HDT_PFCONV_W(BF)                                                                      \
  switch (a.width) {                                                                          \
    case 1: HDT_PFCONV(BF, 1); break;                                                         \
    case 2: HDT_PFCONV(BF, 2); break;                                                         \
    case 3: HDT_PFCONV(BF, 3); break;                                                         \
    case 4: HDT_PFCONV(BF, 4); break;                                                         \
    default: return hipErrorInvalidValue;                                                     \
  }
  if (bf16) {
    HDT_PFCONV_W(true)
  } else {
    HDT_PFCONV_W(false)
  }
#undef HDT_PFCONV_W
#undef HDT_PFCONV
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.width < 2) return err;
  const dim3 tgrid((C / cpt + kPfConvThreads - 1) / kPfConvThreads);
  if (bf16) {
    hipLaunchKernelGGL((pf_conv_tail_kernel<true>), tgrid, dim3(kPfConvThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((pf_conv_tail_kernel<false>), tgrid, dim3(kPfConvThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hdt
