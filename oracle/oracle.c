/*
 * oracle.c - plain, slow CPU reference for the speculative tree-verify pass of
 * a hybrid Gated DeltaNet + attention model.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the GPU library, and the GPU library never calls it.
 *
 * Precision: float32 arithmetic throughout (the workload description fixes a
 * float32 oracle), compiled without fast-math and with floating-point
 * contraction off, every sum taken in ascending index order in a plain loop.
 *
 * Sources (page titles and sections; the pages name the layers and the verbs
 * but print no equations):
 *  - "Adding a model", step 4 of "The adapter path in ten steps": the hot
 *    verbs forward_tree / forward_block / commit_tree / rollback_to, and the
 *    rule that every verified row equals the decode step's row.
 *  - "Adding a model", "What is still specific to Qwen3.8": a Gated DeltaNet
 *    layer and attention layer; recurrent state heads of 128 by 128.
 *  - "Adding a model", "The model layer: architecture registry and per-model
 *    state": the state sections (recurrent S) and the K, V views indexed by
 *    token position.
 *  - "One request, end to end", section 2.6 "The decode loop": one forward pass
 *    verifies the whole merged tree; the accepted path's KV rows and recurrent
 *    state are committed.
 *  - The Gated DeltaNet recurrence itself is the published one (S. Yang,
 *    J. Kautz, A. Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with
 *    Delta Rule", ICLR 2025):  S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,
 *    o_t = S_t^T (s q_t), with S of shape d_k x d_v.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - tree: node 0 is the root, parent[i] < i; node i sits at position
 *    L + depth[i]; node i attends to every resident row and to its
 *    ancestors-or-self;
 *  - v head h reads q/k head h / (hv / hk); q head j reads kv head j / (hq / hkv);
 *  - gates a, b arrive as values in (0,1);
 *  - the GDN readout scale s and the attention scale are parameters
 *    (1/sqrt(d_k) and 1/sqrt(D) by default);
 *  - storage layouts: recurrent state [hv][dv][dk] (S[a][c] of head h at
 *    h*dv*dk + c*dk + a); GDN q,k [n][hk][dk], v [n][hv][dv], a,b [n][hv];
 *    attention q [n][hq][D], tree k,v [n][hkv][D], resident cache [hkv][cap][D].
 *  Inputs arrive as float32 values or bfloat16 bit patterns (dtype 0 or 1);
 *  the oracle widens bfloat16 itself.  Outputs are float32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#pragma STDC FP_CONTRACT OFF

#define ORC_MAX_NODES 64

/* Element i of an input array stored as float32 (dtype 0) or bfloat16 bits (dtype 1). */
static float ld(const void *p, int dtype, int64_t i) {
  if (dtype == 0) return ((const float *)p)[i];
  uint32_t b = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

/*
 * Tree metadata.  parent[0] = -1 and 0 <= parent[i] < i for i >= 1.
 * depth[i] = depth[parent[i]] + 1; mask[i] = mask[parent[i]] | bit i (ancestors
 * or self); anc[i*64 + d] = the ancestor of i at depth d for d <= depth[i], -1
 * beyond; pos[i] = L + depth[i].  Returns 0, or -1 for an invalid tree.
 */
int orc_tree_meta(int n, const int32_t *parent, int64_t L, int32_t *depth, uint64_t *mask,
                  int32_t *anc, int64_t *pos) {
  if (n < 1 || n > ORC_MAX_NODES || parent[0] != -1) return -1;
  for (int i = 1; i < n; ++i)
    if (parent[i] < 0 || parent[i] >= i) return -1;
  for (int i = 0; i < n; ++i) {
    const int p = parent[i];
    depth[i] = (p < 0) ? 0 : depth[p] + 1;
    mask[i] = ((p < 0) ? 0 : mask[p]) | (1ULL << i);
    pos[i] = L + depth[i];
    for (int d = 0; d < ORC_MAX_NODES; ++d) anc[i * ORC_MAX_NODES + d] = -1;
    int j = i;
    while (j >= 0) {
      anc[i * ORC_MAX_NODES + depth[j]] = j;
      j = parent[j];
    }
  }
  return 0;
}

/*
 * One Gated DeltaNet step for one head, in the key-by-value orientation
 * (S[a][c], a over d_k, c over d_v), starting from the state P:
 *   A   = alpha * P                         (decay first)
 *   r_c = sum_a A[a][c] k[a]                (k^T S)
 *   u_c = beta * (v_c - r_c)                (delta-rule correction)
 *   S[a][c] = A[a][c] + k[a] u_c            (rank-1 write at key k)
 *   o_c = sum_a S[a][c] (s q[a])            (S q readout)
 * This is the published recurrence S = a (I - b k k^T) P + b k v^T expanded
 * column by column.  P and S use the [c][a] storage; they may not alias.
 */
static void gdn_step(int dk, int dv, const float *P, float *S, const float *k, const float *q,
                     const float *v, float alpha, float beta, float scale, float *o) {
  float *A = (float *)malloc(sizeof(float) * (size_t)dk);
  for (int c = 0; c < dv; ++c) {
    const float *Pc = P + (size_t)c * dk;
    float *Sc = S + (size_t)c * dk;
    for (int a = 0; a < dk; ++a) A[a] = alpha * Pc[a];
    float r = 0.0f;
    for (int a = 0; a < dk; ++a) r = r + A[a] * k[a];
    const float u = beta * (v[c] - r);
    for (int a = 0; a < dk; ++a) Sc[a] = A[a] + k[a] * u;
    if (o) {
      float acc = 0.0f;
      for (int a = 0; a < dk; ++a) acc = acc + Sc[a] * (scale * q[a]);
      o[c] = acc;
    }
  }
  free(A);
}

/*
 * Tree recurrence of one GDN layer (all heads).  Nodes are visited in index
 * order, which is a parent-first order; node i starts from S_base when it is
 * the root and from its parent's state otherwise.
 *   S_base [hv][dv][dk] float32; q,k [n][hk][dk]; v [n][hv][dv]; alpha,beta [n][hv].
 *   o [n][hv][dv] float32 out.  S_nodes (optional) [n][hv][dv][dk] float32 out:
 *   the state after each node.
 */
void orc_gdn_tree(int dk, int dv, int hk, int hv, int n, const int32_t *parent,
                  const float *S_base, const void *q, const void *k, const void *v,
                  const void *alpha, const void *beta, int dtype, float scale, float *o,
                  float *S_nodes) {
  const size_t hs = (size_t)dv * dk;
  float *all = S_nodes ? S_nodes : (float *)malloc(sizeof(float) * hs * hv * (size_t)n);
  float *kf = (float *)malloc(sizeof(float) * (size_t)dk);
  float *qf = (float *)malloc(sizeof(float) * (size_t)dk);
  float *vf = (float *)malloc(sizeof(float) * (size_t)dv);
  const int ratio = hv / hk;
  for (int i = 0; i < n; ++i) {
    for (int h = 0; h < hv; ++h) {
      const int g = h / ratio;
      for (int a = 0; a < dk; ++a) {
        kf[a] = ld(k, dtype, ((int64_t)i * hk + g) * dk + a);
        qf[a] = ld(q, dtype, ((int64_t)i * hk + g) * dk + a);
      }
      for (int c = 0; c < dv; ++c) vf[c] = ld(v, dtype, ((int64_t)i * hv + h) * dv + c);
      const float al = ld(alpha, dtype, (int64_t)i * hv + h);
      const float be = ld(beta, dtype, (int64_t)i * hv + h);
      const float *P = (parent[i] < 0) ? S_base + (size_t)h * hs
                                       : all + ((size_t)parent[i] * hv + h) * hs;
      float *S = all + ((size_t)i * hv + h) * hs;
      gdn_step(dk, dv, P, S, kf, qf, vf, al, be, scale, o + ((size_t)i * hv + h) * dv);
    }
  }
  free(kf);
  free(qf);
  free(vf);
  if (!S_nodes) free(all);
}

/*
 * Committed recurrent state after accepting `path` (m nodes, a root path):
 * the plain sequential recurrence from S_base over the path's inputs, written
 * to S_out [hv][dv][dk].  It recomputes every step and reuses nothing from a
 * tree pass.
 */
void orc_gdn_commit(int dk, int dv, int hk, int hv, int m, const int32_t *path,
                    const float *S_base, const void *k, const void *v, const void *alpha,
                    const void *beta, int dtype, float *S_out) {
  const size_t hs = (size_t)dv * dk;
  float *cur = (float *)malloc(sizeof(float) * hs);
  float *nxt = (float *)malloc(sizeof(float) * hs);
  float *kf = (float *)malloc(sizeof(float) * (size_t)dk);
  float *vf = (float *)malloc(sizeof(float) * (size_t)dv);
  const int ratio = hv / hk;
  for (int h = 0; h < hv; ++h) {
    memcpy(cur, S_base + (size_t)h * hs, sizeof(float) * hs);
    for (int d = 0; d < m; ++d) {
      const int i = path[d];
      const int g = h / ratio;
      for (int a = 0; a < dk; ++a) kf[a] = ld(k, dtype, ((int64_t)i * hk + g) * dk + a);
      for (int c = 0; c < dv; ++c) vf[c] = ld(v, dtype, ((int64_t)i * hv + h) * dv + c);
      gdn_step(dk, dv, cur, nxt, kf, kf, vf, ld(alpha, dtype, (int64_t)i * hv + h),
               ld(beta, dtype, (int64_t)i * hv + h), 0.0f, NULL);
      float *t = cur;
      cur = nxt;
      nxt = t;
    }
    memcpy(S_out + (size_t)h * hs, cur, sizeof(float) * hs);
  }
  free(cur);
  free(nxt);
  free(kf);
  free(vf);
}

/*
 * Ancestor-masked attention for one row: node `node`, q head `j`.
 * The row's keys, in ascending position order, are the resident rows
 * 0..L-1 of kv head j/(hq/hkv), then positions L+d for d = 0..depth[node],
 * whose key/value is the tree row of the node's ancestor at depth d.
 *   z_t = scale * (q . k_t);  m = max z;  w_t = exp(z_t - m);
 *   o = (sum_t w_t v_t) / (sum_t w_t).
 * Kc, Vc [hkv][cap][D]; q [n][hq][D]; kt, vt [n][hkv][D]; out o [D].
 */
void orc_attn_row(int hq, int hkv, int D, int n, const int32_t *parent, int64_t L, int64_t cap,
                  const void *Kc, const void *Vc, const void *q, const void *kt, const void *vt,
                  int dtype, float scale, int node, int j, float *o) {
  int32_t path[ORC_MAX_NODES];
  int depth = 0;
  for (int x = node; x >= 0; x = parent[x]) path[depth++] = x;
  /* path[depth-1] is the root; the ancestor at depth d is path[depth-1-d]. */
  const int m_head = j / (hq / hkv);
  const int64_t nkeys = L + depth;
  float *qf = (float *)malloc(sizeof(float) * (size_t)D);
  float *z = (float *)malloc(sizeof(float) * (size_t)nkeys);
  for (int d = 0; d < D; ++d) qf[d] = ld(q, dtype, ((int64_t)node * hq + j) * D + d);
  for (int64_t t = 0; t < nkeys; ++t) {
    float dot = 0.0f;
    for (int d = 0; d < D; ++d) {
      float kv;
      if (t < L)
        kv = ld(Kc, dtype, ((int64_t)m_head * cap + t) * D + d);
      else
        kv = ld(kt, dtype, ((int64_t)path[depth - 1 - (t - L)] * hkv + m_head) * D + d);
      dot = dot + qf[d] * kv;
    }
    z[t] = scale * dot;
  }
  float mx = -INFINITY;
  for (int64_t t = 0; t < nkeys; ++t) mx = z[t] > mx ? z[t] : mx;
  float l = 0.0f;
  for (int d = 0; d < D; ++d) o[d] = 0.0f;
  for (int64_t t = 0; t < nkeys; ++t) {
    const float w = expf(z[t] - mx);
    l = l + w;
    for (int d = 0; d < D; ++d) {
      float vv;
      if (t < L)
        vv = ld(Vc, dtype, ((int64_t)m_head * cap + t) * D + d);
      else
        vv = ld(vt, dtype, ((int64_t)path[depth - 1 - (t - L)] * hkv + m_head) * D + d);
      o[d] = o[d] + w * vv;
    }
  }
  for (int d = 0; d < D; ++d) o[d] = o[d] / l;
  free(qf);
  free(z);
}

/* All rows of one attention layer: o [n][hq][D] float32. */
void orc_attn_tree(int hq, int hkv, int D, int n, const int32_t *parent, int64_t L, int64_t cap,
                   const void *Kc, const void *Vc, const void *q, const void *kt, const void *vt,
                   int dtype, float scale, float *o) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < hq; ++j)
      orc_attn_row(hq, hkv, D, n, parent, L, cap, Kc, Vc, q, kt, vt, dtype, scale, i, j,
                   o + ((size_t)i * hq + j) * D);
}

/*
 * Short causal convolution of a Gated DeltaNet layer over a tree (the gdn.conv
 * state section of "Adding a model", "The model layer: architecture registry
 * and per-model state": the conv tails kept beside the recurrent state).  The
 * layer's q, k, v channels pass through a depthwise causal convolution of width
 * w along the token axis, then SiLU, and q and k are L2-normalised per head
 * (the published Gated DeltaNet block; the pages name only the section).  Along
 * a tree, the inputs a node sees are those of its root path: its own, its
 * ancestors', and before the root the slot's committed tail.
 *
 * Channel space (C = 2 hk dk + hv dv channels): q channels (head-major), then k,
 * then v.  For node i at depth d and channel c:
 *   x(r) = input of the ancestor-or-self r steps above i  for 0 <= r <= d,
 *          tail[(w-1) - (r - d)][c]                        for r > d
 *   acc  = sum_{j=0}^{w-1} W[c][j] * x(w-1-j)   (ascending j; tap w-1 is the node)
 *   y    = acc / (1 + exp(-acc))                (SiLU)
 * and for every q or k head, y <- y / sqrt(sum_a y_a^2 + eps), the sum ascending.
 *   W [C][w] float32; tail [w-1][C] (row w-2 is the newest committed input);
 *   q,k [n][hk][dk], v [n][hv][dv] pre-conv inputs; outputs float32, same shapes.
 */
void orc_gdn_conv(int hk, int dk, int hv, int dv, int w, int n, const int32_t *parent,
                  const void *tail, const void *q, const void *k, const void *v,
                  const float *W, int dtype, float eps, float *qo, float *ko, float *vo) {
  const int64_t CQ = (int64_t)hk * dk, C = 2 * CQ + (int64_t)hv * dv;
  int32_t up[8];  /* up[r]: the ancestor r steps above node i (w <= 8) */
  for (int i = 0; i < n; ++i) {
    int d = 0;
    for (int x = parent[i]; x >= 0; x = parent[x]) ++d;  /* depth of i */
    up[0] = i;
    for (int r = 1; r < w && r <= d; ++r) up[r] = parent[up[r - 1]];
    for (int64_t c = 0; c < C; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < w; ++j) {
        const int r = w - 1 - j;  /* steps above node i */
        float xin;
        if (r <= d) {
          const int node = up[r];
          if (c < CQ)
            xin = ld(q, dtype, (int64_t)node * CQ + c);
          else if (c < 2 * CQ)
            xin = ld(k, dtype, (int64_t)node * CQ + (c - CQ));
          else
            xin = ld(v, dtype, (int64_t)node * hv * dv + (c - 2 * CQ));
        } else {
          xin = ld(tail, dtype, (int64_t)((w - 1) - (r - d)) * C + c);
        }
        acc = acc + W[c * w + j] * xin;
      }
      const float y = acc / (1.0f + expf(-acc));
      if (c < CQ)
        qo[(int64_t)i * CQ + c] = y;
      else if (c < 2 * CQ)
        ko[(int64_t)i * CQ + (c - CQ)] = y;
      else
        vo[(int64_t)i * hv * dv + (c - 2 * CQ)] = y;
    }
    for (int which = 0; which < 2; ++which) {
      float *base = (which == 0 ? qo : ko) + (int64_t)i * CQ;
      for (int g = 0; g < hk; ++g) {
        float ss = 0.0f;
        for (int a = 0; a < dk; ++a) ss = ss + base[g * dk + a] * base[g * dk + a];
        const float inv = 1.0f / sqrtf(ss + eps);
        for (int a = 0; a < dk; ++a) base[g * dk + a] = base[g * dk + a] * inv;
      }
    }
  }
}
