/*
 * One verify round through the C ABI alone (include/hdt.h), checked against the CPU
 * oracle: a GDN layer and an attention layer with bf16 storage, a 6-node tree over 1,000
 * resident tokens, forward_tree, then commit_tree of a root path.  Inputs come from the
 * seeded generator (libsynth); expected values from the oracle (liboracle).  Test
 * infrastructure: run by tests/test_gpu_c_abi.py.  Prints PASS and exits 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "hdt.h"

/* libsynth */
uint64_t synth_key(uint64_t seed, const char *name);
void synth_fill(uint64_t key, int kind, int64_t row0, int64_t rows, int64_t cols, double scale,
                float *out_f32, uint16_t *out_bf16);
/* liboracle */
void orc_gdn_tree(int dk, int dv, int hk, int hv, int n, const int32_t *parent,
                  const float *S_base, const void *q, const void *k, const void *v,
                  const void *alpha, const void *beta, int dtype, float scale, float *o,
                  float *S_nodes);
void orc_gdn_commit(int dk, int dv, int hk, int hv, int m, const int32_t *path,
                    const float *S_base, const void *k, const void *v, const void *alpha,
                    const void *beta, int dtype, float *S_out);
void orc_attn_tree(int hq, int hkv, int D, int n, const int32_t *parent, int64_t L, int64_t cap,
                   const void *Kc, const void *Vc, const void *q, const void *kt, const void *vt,
                   int dtype, float scale, float *o);

enum { NORMAL = 0, NORMAL_L2 = 1, SIGMOID = 2, EXP_NEG_SP = 3 };
enum { HK = 2, HV = 4, DK = 128, HQ = 12, HKV = 2, D = 256, N = 6, L = 1000, CAP = 1100 };
static const uint64_t SEED = 20261206;

#define CHECK_HIP(x)                                                      \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
      exit(2);                                                            \
    }                                                                     \
  } while (0)
#define CHECK_HDT(eng, x)                                                 \
  do {                                                                    \
    hdt_status s_ = (x);                                                  \
    if (s_ != HDT_OK) {                                                   \
      fprintf(stderr, "%s: %d %s\n", #x, (int)s_, hdt_last_error(eng));   \
      exit(3);                                                            \
    }                                                                     \
  } while (0)

static uint16_t *gen_bf16(const char *name, int kind, int64_t rows, int64_t cols) {
  uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * rows * cols);
  synth_fill(synth_key(SEED, name), kind, 0, rows, cols, 1.0, NULL, h);
  return h;
}

static void *to_dev(const void *h, size_t bytes) {
  void *d = NULL;
  CHECK_HIP(hipMalloc(&d, bytes));
  CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}

static float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* max |got - want| / max |want| over n values; got in bf16 bits or float32 */
static double rel_err(const void *got, int got_bf16, const float *want, size_t n) {
  double num = 0.0, den = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double g = got_bf16 ? bf16f(((const uint16_t *)got)[i]) : ((const float *)got)[i];
    if (!isfinite(g)) return INFINITY;
    num = fmax(num, fabs(g - want[i]));
    den = fmax(den, fabs(want[i]));
  }
  return num / den;
}

int main(void) {
  const int32_t parent[N] = {-1, 0, 1, 1, 3, 2};
  const int32_t path[4] = {0, 1, 3, 4};
  /* GDN layer: inputs and committed state */
  uint16_t *q = gen_bf16("c/gdn/q", NORMAL_L2, N * HK, DK);
  uint16_t *k = gen_bf16("c/gdn/k", NORMAL_L2, N * HK, DK);
  uint16_t *v = gen_bf16("c/gdn/v", NORMAL, N * HV, DK);
  uint16_t *a = gen_bf16("c/gdn/alpha", EXP_NEG_SP, N, HV);
  uint16_t *b = gen_bf16("c/gdn/beta", SIGMOID, N, HV);
  float *S = (float *)malloc(sizeof(float) * HV * DK * DK);
  synth_fill(synth_key(SEED, "c/gdn/S"), NORMAL, 0, HV * DK, DK, sqrt(1.0 / DK), S, NULL);
  /* attention layer: tree inputs and the resident cache rows [0, L) */
  uint16_t *aq = gen_bf16("c/attn/q", NORMAL_L2, N * HQ, D);
  uint16_t *ak = gen_bf16("c/attn/k", NORMAL_L2, N * HKV, D);
  uint16_t *av = gen_bf16("c/attn/v", NORMAL, N * HKV, D);
  uint16_t *Kc = (uint16_t *)calloc((size_t)HKV * CAP * D, 2);
  uint16_t *Vc = (uint16_t *)calloc((size_t)HKV * CAP * D, 2);
  for (int h = 0; h < HKV; ++h) {
    char nk[32], nv[32];
    snprintf(nk, sizeof nk, "c/K/%d", h);
    snprintf(nv, sizeof nv, "c/V/%d", h);
    synth_fill(synth_key(SEED, nk), NORMAL_L2, 0, L, D, 1.0, NULL, Kc + (size_t)h * CAP * D);
    synth_fill(synth_key(SEED, nv), NORMAL, 0, L, D, 1.0, NULL, Vc + (size_t)h * CAP * D);
  }

  float *dS = (float *)to_dev(S, sizeof(float) * HV * DK * DK);
  void *dKc = to_dev(Kc, (size_t)HKV * CAP * D * 2), *dVc = to_dev(Vc, (size_t)HKV * CAP * D * 2);
  hdt_layer_io io[2];
  io[0].q = to_dev(q, (size_t)N * HK * DK * 2);
  io[0].k = to_dev(k, (size_t)N * HK * DK * 2);
  io[0].v = to_dev(v, (size_t)N * HV * DK * 2);
  io[0].alpha = to_dev(a, (size_t)N * HV * 2);
  io[0].beta = to_dev(b, (size_t)N * HV * 2);
  CHECK_HIP(hipMalloc(&io[0].o, (size_t)N * HV * DK * 2));
  io[1].q = to_dev(aq, (size_t)N * HQ * D * 2);
  io[1].k = to_dev(ak, (size_t)N * HKV * D * 2);
  io[1].v = to_dev(av, (size_t)N * HKV * D * 2);
  io[1].alpha = io[1].beta = NULL;
  CHECK_HIP(hipMalloc(&io[1].o, (size_t)N * HQ * D * 2));

  const uint8_t kinds[2] = {0, 1};
  hdt_model_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.n_layers = 2;
  desc.layer_kind = kinds;
  desc.gdn_hk = HK, desc.gdn_hv = HV, desc.gdn_dk = DK, desc.gdn_dv = DK;
  desc.attn_hq = HQ, desc.attn_hkv = HKV, desc.attn_d = D;
  desc.io_dtype = HDT_BF16;
  desc.max_nodes = N;
  hdt_slot_desc slot;
  memset(&slot, 0, sizeof slot);
  slot.gdn_state = dS, slot.k_cache = dKc, slot.v_cache = dVc, slot.capacity = CAP, slot.length = L;
  hdt_engine *eng = NULL;
  if (hdt_create(&desc, 1, &slot, &eng) != HDT_OK) {
    fprintf(stderr, "hdt_create failed\n");
    return 4;
  }
  const hdt_tree tree = {0, N, parent, io};
  CHECK_HDT(eng, hdt_forward_tree(eng, 1, &tree, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  /* outputs against the oracle */
  uint16_t *go = (uint16_t *)malloc((size_t)N * HQ * D * 2);
  float *ref = (float *)malloc(sizeof(float) * N * HQ * D);
  CHECK_HIP(hipMemcpy(go, io[0].o, (size_t)N * HV * DK * 2, hipMemcpyDeviceToHost));
  orc_gdn_tree(DK, DK, HK, HV, N, parent, S, q, k, v, a, b, 1, (float)(1.0 / sqrt(DK)), ref, NULL);
  const double e_gdn = rel_err(go, 1, ref, (size_t)N * HV * DK);
  uint16_t *eager_gdn = (uint16_t *)malloc((size_t)N * HV * DK * 2);
  memcpy(eager_gdn, go, (size_t)N * HV * DK * 2);
  CHECK_HIP(hipMemcpy(go, io[1].o, (size_t)N * HQ * D * 2, hipMemcpyDeviceToHost));
  orc_attn_tree(HQ, HKV, D, N, parent, L, CAP, Kc, Vc, aq, ak, av, 1, 1.0f / 16.0f, ref);
  const double e_att = rel_err(go, 1, ref, (size_t)N * HQ * D);
  uint16_t *eager_att = (uint16_t *)malloc((size_t)N * HQ * D * 2);
  memcpy(eager_att, go, (size_t)N * HQ * D * 2);

  /* a state snapshot before the commit (restored at the end) */
  int64_t snap_bytes = 0;
  CHECK_HDT(eng, hdt_state_bytes(eng, &snap_bytes));
  void *snap = NULL;
  CHECK_HIP(hipMalloc(&snap, (size_t)snap_bytes));
  CHECK_HDT(eng, hdt_state_copy(eng, 0, snap, snap_bytes, 0, NULL));

  /* commit a root path: the state against the oracle's sequential recurrence, the cache
     rows bit for bit */
  CHECK_HDT(eng, hdt_commit_tree(eng, 0, path, 4, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  float *gS = (float *)malloc(sizeof(float) * HV * DK * DK);
  float *rS = (float *)malloc(sizeof(float) * HV * DK * DK);
  CHECK_HIP(hipMemcpy(gS, dS, sizeof(float) * HV * DK * DK, hipMemcpyDeviceToHost));
  orc_gdn_commit(DK, DK, HK, HV, 4, path, S, k, v, a, b, 1, rS);
  const double e_state = rel_err(gS, 0, rS, (size_t)HV * DK * DK);
  uint16_t *rows = (uint16_t *)malloc((size_t)HKV * CAP * D * 2);
  CHECK_HIP(hipMemcpy(rows, dKc, (size_t)HKV * CAP * D * 2, hipMemcpyDeviceToHost));
  int rows_ok = 1;
  for (int h = 0; h < HKV; ++h)
    for (int d = 0; d < 4; ++d)
      rows_ok &= memcmp(rows + ((size_t)h * CAP + L + d) * D, ak + ((size_t)path[d] * HKV + h) * D, D * 2) == 0;
  int64_t len = 0;
  CHECK_HDT(eng, hdt_kv_length(eng, 0, &len));

  /* restore the snapshot: the committed state before the round, bit for bit, at length L */
  CHECK_HDT(eng, hdt_state_copy(eng, 0, snap, snap_bytes, 1, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(gS, dS, sizeof(float) * HV * DK * DK, hipMemcpyDeviceToHost));
  int64_t len_back = 0;
  CHECK_HDT(eng, hdt_kv_length(eng, 0, &len_back));
  const int restored = memcmp(gS, S, sizeof(float) * HV * DK * DK) == 0 && len_back == L;
  CHECK_HIP(hipFree(snap));

  /* the same round through a reusable graph: the eager pass's bits; then dropped */
  hdt_graph *graph = NULL;
  CHECK_HDT(eng, hdt_graph_create(eng, &graph));
  CHECK_HIP(hipMemset(io[0].o, 0, (size_t)N * HV * DK * 2));
  CHECK_HIP(hipMemset(io[1].o, 0, (size_t)N * HQ * D * 2));
  CHECK_HDT(eng, hdt_graph_forward(graph, 1, &tree, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(go, io[0].o, (size_t)N * HV * DK * 2, hipMemcpyDeviceToHost));
  int graph_same = memcmp(go, eager_gdn, (size_t)N * HV * DK * 2) == 0;
  CHECK_HIP(hipMemcpy(go, io[1].o, (size_t)N * HQ * D * 2, hipMemcpyDeviceToHost));
  graph_same &= memcmp(go, eager_att, (size_t)N * HQ * D * 2) == 0;
  CHECK_HDT(eng, hdt_rollback_to(eng, 0, L, NULL));
  hdt_graph_destroy(graph);
  hdt_destroy(eng);

  printf("gdn output %.3e, attention output %.3e, committed state %.3e, rows %s, length %lld, "
         "snapshot restore %s, graph round %s\n",
         e_gdn, e_att, e_state, rows_ok ? "equal" : "DIFFER", (long long)len, restored ? "exact" : "WRONG",
         graph_same ? "equal" : "DIFFER");
  const int ok = e_gdn <= 2e-2 && e_att <= 2e-2 && e_state <= 2e-3 && rows_ok && len == L + 4 && restored &&
                 graph_same;
  printf("%s\n", ok ? "PASS" : "FAIL");
  return ok ? 0 : 1;
}
