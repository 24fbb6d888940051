/*
 * A plain C user of liblsh.so: only include/lsh.h and the HIP runtime API,
 * no C++ and no Python. With K = 0 every score is 0, so each query attends
 * all Skv keys with weight 1/Skv (the softmax of a constant row, "LLM Lab
 * Notes 05", sections 2-3): O = the mean of the head's V rows and
 * LSE = log(Skv). On the current GPU it checks:
 *  - lsh_attn_fwd on that closed form for bf16 and float32 inputs, on a
 *    stream of its own, in the [B, S, H, D] layout and with head-major
 *    strides (the same bits);
 *  - two lsh_attn_partial calls over a split of the keys merged by
 *    lsh_lse_merge, and the same blocks folded by
 *    lsh_attn_partial_accumulate (the first fold equal to the partial bit
 *    for bit): the closed form again;
 *  - lsh_head_permute moves every bf16 element where the header says;
 *  - lsh_attn_fwd_blocksparse_noalloc with an all-ones mask gives the
 *    dense call's bits;
 *  - lsh_attn_bwd on the closed form: dQ = scale dS K = 0 exactly, and
 *    dV_j = sum_i P_ij dO_i = (1/Skv) sum_i dO_i for every key j;
 *  - an unsupported head_dim is refused before any HIP call, with a
 *    message from lsh_last_error().
 * Exit status 0 when every check passes; the first failure is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lsh.h"

#define CHECK_HIP(x)                                                    \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), \
              __FILE__, __LINE__);                                      \
      exit(1);                                                          \
    }                                                                   \
  } while (0)

#define CHECK_LSH(x)                                                           \
  do {                                                                         \
    lsh_status s_ = (x);                                                       \
    if (s_ != LSH_OK) {                                                        \
      fprintf(stderr, "%s at line %d: %s: %s\n", #x, __LINE__, lsh_status_str(s_), \
              lsh_last_error());                                               \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

#define FAIL(...)                 \
  do {                            \
    fprintf(stderr, __VA_ARGS__); \
    fputc('\n', stderr);          \
    exit(1);                      \
  } while (0)

enum { B = 2, SQ = 300, SKV = 257, H = 3, D = LSH_HEAD_DIM, SPLIT = 128 };
static const size_t NQ = (size_t)B * SQ * H * D, NKV = (size_t)B * SKV * H * D,
                    NL = (size_t)B * H * SQ;

/* bf16 bits of a float that bf16 represents exactly */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

/* multiples of 1/8 in [-4, 4): exact in bf16 */
static float v_value(int b, int j, int h, int d) {
  return (float)(((b * 131 + j * 17 + h * 7 + d * 3) % 64) - 32) / 8.0f;
}
static float q_value(size_t i) { return (float)((int)(i % 29) - 14) / 4.0f; }
static float do_value(int b, int i, int h, int d) {
  return (float)(((b * 37 + i * 11 + h * 5 + d) % 32) - 16) / 16.0f;
}

static void put(unsigned char* buf, size_t i, float x, int dtype) {
  if (dtype == LSH_BF16) {
    const uint16_t w = to_bf16(x);
    memcpy(buf + 2 * i, &w, 2);
  } else {
    memcpy(buf + 4 * i, &x, 4);
  }
}

static void* dev_copy(const void* host, size_t bytes) {
  void* p;
  CHECK_HIP(hipMalloc(&p, bytes));
  CHECK_HIP(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
  return p;
}

/* the closed-form inputs: Q (irrelevant), K = 0, V; head_major selects the
   storage order [B, H, S, D] instead of [B, S, H, D] */
typedef struct {
  void *q, *k, *v;
  int dtype, head_major;
} inputs;

static inputs make_inputs(int dtype, int head_major) {
  const size_t eb = dtype == LSH_BF16 ? 2 : 4;
  unsigned char* hq = calloc(NQ, eb);
  unsigned char* hk = calloc(NKV, eb);
  unsigned char* hv = calloc(NKV, eb);
  if (!hq || !hk || !hv) FAIL("out of host memory");
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < SKV; ++s)
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
          const size_t i = head_major ? (((size_t)b * H + h) * SKV + s) * D + d
                                      : (((size_t)b * SKV + s) * H + h) * D + d;
          put(hv, i, v_value(b, s, h, d), dtype);
        }
  for (size_t i = 0; i < NQ; ++i) put(hq, i, q_value(i), dtype);
  inputs in = {dev_copy(hq, NQ * eb), dev_copy(hk, NKV * eb), dev_copy(hv, NKV * eb), dtype,
               head_major};
  free(hq);
  free(hk);
  free(hv);
  return in;
}

static lsh_attn_args make_args(const inputs* in, float* o, float* lse) {
  lsh_attn_args a;
  memset(&a, 0, sizeof(a));
  a.q = in->q;
  a.k = in->k;
  a.v = in->v;
  a.o = o;
  a.lse = lse;
  a.dtype = in->dtype;
  a.B = B;
  a.Sq = SQ;
  a.Skv = SKV;
  a.H = H;
  a.D = D;
  const int hm = in->head_major;
  const int64_t qs[3] = {hm ? (int64_t)H * SQ * D : (int64_t)SQ * H * D, hm ? D : (int64_t)H * D,
                         hm ? (int64_t)SQ * D : D};
  const int64_t ks[3] = {hm ? (int64_t)H * SKV * D : (int64_t)SKV * H * D,
                         hm ? D : (int64_t)H * D, hm ? (int64_t)SKV * D : D};
  const int64_t os[3] = {(int64_t)SQ * H * D, (int64_t)H * D, D};
  memcpy(a.q_stride, qs, sizeof(qs));
  memcpy(a.k_stride, ks, sizeof(ks));
  memcpy(a.v_stride, ks, sizeof(ks));
  memcpy(a.o_stride, os, sizeof(os));
  a.scale = 1.0f / sqrtf((float)D);
  return a;
}

static void* dmalloc(size_t bytes) {
  void* p;
  CHECK_HIP(hipMalloc(&p, bytes));
  return p;
}

static void* to_host(const void* dev, size_t bytes) {
  void* h = malloc(bytes);
  if (!h) FAIL("out of host memory");
  CHECK_HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  return h;
}

/* max |O - mean(V)| and max |LSE - log(Skv)| over all rows */
static void closed_form_errors(const float* o, const float* lse, double* eo, double* el) {
  *eo = 0.0;
  *el = 0.0;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        double mean = 0.0;
        for (int j = 0; j < SKV; ++j) mean += v_value(b, j, h, d);
        mean /= SKV;
        for (int i = 0; i < SQ; ++i) {
          const double e = fabs(o[(((size_t)b * SQ + i) * H + h) * D + d] - mean);
          if (e > *eo) *eo = e;
        }
      }
  for (size_t i = 0; i < NL; ++i) {
    const double e = fabs(lse[i] - log((double)SKV));
    if (e > *el) *el = e;
  }
}

static void expect_closed_form(const char* what, const float* o, const float* lse) {
  double eo, el;
  closed_form_errors(o, lse, &eo, &el);
  if (!(eo <= 1e-5 && el <= 1e-5))
    FAIL("%s: max |O - mean(V)| = %.3e, max |LSE - log(Skv)| = %.3e", what, eo, el);
  printf("%s: max |O - mean(V)| = %.3e, max |LSE - log(Skv)| = %.3e\n", what, eo, el);
}

int main(void) {
  if (lsh_abi_version() != LSH_ABI_VERSION)
    FAIL("ABI version %d, header %d", lsh_abi_version(), LSH_ABI_VERSION);
  CHECK_LSH(lsh_device_check());
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  float* o = dmalloc(NQ * 4);
  float* lse = dmalloc(NL * 4);
  float* o2 = dmalloc(NQ * 4);
  float* lse2 = dmalloc(NL * 4);

  /* forward: two dtypes, two layouts */
  const int dtypes[2] = {LSH_BF16, LSH_F32};
  for (int t = 0; t < 2; ++t) {
    inputs a_in = make_inputs(dtypes[t], 0), b_in = make_inputs(dtypes[t], 1);
    lsh_attn_args a = make_args(&a_in, o, lse), b = make_args(&b_in, o2, lse2);
    CHECK_LSH(lsh_attn_fwd(&a, (lsh_stream)s));
    CHECK_LSH(lsh_attn_fwd(&b, (lsh_stream)s));
    CHECK_HIP(hipStreamSynchronize(s));
    float *ho = to_host(o, NQ * 4), *hl = to_host(lse, NL * 4);
    float *ho2 = to_host(o2, NQ * 4), *hl2 = to_host(lse2, NL * 4);
    expect_closed_form(dtypes[t] == LSH_BF16 ? "fwd bf16" : "fwd f32", ho, hl);
    if (memcmp(ho, ho2, NQ * 4) || memcmp(hl, hl2, NL * 4))
      FAIL("dtype %d: head-major layout changed the result bits", dtypes[t]);
    free(ho), free(hl), free(ho2), free(hl2);
    CHECK_HIP(hipFree(a_in.q)); CHECK_HIP(hipFree(a_in.k)); CHECK_HIP(hipFree(a_in.v));
    CHECK_HIP(hipFree(b_in.q)); CHECK_HIP(hipFree(b_in.k)); CHECK_HIP(hipFree(b_in.v));
  }
  printf("fwd: layouts bit-identical\n");

  /* the bf16 [B, S, H, D] problem for the other entry points */
  inputs in = make_inputs(LSH_BF16, 0);
  lsh_attn_args full = make_args(&in, o, lse);
  CHECK_LSH(lsh_attn_fwd(&full, (lsh_stream)s));
  float *o_parts = dmalloc(2 * NQ * 4), *l_parts = dmalloc(2 * NL * 4);
  const int64_t block0[2] = {0, SPLIT}, blen[2] = {SPLIT, SKV - SPLIT};
  for (int p = 0; p < 2; ++p) {
    lsh_attn_args a = make_args(&in, o_parts + p * NQ, l_parts + p * NL);
    a.k = (const uint16_t*)in.k + block0[p] * H * D;
    a.v = (const uint16_t*)in.v + block0[p] * H * D;
    a.Skv = blen[p];
    CHECK_LSH(lsh_attn_partial(&a, (lsh_stream)s));
  }
  CHECK_LSH(lsh_lse_merge(o_parts, l_parts, 2, B, SQ, H, D, o2, lse2, (lsh_stream)s));
  CHECK_HIP(hipStreamSynchronize(s));
  {
    float *ho = to_host(o2, NQ * 4), *hl = to_host(lse2, NL * 4);
    expect_closed_form("partials + merge", ho, hl);
    free(ho), free(hl);
  }
  /* folded on arrival, into O = 0, LSE = -inf */
  {
    float* hz = calloc(NQ, 4);
    float* hinf = malloc(NL * 4);
    if (!hz || !hinf) FAIL("out of host memory");
    for (size_t i = 0; i < NL; ++i) hinf[i] = -INFINITY;
    CHECK_HIP(hipMemcpy(o2, hz, NQ * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(lse2, hinf, NL * 4, hipMemcpyHostToDevice));
    for (int p = 0; p < 2; ++p) {
      lsh_attn_args a = make_args(&in, o2, lse2);
      a.k = (const uint16_t*)in.k + block0[p] * H * D;
      a.v = (const uint16_t*)in.v + block0[p] * H * D;
      a.Skv = blen[p];
      CHECK_LSH(lsh_attn_partial_accumulate(&a, (lsh_stream)s));
      if (p == 0) {
        CHECK_HIP(hipStreamSynchronize(s));
        float *f = to_host(o2, NQ * 4), *fp = to_host(o_parts, NQ * 4);
        float *fl = to_host(lse2, NL * 4), *flp = to_host(l_parts, NL * 4);
        if (memcmp(f, fp, NQ * 4) || memcmp(fl, flp, NL * 4))
          FAIL("the first fold differs from lsh_attn_partial");
        free(f), free(fp), free(fl), free(flp);
      }
    }
    CHECK_HIP(hipStreamSynchronize(s));
    float *ho = to_host(o2, NQ * 4), *hl = to_host(lse2, NL * 4);
    expect_closed_form("folded on arrival", ho, hl);
    free(ho), free(hl), free(hz), free(hinf);
  }

  /* head permute of V, heads [1, 3) */
  {
    const int h0 = 1, hc = 2;
    uint16_t* dst = dmalloc((size_t)B * hc * SKV * D * 2);
    CHECK_LSH(lsh_head_permute(in.v, dst, LSH_BF16, B, SKV, H, D, h0, hc, (lsh_stream)s));
    CHECK_HIP(hipStreamSynchronize(s));
    uint16_t* hd = to_host(dst, (size_t)B * hc * SKV * D * 2);
    for (int b = 0; b < B; ++b)
      for (int h = h0; h < h0 + hc; ++h)
        for (int j = 0; j < SKV; ++j)
          for (int d = 0; d < D; ++d)
            if (hd[(((size_t)b * hc + (h - h0)) * SKV + j) * D + d] != to_bf16(v_value(b, j, h, d)))
              FAIL("permute: element (%d, %d, %d, %d) misplaced", b, j, h, d);
    printf("head permute: every element where the header says\n");
    free(hd);
    CHECK_HIP(hipFree(dst));
  }

  /* block-sparse, allocation-free, all-ones mask = dense bits */
  {
    const size_t nm = (size_t)B * H * ((SQ + 127) / 128) * ((SKV + 127) / 128);
    unsigned char* hm = malloc(nm);
    if (!hm) FAIL("out of host memory");
    memset(hm, 1, nm);
    unsigned char* dm = dev_copy(hm, nm);
    lsh_attn_args a = make_args(&in, o2, lse2);
    CHECK_LSH(lsh_attn_fwd_blocksparse_noalloc(&a, dm, (lsh_stream)s));
    CHECK_HIP(hipStreamSynchronize(s));
    float *d1 = to_host(o, NQ * 4), *d2 = to_host(o2, NQ * 4);
    float *l1 = to_host(lse, NL * 4), *l2 = to_host(lse2, NL * 4);
    if (memcmp(d1, d2, NQ * 4) || memcmp(l1, l2, NL * 4))
      FAIL("all-ones block-sparse differs from dense");
    printf("block-sparse (allocation-free), all-ones mask: the dense bits\n");
    free(d1), free(d2), free(l1), free(l2), free(hm);
    CHECK_HIP(hipFree(dm));
  }

  /* backward on the closed form */
  {
    uint16_t* hdo = malloc(NQ * 2);
    if (!hdo) FAIL("out of host memory");
    for (int b = 0; b < B; ++b)
      for (int i = 0; i < SQ; ++i)
        for (int h = 0; h < H; ++h)
          for (int d = 0; d < D; ++d)
            hdo[(((size_t)b * SQ + i) * H + h) * D + d] = to_bf16(do_value(b, i, h, d));
    void* ddo = dev_copy(hdo, NQ * 2);
    float *dq = dmalloc(NQ * 4), *dk = dmalloc(NKV * 4), *dv = dmalloc(NKV * 4);
    lsh_attn_bwd_args g;
    memset(&g, 0, sizeof(g));
    g.q = in.q;
    g.k = in.k;
    g.v = in.v;
    g.dout = ddo;
    g.o = o;
    g.lse = lse;
    g.dq = dq;
    g.dk = dk;
    g.dv = dv;
    g.dtype = LSH_BF16;
    g.B = B;
    g.Sq = SQ;
    g.Skv = SKV;
    g.H = H;
    g.D = D;
    memcpy(g.q_stride, full.q_stride, sizeof(g.q_stride));
    memcpy(g.k_stride, full.k_stride, sizeof(g.k_stride));
    memcpy(g.v_stride, full.v_stride, sizeof(g.v_stride));
    memcpy(g.do_stride, full.q_stride, sizeof(g.do_stride));
    memcpy(g.o_stride, full.o_stride, sizeof(g.o_stride));
    memcpy(g.dq_stride, full.o_stride, sizeof(g.dq_stride));
    const int64_t kvs[3] = {(int64_t)SKV * H * D, (int64_t)H * D, D};
    memcpy(g.dk_stride, kvs, sizeof(kvs));
    memcpy(g.dv_stride, kvs, sizeof(kvs));
    g.scale = full.scale;
    const size_t ws_bytes = lsh_attn_bwd_workspace(&g);
    if (ws_bytes == 0) FAIL("lsh_attn_bwd_workspace: %s", lsh_last_error());
    void* ws = dmalloc(ws_bytes);
    CHECK_LSH(lsh_attn_bwd(&g, ws, ws_bytes, (lsh_stream)s));
    CHECK_HIP(hipStreamSynchronize(s));
    float *hq = to_host(dq, NQ * 4), *hv = to_host(dv, NKV * 4);
    for (size_t i = 0; i < NQ; ++i)
      if (hq[i] != 0.0f) FAIL("dQ[%zu] = %g, not 0 (K = 0)", i, (double)hq[i]);
    double worst = 0.0, top = 0.0;
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
          double want = 0.0;
          for (int i = 0; i < SQ; ++i) want += do_value(b, i, h, d);
          want /= SKV;
          for (int j = 0; j < SKV; ++j) {
            const double got = hv[(((size_t)b * SKV + j) * H + h) * D + d];
            if (fabs(want) > top) top = fabs(want);
            if (fabs(got - want) > worst) worst = fabs(got - want);
          }
        }
    /* P = 1/Skv is rounded to bf16 before dV = P^T dO: relative 2^-9 */
    if (!(worst <= 4e-3 * top))
      FAIL("dV: max error %.3e against max |dV| %.3e", worst, top);
    printf("bwd: dQ = 0 exactly; dV = sum_i dO_i / Skv within %.2e of max |dV|\n", worst / top);
    free(hq), free(hv), free(hdo);
    CHECK_HIP(hipFree(ddo)); CHECK_HIP(hipFree(dq)); CHECK_HIP(hipFree(dk));
    CHECK_HIP(hipFree(dv)); CHECK_HIP(hipFree(ws));
  }

  /* refused before any HIP call */
  {
    lsh_attn_args bad = full;
    bad.D = 64;
    const lsh_status st = lsh_attn_fwd(&bad, NULL);
    if (st != LSH_ERR_UNSUPPORTED || lsh_last_error()[0] == '\0')
      FAIL("D = 64: status %d (%s)", (int)st, lsh_last_error());
    printf("D = 64 refused: %s\n", lsh_last_error());
  }

  CHECK_HIP(hipFree(in.q)); CHECK_HIP(hipFree(in.k)); CHECK_HIP(hipFree(in.v));
  CHECK_HIP(hipFree(o)); CHECK_HIP(hipFree(lse)); CHECK_HIP(hipFree(o2));
  CHECK_HIP(hipFree(lse2)); CHECK_HIP(hipFree(o_parts)); CHECK_HIP(hipFree(l_parts));
  CHECK_HIP(hipStreamDestroy(s));
  printf("c abi ok\n");
  return 0;
}
