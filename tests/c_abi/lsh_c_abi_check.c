/*
 * A plain C user of liblsh.so: only include/lsh.h and the HIP runtime API,
 * no C++ and no Python. It checks, on the current GPU:
 *  - lsh_attn_fwd on a closed form: with K = 0 every score is 0, so each
 *    query attends all Skv keys with weight 1/Skv (the softmax of a constant
 *    row, "LLM Lab Notes 05", sections 2-3): O = the mean of the head's V
 *    rows and LSE = log(Skv), for bf16 and float32 inputs, on a stream of
 *    its own;
 *  - the same call in a non-default layout (heads outermost, i.e. the
 *    strides of a [B, H, S, D] buffer) gives the same bits;
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

#define CHECK_HIP(x)                                                   \
  do {                                                                 \
    hipError_t e_ = (x);                                               \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), \
              __FILE__, __LINE__);                                     \
      return 1;                                                        \
    }                                                                  \
  } while (0)

enum { B = 2, SQ = 300, SKV = 257, H = 3, D = LSH_HEAD_DIM };

/* bf16 bits of a float that bf16 represents exactly */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}

/* value of V[b, j, h, d]: multiples of 1/8 in [-4, 4), exact in bf16 */
static float v_value(int b, int j, int h, int d) {
  return (float)(((b * 131 + j * 17 + h * 7 + d * 3) % 64) - 32) / 8.0f;
}

/* one forward with the given dtype and layout; returns 0 on success and
   fills o_host / lse_host */
static int run(int dtype, int head_major, float* o_host, float* lse_host) {
  const size_t n_q = (size_t)B * SQ * H * D, n_kv = (size_t)B * SKV * H * D;
  const size_t eb = dtype == LSH_BF16 ? 2 : 4;
  unsigned char* hq = calloc(n_q, eb);
  unsigned char* hk = calloc(n_kv, eb);
  unsigned char* hv = calloc(n_kv, eb);
  if (!hq || !hk || !hv) return 1;
  /* element (b, s, h, d) of an [B, S, H, D] or [B, H, S, D] buffer */
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < SKV; ++s)
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
          const size_t i = head_major ? (((size_t)b * H + h) * SKV + s) * D + d
                                      : (((size_t)b * SKV + s) * H + h) * D + d;
          const float x = v_value(b, s, h, d);
          if (dtype == LSH_BF16) {
            const uint16_t w = to_bf16(x);
            memcpy(hv + 2 * i, &w, 2);
          } else {
            memcpy(hv + 4 * i, &x, 4);
          }
        }
  for (size_t i = 0; i < n_q; ++i) {   /* Q is irrelevant when K = 0 */
    const float x = (float)((int)(i % 29) - 14) / 4.0f;
    if (dtype == LSH_BF16) {
      const uint16_t w = to_bf16(x);
      memcpy(hq + 2 * i, &w, 2);
    } else {
      memcpy(hq + 4 * i, &x, 4);
    }
  }
  void *dq, *dk, *dv;
  float *dout, *dlse;
  CHECK_HIP(hipMalloc(&dq, n_q * eb));
  CHECK_HIP(hipMalloc(&dk, n_kv * eb));
  CHECK_HIP(hipMalloc(&dv, n_kv * eb));
  CHECK_HIP(hipMalloc((void**)&dout, n_q * 4));
  CHECK_HIP(hipMalloc((void**)&dlse, (size_t)B * H * SQ * 4));
  CHECK_HIP(hipMemcpy(dq, hq, n_q * eb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, hk, n_kv * eb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, hv, n_kv * eb, hipMemcpyHostToDevice));

  lsh_attn_args a;
  memset(&a, 0, sizeof(a));
  a.q = dq;
  a.k = dk;
  a.v = dv;
  a.o = dout;
  a.lse = dlse;
  a.dtype = dtype;
  a.B = B;
  a.Sq = SQ;
  a.Skv = SKV;
  a.H = H;
  a.D = D;
  const int64_t sq_b = head_major ? (int64_t)H * SQ * D : (int64_t)SQ * H * D;
  const int64_t sq_s = head_major ? D : (int64_t)H * D;
  const int64_t sq_h = head_major ? (int64_t)SQ * D : D;
  const int64_t skv_b = head_major ? (int64_t)H * SKV * D : (int64_t)SKV * H * D;
  const int64_t skv_h = head_major ? (int64_t)SKV * D : D;
  const int64_t qs[3] = {sq_b, sq_s, sq_h}, ks[3] = {skv_b, sq_s, skv_h};
  const int64_t os[3] = {(int64_t)SQ * H * D, (int64_t)H * D, D};
  memcpy(a.q_stride, qs, sizeof(qs));
  memcpy(a.k_stride, ks, sizeof(ks));
  memcpy(a.v_stride, ks, sizeof(ks));
  memcpy(a.o_stride, os, sizeof(os));
  a.scale = 1.0f / sqrtf((float)D);

  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  const lsh_status st = lsh_attn_fwd(&a, (lsh_stream)s);
  if (st != LSH_OK) {
    fprintf(stderr, "lsh_attn_fwd: %s: %s\n", lsh_status_str(st), lsh_last_error());
    return 1;
  }
  CHECK_HIP(hipStreamSynchronize(s));
  CHECK_HIP(hipMemcpy(o_host, dout, n_q * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse_host, dlse, (size_t)B * H * SQ * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipStreamDestroy(s));
  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dlse));
  free(hq);
  free(hk);
  free(hv);
  return 0;
}

int main(void) {
  if (lsh_abi_version() != LSH_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", lsh_abi_version(), LSH_ABI_VERSION);
    return 1;
  }
  if (lsh_device_check() != LSH_OK) {
    fprintf(stderr, "no gfx950 device: %s\n", lsh_last_error());
    return 1;
  }
  const size_t n_q = (size_t)B * SQ * H * D;
  float* o = malloc(n_q * 4);
  float* o2 = malloc(n_q * 4);
  float* lse = malloc((size_t)B * H * SQ * 4);
  float* lse2 = malloc((size_t)B * H * SQ * 4);
  if (!o || !o2 || !lse || !lse2) return 1;
  const int dtypes[2] = {LSH_BF16, LSH_F32};
  for (int t = 0; t < 2; ++t) {
    if (run(dtypes[t], 0, o, lse) || run(dtypes[t], 1, o2, lse2)) return 1;
    double worst_o = 0.0, worst_l = 0.0;
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
          double mean = 0.0;
          for (int j = 0; j < SKV; ++j) mean += v_value(b, j, h, d);
          mean /= SKV;
          for (int i = 0; i < SQ; ++i) {
            const double e = fabs(o[(((size_t)b * SQ + i) * H + h) * D + d] - mean);
            if (e > worst_o) worst_o = e;
          }
        }
    for (size_t i = 0; i < (size_t)B * H * SQ; ++i) {
      const double e = fabs(lse[i] - log((double)SKV));
      if (e > worst_l) worst_l = e;
    }
    if (!(worst_o <= 1e-5 && worst_l <= 1e-5)) {
      fprintf(stderr, "dtype %d: max |O - mean(V)| = %.3e, max |LSE - log(Skv)| = %.3e\n",
              dtypes[t], worst_o, worst_l);
      return 1;
    }
    if (memcmp(o, o2, n_q * 4) != 0 || memcmp(lse, lse2, (size_t)B * H * SQ * 4) != 0) {
      fprintf(stderr, "dtype %d: head-major layout changed the result bits\n", dtypes[t]);
      return 1;
    }
    printf("dtype %d: max |O - mean(V)| = %.3e, max |LSE - log(Skv)| = %.3e, layouts bit-identical\n",
           dtypes[t], worst_o, worst_l);
  }
  /* refused before any HIP call */
  lsh_attn_args bad;
  memset(&bad, 0, sizeof(bad));
  bad.q = bad.k = bad.v = (const void*)(uintptr_t)4096;
  bad.o = bad.lse = (float*)(uintptr_t)4096;
  bad.dtype = LSH_BF16;
  bad.B = bad.Sq = bad.Skv = bad.H = 1;
  bad.D = 64;
  bad.scale = 1.0f;
  const lsh_status st = lsh_attn_fwd(&bad, NULL);
  if (st != LSH_ERR_UNSUPPORTED || lsh_last_error()[0] == '\0') {
    fprintf(stderr, "D = 64: status %d (%s)\n", (int)st, lsh_last_error());
    return 1;
  }
  printf("D = 64 refused: %s\n", lsh_last_error());
  free(o);
  free(o2);
  free(lse);
  free(lse2);
  printf("c abi ok\n");
  return 0;
}
