// Drives libsprint.so through its C ABI alone (hipMalloc'd buffers, no
// PyTorch, no Python), on cases whose results have closed forms:
//  - block attention over keys that are all the same vector: every query's
//    softmax is uniform, so O is the mean of the value rows;
//  - the LM-head confidence with an all-zero head: every logit is 0, so the
//    top-1 probability is 1/V and the argmax is the first token;
//  - one unmask step on a fully masked block with nothing above tau accepts
//    exactly ceil(m / steps_left) positions;
//  - the host keep counts floor(r * n), and NULL buffers are rejected.
// With --host-only it stops after the checks that need no GPU.
// Exit status 0 when every check holds.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sprint.h"

#define HIP_OK(x)                                                        \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
      exit(2);                                                           \
    }                                                                    \
  } while (0)

#define SPRINT_OK_(x)                                                    \
  do {                                                                   \
    int s_ = (x);                                                        \
    if (s_ != SPRINT_OK) {                                               \
      fprintf(stderr, "%s: %s\n", #x, sprint_strerror(s_));              \
      exit(3);                                                           \
    }                                                                    \
  } while (0)

static uint16_t to_bf16(float f) {   // exact for the values used here
  uint32_t u;
  memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int failures = 0;
static void check(bool ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(int argc, char** argv) {
  // ---------------------------------------------------------------- host
  check(sprint_keep_count(0.8, 3072) == 2457, "keep_count(0.8, 3072) == 2457");
  check(sprint_keep_count(1.0, 1024) == 1024, "keep_count(1.0, 1024) == 1024");
  check(block_attend(NULL, 1, 32, 8, NULL, NULL, NULL, 0, 0, NULL, NULL, 2, 128, 0.1f,
                     SPRINT_BF16, NULL, NULL, 0, NULL) == SPRINT_EINVAL,
        "NULL buffers are rejected before any HIP call");
  if (argc > 1 && strcmp(argv[1], "--host-only") == 0) {
    printf("%s\n", failures ? "FAILED" : "all checks passed");
    return failures ? 1 : 0;
  }

  // ---------------------------------------------------------------- attention
  const int nseq = 1, Lq = 32, Hq = 8, Hkv = 2, D = 128, L = 300;
  const size_t q_n = (size_t)nseq * Lq * Hq * D, kv_n = (size_t)L * Hkv * D;
  const size_t b_n = (size_t)nseq * Lq * Hkv * D;
  uint16_t* hq = (uint16_t*)malloc(q_n * 2);
  uint16_t* hk = (uint16_t*)malloc(kv_n * 2);
  uint16_t* hv = (uint16_t*)malloc(kv_n * 2);
  uint16_t* hkb = (uint16_t*)malloc(b_n * 2);
  uint16_t* hvb = (uint16_t*)malloc(b_n * 2);
  srand(7);
  for (size_t i = 0; i < q_n; ++i) hq[i] = to_bf16((float)((rand() % 17) - 8) / 8.f);
  // every key (prefix and block) is the same vector per KV head
  for (size_t i = 0; i < kv_n; ++i) hk[i] = to_bf16((float)((i % D) % 5) / 4.f);
  for (size_t i = 0; i < b_n; ++i) hkb[i] = to_bf16((float)((i % D) % 5) / 4.f);
  for (size_t i = 0; i < kv_n; ++i) hv[i] = to_bf16((float)((rand() % 33) - 16) / 16.f);
  for (size_t i = 0; i < b_n; ++i) hvb[i] = to_bf16((float)((rand() % 33) - 16) / 16.f);
  int32_t hcu[2] = {0, L};
  void *dq, *dk, *dv, *dkb, *dvb, *dO, *dws;
  int32_t* dcu;
  HIP_OK(hipMalloc(&dq, q_n * 2));
  HIP_OK(hipMalloc(&dk, kv_n * 2));
  HIP_OK(hipMalloc(&dv, kv_n * 2));
  HIP_OK(hipMalloc(&dkb, b_n * 2));
  HIP_OK(hipMalloc(&dvb, b_n * 2));
  HIP_OK(hipMalloc(&dO, q_n * 2));
  HIP_OK(hipMalloc((void**)&dcu, sizeof(hcu)));
  HIP_OK(hipMemcpy(dq, hq, q_n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, kv_n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, kv_n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dkb, hkb, b_n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dvb, hvb, b_n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dcu, hcu, sizeof(hcu), hipMemcpyHostToDevice));
  const size_t ws_a = block_attend_ws(nseq, Lq, Hq, Hkv, D, L, 1);
  HIP_OK(hipMalloc(&dws, ws_a > 256 ? ws_a : 256));
  SPRINT_OK_(block_attend(dq, nseq, Lq, Hq, dk, dv, dcu, L, L, dkb, dvb, Hkv, D,
                          1.f / sqrtf((float)D), SPRINT_BF16, dO, dws, ws_a, NULL));
  HIP_OK(hipDeviceSynchronize());
  uint16_t* ho = (uint16_t*)malloc(q_n * 2);
  HIP_OK(hipMemcpy(ho, dO, q_n * 2, hipMemcpyDeviceToHost));
  double max_err = 0.0;
  for (int i = 0; i < Lq; ++i)
    for (int h = 0; h < Hq; ++h) {
      const int g = h * Hkv / Hq;
      for (int d = 0; d < D; ++d) {
        double mean = 0.0;
        for (int j = 0; j < L; ++j) mean += from_bf16(hv[((size_t)j * Hkv + g) * D + d]);
        for (int j = 0; j < Lq; ++j) mean += from_bf16(hvb[((size_t)j * Hkv + g) * D + d]);
        mean /= (L + Lq);
        const double got = from_bf16(ho[(((size_t)i * Hq) + h) * D + d]);
        const double err = fabs(got - mean);
        if (err > max_err) max_err = err;
      }
    }
  printf("     attention max |O - mean(V)| = %.3g\n", max_err);
  check(max_err <= 2e-2, "attention over identical keys gives the mean of V");

  // ---------------------------------------------------------------- LM head
  const int M = 32, H = 2048, V = 1000;
  void *dx, *dw, *dws2;
  float* dconf;
  int32_t* darg;
  HIP_OK(hipMalloc(&dx, (size_t)M * H * 2));
  HIP_OK(hipMalloc(&dw, (size_t)V * H * 2));
  HIP_OK(hipMemset(dx, 0x3f, (size_t)M * H * 2));   // any finite hidden states
  HIP_OK(hipMemset(dw, 0, (size_t)V * H * 2));
  HIP_OK(hipMalloc((void**)&dconf, M * 4));
  HIP_OK(hipMalloc((void**)&darg, M * 4));
  const size_t ws_l = lmhead_confidence_ws(M, H, V, SPRINT_BF16);
  HIP_OK(hipMalloc(&dws2, ws_l));
  SPRINT_OK_(lmhead_confidence(dx, M, H, dw, V, SPRINT_BF16, dconf, darg, NULL, dws2, ws_l, NULL));
  HIP_OK(hipDeviceSynchronize());
  float hconf[M];
  int32_t harg[M];
  HIP_OK(hipMemcpy(hconf, dconf, sizeof(hconf), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(harg, darg, sizeof(harg), hipMemcpyDeviceToHost));
  bool lm_ok = true;
  for (int i = 0; i < M; ++i) lm_ok = lm_ok && fabsf(hconf[i] - 1.f / V) <= 1e-6f && harg[i] == 0;
  check(lm_ok, "zero LM head: confidence 1/V, argmax 0");

  // ---------------------------------------------------------------- unmask
  uint8_t* dmask;
  int32_t *dtok, *dacc;
  HIP_OK(hipMalloc((void**)&dmask, M));
  HIP_OK(hipMalloc((void**)&dtok, M * 4));
  HIP_OK(hipMalloc((void**)&dacc, 4));
  HIP_OK(hipMemset(dmask, 1, M));
  HIP_OK(hipMemset(dtok, 0xff, M * 4));
  SPRINT_OK_(unmask_select(dconf, darg, 1, M, 0.95f, 9, dmask, dtok, dacc, NULL));
  HIP_OK(hipDeviceSynchronize());
  uint8_t hmask[M];
  int32_t hacc;
  HIP_OK(hipMemcpy(hmask, dmask, M, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&hacc, dacc, 4, hipMemcpyDeviceToHost));
  int still = 0;
  for (int i = 0; i < M; ++i) still += hmask[i];
  check(hacc == 4 && still == M - 4, "unmask accepts ceil(32 / 9) = 4 positions");

  // ---------------------------------------------------------------- both, in one call
  void* dws3;
  const size_t ws_f = lmhead_confidence_unmask_ws(1, M, H, V, SPRINT_BF16);
  HIP_OK(hipMalloc(&dws3, ws_f));
  HIP_OK(hipMemset(dws3, 0x5a, ws_f));   // the call sets what it needs
  HIP_OK(hipMemset(dmask, 1, M));
  HIP_OK(hipMemset(dtok, 0xff, M * 4));
  HIP_OK(hipMemset(dconf, 0, M * 4));
  SPRINT_OK_(lmhead_confidence_unmask(dx, 1, M, H, dw, V, SPRINT_BF16, dconf, darg, 0.95f, 9, dmask,
                                      dtok, dacc, dws3, ws_f, NULL));
  HIP_OK(hipDeviceSynchronize());
  int32_t htok[M];
  HIP_OK(hipMemcpy(hconf, dconf, sizeof(hconf), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hmask, dmask, M, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(htok, dtok, sizeof(htok), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&hacc, dacc, 4, hipMemcpyDeviceToHost));
  bool f_ok = hacc == 4;
  int accepted = 0;
  for (int i = 0; i < M; ++i) {
    f_ok = f_ok && fabsf(hconf[i] - 1.f / V) <= 1e-6f;
    if (hmask[i] == 0) {
      ++accepted;
      f_ok = f_ok && htok[i] == 0;
    } else {
      f_ok = f_ok && htok[i] == -1;
    }
  }
  check(f_ok && accepted == 4,
        "LM head and unmask in one call: confidence 1/V, 4 positions take token 0");
  HIP_OK(hipFree(dws3));

  // ---------------------------------------------------------------- errors
  check(block_attend(dq, nseq, Lq, Hq, dk, dv, dcu, L, L, dkb, dvb, 3, D, 0.1f, SPRINT_BF16, dO,
                     dws, ws_a, NULL) == SPRINT_EINVAL,
        "Hq % Hkv != 0 is rejected before any launch");

  void* bufs[] = {dq, dk, dv, dkb, dvb, dO, dcu, dws, dx, dw, dws2, dconf, darg, dmask, dtok, dacc};
  for (void* b : bufs) HIP_OK(hipFree(b));
  free(hq); free(hk); free(hv); free(hkb); free(hvb); free(ho);
  printf("%s\n", failures ? "FAILED" : "all checks passed");
  return failures ? 1 : 0;
}
