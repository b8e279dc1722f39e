/* A plain C program that uses libccr through its C ABI alone (no Python, no
 * PyTorch: HIP's own runtime from ROCm), checked bit for bit against the C
 * oracle: ring all-reduce, reduce-scatter then all-gather, the staged ring
 * shift and the uniform element all-to-all, on one stream of its own, over
 * ragged sizes, both element types and the copy modes.  Test infrastructure:
 * prints one line per case and "c consumer: ok" at the end; exit status 0
 * only if every case matched. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ccr.h"

/* the oracle's entry points (oracle/ccr_oracle.c) */
int orc_ring_allreduce(void *const *b, float *const *part, int R, int64_t n, int S, int dtype);
int orc_ring_reduce_scatter(void *const *b, float *const *part, int R, int64_t n, int S, int dtype);
int orc_ring_all_gather(void *const *b, int R, int64_t n, int S, int esize);
int orc_alltoall(const void *const *send, void *const *recv, int R, const int64_t *counts,
                 int64_t row_bytes);
void orc_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n);

#define MAXR 16

static int failures = 0;

#define HIPCK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_));   \
      exit(2);                                                                            \
    }                                                                                     \
  } while (0)

#define CCRCK(x)                                                                          \
  do {                                                                                    \
    ccr_status_t s_ = (x);                                                                \
    if (s_ != CCR_OK) {                                                                   \
      fprintf(stderr, "%s:%d %s: status %d: %s\n", __FILE__, __LINE__, #x, (int)s_,       \
              ccr_last_error());                                                          \
      exit(2);                                                                            \
    }                                                                                     \
  } while (0)

/* xorshift64: deterministic inputs, values in [-1, 1) */
static uint64_t rng_state;
static float next_value(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (float)((rng_state >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}

static void fill(void *host, int64_t n, int dtype) {
  if (dtype == CCR_F32) {
    float *f = (float *)host;
    for (int64_t i = 0; i < n; i++) f[i] = next_value();
  } else {
    float *tmp = (float *)malloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; i++) tmp[i] = next_value();
    orc_f32_to_bf16_array(tmp, (uint16_t *)host, n);
    free(tmp);
  }
}

static void report(const char *what, int ok) {
  printf("%s: %s\n", what, ok ? "ok" : "DIFFERS");
  if (!ok) failures++;
}

/* op: 0 all-reduce, 1 reduce-scatter then all-gather */
static void ring_case(ccr_ctx_t ctx, hipStream_t st, int R, int64_t n, int dtype, int op,
                      const char *mode) {
  const int esize = dtype == CCR_F32 ? 4 : 2;
  const size_t bytes = (size_t)n * esize;
  void *host[MAXR], *ref[MAXR], *dev[MAXR];
  rng_state = 0x9E3779B97F4A7C15ull ^ (uint64_t)(R * 1000003 + n * 7 + dtype);
  for (int r = 0; r < R; r++) {
    host[r] = malloc(bytes ? bytes : 1);
    ref[r] = malloc(bytes ? bytes : 1);
    fill(host[r], n, dtype);
    memcpy(ref[r], host[r], bytes);
    HIPCK(hipMalloc(&dev[r], bytes ? bytes : 16));
    HIPCK(hipMemcpy(dev[r], host[r], bytes, hipMemcpyHostToDevice));
  }
  if (op == 0) {
    CCRCK(ccr_allreduce(ctx, dev, R, n, dtype, st));
    if (orc_ring_allreduce(ref, NULL, R, n, 1, dtype) != 0) exit(3);
  } else {
    CCRCK(ccr_reduce_scatter(ctx, dev, R, n, dtype, st));
    CCRCK(ccr_all_gather(ctx, dev, R, n, dtype, st));
    if (orc_ring_reduce_scatter(ref, NULL, R, n, 1, dtype) != 0) exit(3);
    if (orc_ring_all_gather(ref, R, n, 1, esize) != 0) exit(3);
  }
  HIPCK(hipStreamSynchronize(st));
  int ok = 1;
  for (int r = 0; r < R; r++) {
    HIPCK(hipMemcpy(host[r], dev[r], bytes, hipMemcpyDeviceToHost));
    if (memcmp(host[r], ref[r], bytes) != 0) ok = 0;
    HIPCK(hipFree(dev[r]));
    free(host[r]);
    free(ref[r]);
  }
  char what[160];
  snprintf(what, sizeof what, "%s R=%d n=%lld %s %s", op == 0 ? "allreduce" : "reduce_scatter+all_gather", R,
           (long long)n, dtype == CCR_F32 ? "f32" : "bf16", mode);
  report(what, ok);
}

/* the ring shift: recv[(r + 1) % R] <- send[r] */
static void shift_case(ccr_ctx_t ctx, hipStream_t st, int R, int64_t count, const char *mode) {
  const size_t bytes = (size_t)count * 4;
  void *host[MAXR], *dsend[MAXR], *drecv[MAXR];
  rng_state = 0x1234567ull + (uint64_t)count;
  for (int r = 0; r < R; r++) {
    host[r] = malloc(bytes);
    fill(host[r], count, CCR_F32);
    HIPCK(hipMalloc(&dsend[r], bytes));
    HIPCK(hipMalloc(&drecv[r], bytes));
    HIPCK(hipMemcpy(dsend[r], host[r], bytes, hipMemcpyHostToDevice));
    HIPCK(hipMemset(drecv[r], 0, bytes));
  }
  CCRCK(ccr_sendrecv(ctx, (const void *const *)dsend, drecv, R, count, CCR_F32, st));
  HIPCK(hipStreamSynchronize(st));
  int ok = 1;
  void *got = malloc(bytes);
  for (int r = 0; r < R; r++) {
    HIPCK(hipMemcpy(got, drecv[(r + 1) % R], bytes, hipMemcpyDeviceToHost));
    if (memcmp(got, host[r], bytes) != 0) ok = 0;
  }
  free(got);
  for (int r = 0; r < R; r++) {
    HIPCK(hipFree(dsend[r]));
    HIPCK(hipFree(drecv[r]));
    free(host[r]);
  }
  char what[120];
  snprintf(what, sizeof what, "sendrecv ring shift R=%d count=%lld %s", R, (long long)count, mode);
  report(what, ok);
}

/* the uniform element all-to-all (counts NULL), against the oracle's rows */
static void alltoall_case(ccr_ctx_t ctx, hipStream_t st, int R, int64_t count, const char *mode) {
  const size_t bytes = (size_t)count * 2;
  void *hsend[MAXR], *href[MAXR], *dsend[MAXR], *drecv[MAXR];
  int64_t counts[MAXR * MAXR];
  rng_state = 0xABCDEFull + (uint64_t)count;
  for (int r = 0; r < R; r++) {
    hsend[r] = malloc(bytes);
    href[r] = malloc(bytes);
    fill(hsend[r], count, CCR_BF16);
    HIPCK(hipMalloc(&dsend[r], bytes));
    HIPCK(hipMalloc(&drecv[r], bytes));
    HIPCK(hipMemcpy(dsend[r], hsend[r], bytes, hipMemcpyHostToDevice));
    for (int d = 0; d < R; d++) counts[r * R + d] = count / R;  /* elements, one 2-byte row each */
  }
  CCRCK(ccr_alltoall(ctx, (const void *const *)dsend, drecv, R, count, NULL, CCR_BF16, st));
  if (orc_alltoall((const void *const *)hsend, href, R, counts, 2) != 0) exit(3);
  HIPCK(hipStreamSynchronize(st));
  int ok = 1;
  void *got = malloc(bytes);
  for (int d = 0; d < R; d++) {
    HIPCK(hipMemcpy(got, drecv[d], bytes, hipMemcpyDeviceToHost));
    if (memcmp(got, href[d], bytes) != 0) ok = 0;
  }
  free(got);
  for (int r = 0; r < R; r++) {
    HIPCK(hipFree(dsend[r]));
    HIPCK(hipFree(drecv[r]));
    free(hsend[r]);
    free(href[r]);
  }
  char what[120];
  snprintf(what, sizeof what, "alltoall uniform R=%d count=%lld bf16 %s", R, (long long)count, mode);
  report(what, ok);
}

int main(void) {
  printf("c consumer: libccr %s\n", ccr_version());
  fflush(stdout);
  hipStream_t st;
  HIPCK(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
  for (int copy_mode = CCR_COPY_KERNEL; copy_mode <= CCR_COPY_SDMA; copy_mode++) {
    const char *mode = copy_mode == CCR_COPY_SDMA ? "sdma" : "kernel";
    ccr_config_t cfg;
    CCRCK(ccr_config_default(&cfg));
    cfg.copy_mode = copy_mode;
    cfg.staging_chunk_bytes = 1 << 16;
    cfg.staging_slots = 3;
    ccr_ctx_t ctx;
    CCRCK(ccr_ctx_create(0, &cfg, &ctx));
    static const struct { int R; int64_t n; } cases[] = {{2, 1}, {3, 1001}, {4, 3 * 4096 + 5}, {8, 65536 + 9},
                                                          {16, 100003}};
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; i++)
      for (int dtype = CCR_F32; dtype <= CCR_BF16; dtype++)
        for (int op = 0; op <= 1; op++) ring_case(ctx, st, cases[i].R, cases[i].n, dtype, op, mode);
    shift_case(ctx, st, 4, 100000, mode);
    alltoall_case(ctx, st, 8, 8 * 8 * 1000, mode);
    fflush(stdout);
    CCRCK(ccr_ctx_destroy(ctx));
  }
  HIPCK(hipStreamDestroy(st));
  if (failures) {
    printf("c consumer: %d case(s) differ\n", failures);
    return 1;
  }
  printf("c consumer: ok\n");
  return 0;
}
