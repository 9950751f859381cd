/*
 * Round trip through libsplitzip's C ABI from plain C: device buffers from
 * hipMalloc, the default stream, no Python and no PyTorch.  For BF16 and FP8
 * E5M2 inputs with a concentrated exponent distribution (some escapes) it
 * checks that
 *   - the stream size equals the closed form stated in splitzip.h for the
 *     escape count found on the host (elements whose exponent is not in the
 *     codebook), and the header carries n, E and S;
 *   - the decoded tensor equals the input byte for byte, with d_status OK;
 *   - a stream with a damaged magic number sets d_status to E_CORRUPT;
 *   - host-detectable errors (small output, null input, bad codebook) return
 *     their codes;
 *   - splitzip_compress_static, the entry point that allocates nothing,
 *     writes the same stream byte for byte into a buffer with no room for a
 *     workspace, on two calls in a row.
 * Then, on BF16 data, the other entry points from plain C: the device
 * calibration equals the host one, both ablation variants round-trip, and
 * the chunk-pipelined transfer through pinned host memory (four streams)
 * delivers the input with fewer bytes over the link than raw.
 * Exit status 0 when every check holds.  Test infrastructure only.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "splitzip.h"

#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);               \
      fprintf(stderr, "\n");                      \
      exit(1);                                    \
    }                                             \
  } while (0)

#define HIP(call) CHECK((call) == hipSuccess, "%s", #call)

/* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", 2014) */
static uint64_t rng = 0x2545F4914F6CDD1Dull;
static uint64_t next64(void) {
  uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t a256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

static uint64_t rd64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
  return v;
}

static void run(int dtype, size_t n) {
  const int bf16 = dtype == SPLITZIP_BF16;
  const size_t elem = bf16 ? 2 : 1;
  uint8_t* x = (uint8_t*)malloc(n * elem);
  CHECK(x != NULL, "malloc");
  for (size_t i = 0; i < n; ++i) {
    const uint64_t r = next64();
    /* exponent: a binomial around the middle of the range; sign and mantissa uniform */
    if (bf16) {
      const uint32_t e = 110 + (uint32_t)__builtin_popcountll(r & 0xFFFFFF);
      const uint16_t v = (uint16_t)(((r >> 32) & 0x807F) | (e << 7));
      memcpy(x + 2 * i, &v, 2);
    } else {
      const uint32_t e = 4 + (uint32_t)__builtin_popcountll(r & 0xFFFFFF);
      x[i] = (uint8_t)(((r >> 32) & 0x83) | (e << 2));
    }
  }
  uint8_t cb[16];
  CHECK(splitzip_calibrate(dtype, x, n / 4, cb) == SPLITZIP_OK, "calibrate");
  /* escapes counted on the host */
  uint64_t E = 0;
  for (size_t i = 0; i < n; ++i) {
    const uint32_t e = bf16 ? (uint32_t)((x[2 * i] | (x[2 * i + 1] << 8)) >> 7) & 0xFF : (uint32_t)(x[i] >> 2) & 0x1F;
    int in = 0;
    for (int k = 0; k < 16; ++k) in |= cb[k] == e;
    E += !in;
  }
  /* closed-form stream size (layout in splitzip.h) */
  const uint64_t C = (n + 65535) / 65536;
  const uint64_t N0 = a256(64 + 16 + 8 * (C + 1));
  const uint64_t N1 = N0 + a256((n + 1) / 2);
  const uint64_t sm = bf16 ? n : 3 * ((n + 7) / 8);
  const uint64_t S_want = N1 + a256(sm) + 3 * E;

  const size_t cap = splitzip_max_compressed_size(dtype, n, 1);
  CHECK(cap >= S_want, "max size %zu < %llu", cap, (unsigned long long)S_want);
  void *d_in, *d_out, *d_y;
  uint64_t* d_bytes;
  int32_t* d_status;
  HIP(hipMalloc(&d_in, n * elem));
  HIP(hipMalloc(&d_out, cap));
  HIP(hipMalloc(&d_y, n * elem));
  HIP(hipMalloc((void**)&d_bytes, 8));
  HIP(hipMalloc((void**)&d_status, 4));
  HIP(hipMemcpy(d_in, x, n * elem, hipMemcpyHostToDevice));
  HIP(hipMemset(d_status, 0, 4));

  CHECK(splitzip_compress(dtype, d_in, n, cb, 1, 0, d_out, cap, d_bytes, NULL) == SPLITZIP_OK, "compress");
  uint64_t S = 0;
  HIP(hipMemcpy(&S, d_bytes, 8, hipMemcpyDeviceToHost));
  CHECK(S == S_want, "stream size %llu, closed form %llu", (unsigned long long)S, (unsigned long long)S_want);
  uint8_t hdr[64];
  HIP(hipMemcpy(hdr, d_out, 64, hipMemcpyDeviceToHost));
  CHECK(rd64(hdr + 8) == n && rd64(hdr + 16) == E && rd64(hdr + 24) == S, "header n/E/S");

  /* the same stream from the entry point that allocates nothing, into a
   * buffer of exactly the largest stream's size (its workspace is the
   * library's own), twice in a row */
  {
    const uint64_t C1 = (n + 65535) / 65536;
    const uint64_t P = a256(64 + 16 + 8 * (C1 + 1)) + a256((n + 1) / 2) + a256(sm);
    const size_t cap_s = (size_t)a256(P + 3 * (uint64_t)n);
    void* d_s;
    uint64_t* d_sbytes;
    HIP(hipMalloc(&d_s, cap_s));
    HIP(hipMalloc((void**)&d_sbytes, 8));
    uint8_t* a = (uint8_t*)malloc(S);
    uint8_t* b = (uint8_t*)malloc(S);
    CHECK(a != NULL && b != NULL, "malloc");
    HIP(hipMemcpy(a, d_out, S, hipMemcpyDeviceToHost));
    for (int call = 0; call < 2; ++call) {
      HIP(hipMemset(d_s, 0xA5, cap_s));
      CHECK(splitzip_compress_static(dtype, d_in, n, cb, 1, 0, d_s, cap_s, d_sbytes, NULL) == SPLITZIP_OK,
            "compress_static (call %d)", call);
      uint64_t Ss = 0;
      HIP(hipMemcpy(&Ss, d_sbytes, 8, hipMemcpyDeviceToHost));
      CHECK(Ss == S, "static stream size %llu, splitzip_compress %llu", (unsigned long long)Ss,
            (unsigned long long)S);
      HIP(hipMemcpy(b, d_s, S, hipMemcpyDeviceToHost));
      CHECK(memcmp(a, b, S) == 0, "static stream differs from splitzip_compress's (call %d)", call);
    }
    CHECK(splitzip_compress_static(dtype, d_in, n, cb, 1, 0, d_s, cap_s - 1, d_sbytes, NULL) ==
              SPLITZIP_E_CAPACITY, "static: small output");
    HIP(hipDeviceSynchronize());
    free(a);
    free(b);
    HIP(hipFree(d_s));
    HIP(hipFree(d_sbytes));
  }

  CHECK(splitzip_decompress(d_out, S, dtype, n, d_y, d_status, NULL) == SPLITZIP_OK, "decompress");
  uint8_t* y = (uint8_t*)malloc(n * elem);
  CHECK(y != NULL, "malloc");
  int32_t status = -1;
  HIP(hipMemcpy(y, d_y, n * elem, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
  CHECK(status == SPLITZIP_OK, "d_status %d after a valid stream", status);
  CHECK(memcmp(x, y, n * elem) == 0, "round trip differs");

  /* a damaged magic number is reported through d_status */
  const uint8_t bad = 0x00;
  HIP(hipMemcpy(d_out, &bad, 1, hipMemcpyHostToDevice));
  CHECK(splitzip_decompress(d_out, S, dtype, n, d_y, d_status, NULL) == SPLITZIP_OK, "decompress (damaged)");
  HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
  CHECK(status == SPLITZIP_E_CORRUPT, "d_status %d after a damaged stream", status);

  /* host-detectable errors */
  CHECK(splitzip_compress(dtype, d_in, n, cb, 1, 0, d_out, cap - 1, d_bytes, NULL) == SPLITZIP_E_CAPACITY,
        "small output");
  CHECK(splitzip_compress(dtype, NULL, n, cb, 1, 0, d_out, cap, d_bytes, NULL) == SPLITZIP_E_INVALID, "null input");
  uint8_t dup[16];
  memcpy(dup, cb, 16);
  dup[1] = dup[0];
  CHECK(splitzip_compress(dtype, d_in, n, dup, 1, 0, d_out, cap, d_bytes, NULL) == SPLITZIP_E_CODEBOOK,
        "repeated codebook entry");
  HIP(hipDeviceSynchronize());

  printf("c-abi ok: dtype=%d n=%zu escapes=%llu stream=%llu B ratio=%.4f\n", dtype, n, (unsigned long long)E,
         (unsigned long long)S, (double)(n * elem) / (double)S);
  fflush(stdout);
  HIP(hipFree(d_in));
  HIP(hipFree(d_out));
  HIP(hipFree(d_y));
  HIP(hipFree(d_bytes));
  HIP(hipFree(d_status));
  free(x);
  free(y);
}

/* BF16 values with a concentrated exponent distribution (as run()) */
static uint16_t* bf16_data(size_t n) {
  uint16_t* x = (uint16_t*)malloc(n * 2);
  CHECK(x != NULL, "malloc");
  for (size_t i = 0; i < n; ++i) {
    const uint64_t r = next64();
    const uint32_t e = 110 + (uint32_t)__builtin_popcountll(r & 0xFFFFFF);
    x[i] = (uint16_t)(((r >> 32) & 0x807F) | (e << 7));
  }
  return x;
}

static void extras(void) {
  const size_t n = 5 * 65536 + 777;
  uint16_t* x = bf16_data(n);
  uint16_t* y = (uint16_t*)malloc(n * 2);
  CHECK(y != NULL, "malloc");
  void *d_in, *d_y;
  int32_t* d_status;
  uint64_t* d_bytes;
  HIP(hipMalloc(&d_in, n * 2));
  HIP(hipMalloc(&d_y, n * 2));
  HIP(hipMalloc((void**)&d_status, 4));
  HIP(hipMalloc((void**)&d_bytes, 8));
  HIP(hipMemcpy(d_in, x, n * 2, hipMemcpyHostToDevice));

  /* device calibration of the whole tensor equals the host routine */
  uint8_t cb[16], cb_dev[16];
  CHECK(splitzip_calibrate(SPLITZIP_BF16, x, n, cb) == SPLITZIP_OK, "calibrate");
  const size_t work_bytes = splitzip_calibrate_device_work_bytes(SPLITZIP_BF16, 1);
  CHECK(work_bytes > 0, "calibrate work bytes");
  void* d_work;
  uint8_t* d_cb;
  HIP(hipMalloc(&d_work, work_bytes));
  HIP(hipMalloc((void**)&d_cb, 16));
  CHECK(splitzip_calibrate_device(SPLITZIP_BF16, d_in, n, 0, 1, d_cb, d_work, work_bytes, NULL) == SPLITZIP_OK,
        "calibrate_device");
  HIP(hipMemcpy(cb_dev, d_cb, 16, hipMemcpyDeviceToHost));
  CHECK(memcmp(cb, cb_dev, 16) == 0, "device codebook differs from the host one");
  HIP(hipFree(d_work));
  HIP(hipFree(d_cb));

  /* both ablation variants round-trip */
  const int variants[2] = {SPLITZIP_VARIANT_TOP15_SENTINEL, SPLITZIP_VARIANT_TOP8};
  for (int v = 0; v < 2; ++v) {
    const size_t cap = splitzip_variant_max_compressed_size(variants[v], n, 1);
    CHECK(cap > 0, "variant max size");
    void* d_out;
    HIP(hipMalloc(&d_out, cap));
    HIP(hipMemset(d_status, 0, 4));
    CHECK(splitzip_variant_compress(variants[v], d_in, n, cb, 1, 0, d_out, cap, d_bytes, NULL) == SPLITZIP_OK,
          "variant compress");
    uint64_t S = 0;
    HIP(hipMemcpy(&S, d_bytes, 8, hipMemcpyDeviceToHost));
    CHECK(S > 0 && S <= cap, "variant stream size %llu", (unsigned long long)S);
    CHECK(splitzip_variant_decompress(variants[v], d_out, S, n, d_y, d_status, NULL) == SPLITZIP_OK,
          "variant decompress");
    int32_t status = -1;
    HIP(hipMemcpy(y, d_y, n * 2, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
    CHECK(status == SPLITZIP_OK && memcmp(x, y, n * 2) == 0, "variant %d round trip", variants[v]);
    printf("c-abi ok: variant=%d n=%zu stream=%llu B\n", variants[v], n, (unsigned long long)S);
    HIP(hipFree(d_out));
  }

  /* chunk-pipelined transfer through pinned host memory */
  const size_t group = 2 * 65536;
  const uint32_t depth = 4;
  size_t dw = 0, hl = 0;
  CHECK(splitzip_pipeline_sizes(SPLITZIP_BF16, n, 1, 0, group, depth, &dw, &hl) == SPLITZIP_OK, "pipeline sizes");
  void *d_pw, *h_link;
  HIP(hipMalloc(&d_pw, dw));
  HIP(hipHostMalloc(&h_link, hl, hipHostMallocCoherent));
  hipStream_t st[4];
  for (int i = 0; i < 4; ++i) HIP(hipStreamCreate(&st[i]));
  const size_t groups = (n + group - 1) / group;
  uint64_t sent[8] = {0};
  CHECK(groups <= 8, "groups");
  HIP(hipMemset(d_y, 0, n * 2));
  HIP(hipMemset(d_status, 0, 4));
  HIP(hipDeviceSynchronize());
  CHECK(splitzip_pipeline_transfer(SPLITZIP_BF16, d_in, n, cb, 1, 0, group, depth, 1, d_pw, dw, h_link, hl, d_y,
                                   d_status, sent, st) == SPLITZIP_OK,
        "pipeline transfer");
  int32_t status = -1;
  HIP(hipMemcpy(y, d_y, n * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
  CHECK(status == SPLITZIP_OK && memcmp(x, y, n * 2) == 0, "pipeline output differs");
  uint64_t total = 0;
  for (size_t g = 0; g < groups; ++g) total += sent[g];
  CHECK(total > 0 && total < n * 2, "bytes over the link %llu of %zu", (unsigned long long)total, n * 2);
  printf("c-abi ok: pipeline n=%zu groups=%zu link bytes=%llu (raw %zu)\n", n, groups, (unsigned long long)total,
         n * 2);
  for (int i = 0; i < 4; ++i) HIP(hipStreamDestroy(st[i]));
  HIP(hipHostFree(h_link));
  HIP(hipFree(d_pw));

  const char* msg = splitzip_status_string(SPLITZIP_E_CORRUPT);
  CHECK(msg != NULL && msg[0] != 0, "status string");
  fflush(stdout);
  HIP(hipFree(d_in));
  HIP(hipFree(d_y));
  HIP(hipFree(d_status));
  HIP(hipFree(d_bytes));
  free(x);
  free(y);
}

int main(void) {
  run(SPLITZIP_BF16, 3 * 65536 + 12345);
  run(SPLITZIP_FP8_E5M2, 5 * 65536 + 777);
  extras();
  return 0;
}
