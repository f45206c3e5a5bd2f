/*
 * A C99 program that uses the attention library through include/sdpa14.h
 * alone: no Python, no C++.  tests/test_c_consumer.py builds it with gcc and
 * runs it.
 *
 *   c_abi_consumer host
 *       Calls that need no GPU: status names, the workspace and keep-bit
 *       sizes, the RNG state round trip, argument checks and their messages,
 *       and the launch-failure path (SDPA14_FAIL_LAUNCH).
 *   c_abi_consumer gpu DIR B H Sq Sk E causal
 *       Reads DIR/{q,k,v,do}.bin (bf16, contiguous [B, H, S, E]), runs
 *       sdpa_fwd and sdpa_bwd on the current device, and writes
 *       DIR/{out,dq,dk,dv}.bin (bf16) and DIR/lse.bin (fp32).
 *
 * Exit status 0 on success; every failed check prints one line.
 */
#define _POSIX_C_SOURCE 200112L
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sdpa14.h"

static int failures = 0;

#define CHECK(cond, ...)              \
  do {                                \
    if (!(cond)) {                    \
      fprintf(stderr, "FAIL: ");      \
      fprintf(stderr, __VA_ARGS__);   \
      fprintf(stderr, "\n");          \
      ++failures;                     \
    }                                 \
  } while (0)

static sdpa_tensor contiguous(void* data, int64_t B, int64_t H, int64_t S, int64_t E) {
  sdpa_tensor t;
  t.data = data;
  t.dtype = SDPA_BF16;
  t.size[0] = B;
  t.size[1] = H;
  t.size[2] = S;
  t.size[3] = E;
  t.stride[3] = 1;
  t.stride[2] = E;
  t.stride[1] = S * E;
  t.stride[0] = H * S * E;
  return t;
}

static int run_host(void) {
  CHECK(strcmp(sdpa_status_string(SDPA_OK), "SDPA_OK") == 0, "status name of SDPA_OK");
  CHECK(strcmp(sdpa_status_string(SDPA_ERR_WORKSPACE), "SDPA_ERR_WORKSPACE") == 0,
        "status name of SDPA_ERR_WORKSPACE");
  CHECK(sdpa_bwd_workspace_size(2, 12, 1024) == (size_t)2 * 12 * 1024 * 8, "workspace size");
  CHECK(sdpa_bwd_workspace_size(0, 1, 1) == 0, "workspace size of an empty problem");
  CHECK(sdpa_keep_bits_size(1, 1, 1, 1) > 0, "keep-bit size");

  uint64_t seed = 0, offset = 0;
  sdpa_set_rng_state(0xFFFFFFFFFFFFFFFFull, 12345);
  sdpa_get_rng_state(&seed, &offset);
  CHECK(seed == 0xFFFFFFFFFFFFFFFFull && offset == 12345, "RNG state round trip");

  /* Fake, aligned, never dereferenced addresses: validation runs on the host. */
  char* base = (char*)(uintptr_t)0x7F0000000000ull;
  sdpa_tensor q = contiguous(base, 1, 2, 128, 64);
  sdpa_tensor k = contiguous(base + (1 << 20), 1, 2, 128, 64);
  sdpa_tensor v = contiguous(base + (2 << 20), 1, 2, 128, 64);
  sdpa_tensor out = contiguous(base + (3 << 20), 1, 2, 128, 64);
  float* lse = (float*)(base + (4 << 20));

  int rc = sdpa_fwd(NULL, &k, &v, 0.0, 1, NAN, &out, lse, &seed, &offset, NULL);
  CHECK(rc == SDPA_ERR_INVALID, "NULL q gives SDPA_ERR_INVALID (got %d)", rc);
  CHECK(strlen(sdpa_last_error()) > 0, "the error carries a message");

  rc = sdpa_fwd(&q, &k, &v, 1.5, 1, NAN, &out, lse, &seed, &offset, NULL);
  CHECK(rc == SDPA_ERR_INVALID && strstr(sdpa_last_error(), "dropout_p") != NULL,
        "dropout_p = 1.5 is rejected (got %d: %s)", rc, sdpa_last_error());

  sdpa_tensor wide = contiguous(base, 1, 2, 128, 136);
  rc = sdpa_fwd(&wide, &wide, &wide, 0.0, 0, NAN, &out, lse, &seed, &offset, NULL);
  CHECK(rc == SDPA_ERR_UNSUPPORTED || rc == SDPA_ERR_INVALID, "head dim 136 is refused (got %d)",
        rc);

  sdpa_tensor aliased = contiguous(base, 1, 2, 128, 64);
  rc = sdpa_fwd(&q, &k, &v, 0.0, 1, NAN, &aliased, lse, &seed, &offset, NULL);
  CHECK(rc == SDPA_ERR_INVALID && strstr(sdpa_last_error(), "overlaps") != NULL,
        "out on top of q is rejected (got %d: %s)", rc, sdpa_last_error());

  /* Valid arguments with the launch hook set: SDPA_ERR_HIP before any HIP
   * call, and the RNG state stays where it was. */
  setenv("SDPA14_FAIL_LAUNCH", "1", 1);
  sdpa_set_rng_state(7, 100);
  rc = sdpa_fwd(&q, &k, &v, 0.1, 1, NAN, &out, lse, &seed, &offset, NULL);
  CHECK(rc == SDPA_ERR_HIP, "forced launch failure gives SDPA_ERR_HIP (got %d)", rc);
  sdpa_get_rng_state(&seed, &offset);
  CHECK(seed == 7 && offset == 100, "a failed launch leaves the RNG state alone");
  unsetenv("SDPA14_FAIL_LAUNCH");

  printf("host checks: %d failed\n", failures);
  return failures == 0 ? 0 : 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes);
  const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* dir, const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  const size_t put = fwrite(data, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "FAIL: %s: %s\n", #call, hipGetErrorString(e_)); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

static int run_gpu(const char* dir, int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t E,
                   int causal) {
  const size_t nq = (size_t)(B * H * Sq * E) * 2, nk = (size_t)(B * H * Sk * E) * 2;
  const size_t nl = (size_t)(B * H * Sq) * 4;
  void* hq = read_file(dir, "q.bin", nq);
  void* hk = read_file(dir, "k.bin", nk);
  void* hv = read_file(dir, "v.bin", nk);
  void* hdo = read_file(dir, "do.bin", nq);
  if (!hq || !hk || !hv || !hdo) {
    fprintf(stderr, "FAIL: cannot read the inputs from %s\n", dir);
    return 1;
  }
  void *q, *k, *v, *dout, *out, *dq, *dk, *dv, *lse, *ws;
  const size_t wsb = sdpa_bwd_workspace_size(B, H, Sq);
  HIP_OK(hipMalloc(&q, nq));
  HIP_OK(hipMalloc(&k, nk));
  HIP_OK(hipMalloc(&v, nk));
  HIP_OK(hipMalloc(&dout, nq));
  HIP_OK(hipMalloc(&out, nq));
  HIP_OK(hipMalloc(&dq, nq));
  HIP_OK(hipMalloc(&dk, nk));
  HIP_OK(hipMalloc(&dv, nk));
  HIP_OK(hipMalloc(&lse, nl));
  HIP_OK(hipMalloc(&ws, wsb));
  HIP_OK(hipMemcpy(q, hq, nq, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, nk, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, nk, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dout, hdo, nq, hipMemcpyHostToDevice));

  sdpa_tensor tq = contiguous(q, B, H, Sq, E), tk = contiguous(k, B, H, Sk, E);
  sdpa_tensor tv = contiguous(v, B, H, Sk, E), tdo = contiguous(dout, B, H, Sq, E);
  sdpa_tensor to = contiguous(out, B, H, Sq, E), tdq = contiguous(dq, B, H, Sq, E);
  sdpa_tensor tdk = contiguous(dk, B, H, Sk, E), tdv = contiguous(dv, B, H, Sk, E);
  uint64_t seed = 0, offset = 0;
  sdpa_set_rng_state(0, 0);
  int rc = sdpa_fwd(&tq, &tk, &tv, 0.0, causal, NAN, &to, (float*)lse, &seed, &offset, NULL);
  CHECK(rc == SDPA_OK, "sdpa_fwd: %s: %s", sdpa_status_string(rc), sdpa_last_error());
  if (rc == SDPA_OK) {
    rc = sdpa_bwd(&tdo, &tq, &tk, &tv, &to, (const float*)lse, 0.0, causal, seed, offset, NAN,
                  &tdq, &tdk, &tdv, ws, wsb, NULL);
    CHECK(rc == SDPA_OK, "sdpa_bwd: %s: %s", sdpa_status_string(rc), sdpa_last_error());
  }
  HIP_OK(hipDeviceSynchronize());
  if (failures) return 1;

  void* host = malloc(nq > nk ? nq : nk);
  if (!host) return 1;
  struct {
    const char* name;
    void* dev;
    size_t bytes;
  } outs[5] = {{"out.bin", out, nq}, {"lse.bin", lse, nl}, {"dq.bin", dq, nq},
               {"dk.bin", dk, nk},   {"dv.bin", dv, nk}};
  for (int i = 0; i < 5; ++i) {
    HIP_OK(hipMemcpy(host, outs[i].dev, outs[i].bytes, hipMemcpyDeviceToHost));
    CHECK(write_file(dir, outs[i].name, host, outs[i].bytes) == 0, "cannot write %s",
          outs[i].name);
  }
  free(host);
  void* bufs[10] = {q, k, v, dout, out, dq, dk, dv, lse, ws};
  for (int i = 0; i < 10; ++i) HIP_OK(hipFree(bufs[i]));
  free(hq);
  free(hk);
  free(hv);
  free(hdo);
  printf("gpu run: %d failed\n", failures);
  return failures == 0 ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return run_host();
  if (argc == 9 && strcmp(argv[1], "gpu") == 0)
    return run_gpu(argv[2], atoll(argv[3]), atoll(argv[4]), atoll(argv[5]), atoll(argv[6]),
                   atoll(argv[7]), atoi(argv[8]));
  fprintf(stderr, "usage: %s host | gpu DIR B H Sq Sk E causal\n", argv[0]);
  return 2;
}
