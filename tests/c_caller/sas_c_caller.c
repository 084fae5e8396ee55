/*
 * A plain C11 caller of libsas (test tool): shows that the boundary needs no
 * C++, no Python and no torch.  Built with gcc against include/sas.h, linked
 * with libsas.so and the HIP runtime.
 *
 *   sas_c_caller abi
 *       host-only checks: ABI version, status strings, and argument
 *       validation (every call returns before touching a device).
 *   sas_c_caller layer DIR B Hq Hkv n d topk gate
 *       reads DIR/{q,k,v,do}.bin (bf16 [B,H,n,d]) and DIR/s.bin (float32
 *       [B,Hkv,n/64,n/64]); runs sas_select, sas_fwd and sas_bwd on the
 *       null stream; writes DIR/{o,dq,dk,dv}.bin (bf16), DIR/{lse,ds,
 *       s_lse,log_gate}.bin (float32) and DIR/{idx,cnt}.bin (int32).
 * Exit status 0 on success; otherwise the failing step is printed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sas.h"

#define CHECK_SAS(call)                                                              \
  do {                                                                               \
    sas_status st_ = (call);                                                         \
    if (st_ != SAS_OK) {                                                             \
      fprintf(stderr, "%s failed: %s (%s)\n", #call, sas_status_string(st_),         \
              sas_last_hip_error());                                                 \
      return 1;                                                                      \
    }                                                                                \
  } while (0)
#define CHECK_HIP(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s failed: %d\n", #call, (int)e_);                            \
      return 1;                                                                      \
    }                                                                                \
  } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    p = NULL;
  }
  fclose(f);
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const int bad = fwrite(p, 1, bytes, f) != bytes;
  fclose(f);
  return bad;
}

/* device buffer of `bytes`, filled from the host copy when `host` is given */
static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
  if (host && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

static int fetch(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* h = malloc(bytes);
  if (!h) return 1;
  int bad = hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess;
  if (!bad) bad = write_file(dir, name, h, bytes);
  free(h);
  return bad;
}

static int abi_checks(void) {
  int fails = 0;
#define EXPECT(cond)                                         \
  do {                                                       \
    if (!(cond)) {                                           \
      fprintf(stderr, "expectation failed: %s\n", #cond);    \
      ++fails;                                               \
    }                                                        \
  } while (0)
  EXPECT(sas_abi_version() == 4);
  EXPECT(strncmp(sas_status_string(SAS_OK), "SAS_OK", 6) == 0);
  void* fake = (void*)(uintptr_t)0x1000; /* never dereferenced: validation fails first */
  sas_shape good = {1, 8, 2, 512, 128, 4, 0.0f, SAS_BF16, SAS_GATE_SOFTMAX, 0, NULL};
  EXPECT(sas_bwd_workspace_bytes(&good) > 0);
  sas_shape bad_n = good;
  bad_n.n = 500;
  EXPECT(sas_select(&bad_n, fake, fake, fake, fake, fake, NULL) == SAS_ERR_ARG);
  sas_shape bad_dtype = good;
  bad_dtype.dtype = 9;
  EXPECT(sas_fwd(&bad_dtype, fake, fake, fake, fake, fake, fake, fake, fake, NULL) ==
         SAS_ERR_DTYPE);
  sas_shape bad_gate = good;
  bad_gate.gate = 7;
  EXPECT(sas_bwd_workspace_bytes(&bad_gate) == 0);
  EXPECT(sas_select(NULL, fake, fake, fake, fake, fake, NULL) == SAS_ERR_ARG);
  EXPECT(sas_bwd(&good, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                 fake, fake, fake, fake, 1, NULL) == SAS_ERR_WORKSPACE);
  /* packed documents of any length: 100, 64 and 1 tokens */
  const int32_t cu[4] = {0, 100, 164, 165};
  int32_t blk[8], first[4];
  EXPECT(sas_blocks_from_cu_seqlens(cu, 3, blk, first, 4) == 4);
  EXPECT(blk[0] == 0 && blk[1] == 64 && blk[2] == 64 && blk[3] == 36 && blk[4] == 100 &&
         blk[5] == 64 && blk[6] == 164 && blk[7] == 1);
  EXPECT(first[0] == 0 && first[1] == 0 && first[2] == 2 && first[3] == 3);
  EXPECT(sas_blocks_from_cu_seqlens(cu, 3, blk, first, 3) == -1);
  sas_shape packed = good;
  packed.n = 165;
  packed.nb = 4;
  packed.blocks = (const int32_t*)fake;
  EXPECT(sas_bwd_workspace_bytes(&packed) > 0);
  packed.nb = 0;
  EXPECT(sas_bwd_workspace_bytes(&packed) == 0);
  sas_decode_paged_shape ps = {2, 8, 2, 8192, 100, 128, 32, 0.0f, SAS_BF16, SAS_GATE_EXTERNAL};
  EXPECT(sas_decode_paged_workspace_bytes(&ps) > 0);
  ps.max_blocks = SAS_MAX_DECODE_BLOCKS + 1;
  EXPECT(sas_decode_paged_workspace_bytes(&ps) == 0);
#undef EXPECT
  if (fails == 0) printf("abi checks ok\n");
  return fails != 0;
}

static int layer(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s layer DIR B Hq Hkv n d topk gate\n", argv[0]);
    return 2;
  }
  const char* dir = argv[2];
  sas_shape sh;
  sh.B = atoi(argv[3]);
  sh.Hq = atoi(argv[4]);
  sh.Hkv = atoi(argv[5]);
  sh.n = atoi(argv[6]);
  sh.d = atoi(argv[7]);
  sh.topk = atoi(argv[8]);
  sh.scale = 0.0f;
  sh.dtype = SAS_BF16;
  sh.gate = atoi(argv[9]);
  sh.nb = 0;          /* blocks of 64 tokens, no block table */
  sh.blocks = NULL;
  if (sh.B < 1 || sh.Hq < 1 || sh.Hkv < 1 || sh.n < 64 || sh.d < 1 || sh.topk < 0) {
    fprintf(stderr, "bad shape arguments\n");
    return 2;
  }
  const size_t nb = (size_t)sh.n / SAS_BLOCK;
  const size_t qn = (size_t)sh.B * sh.Hq * sh.n * sh.d, kn = (size_t)sh.B * sh.Hkv * sh.n * sh.d;
  const size_t rows = (size_t)sh.B * sh.Hkv * nb, K = sh.topk > 0 ? (size_t)sh.topk : 1;
  const size_t sn = rows * nb;

  void* hq = read_file(dir, "q.bin", qn * 2);
  void* hk = read_file(dir, "k.bin", kn * 2);
  void* hv = read_file(dir, "v.bin", kn * 2);
  void* hdo = read_file(dir, "do.bin", qn * 2);
  void* hs = read_file(dir, "s.bin", sn * 4);
  if (!hq || !hk || !hv || !hdo || !hs) {
    fprintf(stderr, "cannot read the inputs in %s\n", dir);
    return 1;
  }
  void* q = to_device(hq, qn * 2);
  void* k = to_device(hk, kn * 2);
  void* v = to_device(hv, kn * 2);
  void* dO = to_device(hdo, qn * 2);
  float* s = (float*)to_device(hs, sn * 4);
  int32_t* idx = (int32_t*)to_device(NULL, rows * K * 4);
  int32_t* cnt = (int32_t*)to_device(NULL, rows * 4);
  float* lg = (float*)to_device(NULL, rows * K * 4);
  float* s_lse = (float*)to_device(NULL, rows * 4);
  void* o = to_device(NULL, qn * 2);
  float* lse = (float*)to_device(NULL, (size_t)sh.B * sh.Hq * sh.n * 4);
  void* dq = to_device(NULL, qn * 2);
  void* dk = to_device(NULL, kn * 2);
  void* dv = to_device(NULL, kn * 2);
  float* ds = (float*)to_device(NULL, sn * 4);
  const size_t ws_bytes = sas_bwd_workspace_bytes(&sh);
  void* ws = to_device(NULL, ws_bytes);
  if (!q || !k || !v || !dO || !s || !idx || !cnt || !lg || !s_lse || !o || !lse || !dq || !dk ||
      !dv || !ds || !ws) {
    fprintf(stderr, "device allocation failed\n");
    return 1;
  }
  CHECK_SAS(sas_select(&sh, s, idx, cnt, lg, s_lse, NULL));
  CHECK_SAS(sas_fwd(&sh, q, k, v, idx, cnt, lg, o, lse, NULL));
  CHECK_SAS(sas_bwd(&sh, q, k, v, o, dO, lse, idx, cnt, lg, s, s_lse, dq, dk, dv, ds, ws,
                    ws_bytes, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  if (fetch(dir, "o.bin", o, qn * 2) || fetch(dir, "dq.bin", dq, qn * 2) ||
      fetch(dir, "dk.bin", dk, kn * 2) || fetch(dir, "dv.bin", dv, kn * 2) ||
      fetch(dir, "lse.bin", lse, (size_t)sh.B * sh.Hq * sh.n * 4) ||
      fetch(dir, "ds.bin", ds, sn * 4) || fetch(dir, "s_lse.bin", s_lse, rows * 4) ||
      fetch(dir, "log_gate.bin", lg, rows * K * 4) || fetch(dir, "idx.bin", idx, rows * K * 4) ||
      fetch(dir, "cnt.bin", cnt, rows * 4)) {
    fprintf(stderr, "cannot write the outputs to %s\n", dir);
    return 1;
  }
  void* bufs[] = {q, k, v, dO, s, idx, cnt, lg, s_lse, o, lse, dq, dk, dv, ds, ws};
  for (size_t j = 0; j < sizeof bufs / sizeof bufs[0]; ++j) CHECK_HIP(hipFree(bufs[j]));
  free(hq);
  free(hk);
  free(hv);
  free(hdo);
  free(hs);
  printf("layer ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "abi") == 0) return abi_checks();
  if (argc >= 2 && strcmp(argv[1], "layer") == 0) return layer(argc, argv);
  fprintf(stderr, "usage: %s abi | layer DIR B Hq Hkv n d topk gate\n", argv[0]);
  return 2;
}
