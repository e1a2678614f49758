/*
 * A plain C99 client of librnq.so: it includes only include/rnq.h and the HIP
 * runtime's C API, so it checks that the boundary is usable without C++,
 * Python or torch.
 *
 *   c_client qk IN OUT    run rnq_qk_norm_rope_fp8 on the problem in IN and
 *                         write the codes and scales to OUT
 *   c_client errors       check the argument validation statuses (no launch)
 *
 * IN (little-endian): five int64 (tokens, q_heads, kv_heads, head_dim,
 * rope_dim), an int64 dtype (rnq_dtype), then q [T*Hq*D] and k [T*Hk*D] as
 * 16-bit words, wq [D] and wk [D] as 16-bit words, cos and sin [T*R/2] fp32.
 * OUT: q codes [T*Hq*D] bytes, k codes [T*Hk*D] bytes, q scales [T*Hq] and k
 * scales [T*Hk] fp32. The inputs are copied to device memory, the call runs
 * on the null stream, and the outputs are copied back after a synchronise.
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rnq.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "c_client: %s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p == NULL || fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

/* host buffer -> new device buffer (NULL on failure) */
static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  if (!hip_ok(hipMalloc(&d, bytes ? bytes : 16), "hipMalloc")) return NULL;
  if (bytes && !hip_ok(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device")) {
    hipFree(d);
    return NULL;
  }
  return d;
}

static int run_qk(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (f == NULL) {
    fprintf(stderr, "c_client: cannot open %s\n", in_path);
    return 1;
  }
  int64_t hdr[6];
  if (fread(hdr, sizeof(int64_t), 6, f) != 6) {
    fprintf(stderr, "c_client: short header\n");
    fclose(f);
    return 1;
  }
  const int64_t T = hdr[0], Hq = hdr[1], Hk = hdr[2], D = hdr[3], R = hdr[4], dtype = hdr[5];
  if (T < 1 || Hq < 1 || Hk < 0 || D < 1 || R < 0 || T > (1 << 20) || Hq > 1024 || Hk > 1024 || D > 512) {
    fprintf(stderr, "c_client: header out of range\n");
    fclose(f);
    return 1;
  }
  const size_t nq = (size_t)(T * Hq * D), nk = (size_t)(T * Hk * D), nt = (size_t)(T * (R / 2));
  void* hq = read_block(f, 2 * nq);
  void* hk = read_block(f, 2 * nk);
  void* hwq = read_block(f, 2 * (size_t)D);
  void* hwk = read_block(f, 2 * (size_t)D);
  void* hc = read_block(f, 4 * nt);
  void* hs = read_block(f, 4 * nt);
  fclose(f);
  int rc = 1;
  void *dq = NULL, *dk = NULL, *dwq = NULL, *dwk = NULL, *dc = NULL, *ds = NULL;
  void *dq8 = NULL, *dk8 = NULL, *dqs = NULL, *dks = NULL;
  uint8_t *q8 = NULL, *k8 = NULL;
  float *qs = NULL, *ks = NULL;
  if (!hq || !hk || !hwq || !hwk || !hc || !hs) {
    fprintf(stderr, "c_client: short input\n");
    goto done;
  }
  dq = to_device(hq, 2 * nq);
  dk = to_device(hk, 2 * nk);
  dwq = to_device(hwq, 2 * (size_t)D);
  dwk = to_device(hwk, 2 * (size_t)D);
  dc = to_device(hc, 4 * nt);
  ds = to_device(hs, 4 * nt);
  if (!dq || !dk || !dwq || !dwk || !dc || !ds) goto done;
  if (!hip_ok(hipMalloc(&dq8, nq), "hipMalloc") || !hip_ok(hipMalloc(&dk8, nk ? nk : 16), "hipMalloc") ||
      !hip_ok(hipMalloc(&dqs, 4 * (size_t)(T * Hq)), "hipMalloc") ||
      !hip_ok(hipMalloc(&dks, 4 * (size_t)(T * (Hk ? Hk : 1))), "hipMalloc"))
    goto done;
  {
    const rnq_status st = rnq_qk_norm_rope_fp8(dq, Hk ? dk : NULL, dwq, Hk ? dwk : NULL, R ? (const float*)dc : NULL,
                                               R ? (const float*)ds : NULL, (uint8_t*)dq8, Hk ? (uint8_t*)dk8 : NULL,
                                               (float*)dqs, Hk ? (float*)dks : NULL, NULL, NULL, T, Hq, Hk, D, R,
                                               1e-6f, 448.0f, (int)dtype, NULL);
    if (st != RNQ_OK) {
      fprintf(stderr, "c_client: rnq_qk_norm_rope_fp8: %s (%s)\n", rnq_status_string(st), rnq_last_error());
      goto done;
    }
  }
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) goto done;
  q8 = (uint8_t*)malloc(nq);
  k8 = (uint8_t*)malloc(nk ? nk : 1);
  qs = (float*)malloc(4 * (size_t)(T * Hq));
  ks = (float*)malloc(4 * (size_t)(T * (Hk ? Hk : 1)));
  if (!q8 || !k8 || !qs || !ks) goto done;
  if (!hip_ok(hipMemcpy(q8, dq8, nq, hipMemcpyDeviceToHost), "hipMemcpy to host") ||
      (nk && !hip_ok(hipMemcpy(k8, dk8, nk, hipMemcpyDeviceToHost), "hipMemcpy to host")) ||
      !hip_ok(hipMemcpy(qs, dqs, 4 * (size_t)(T * Hq), hipMemcpyDeviceToHost), "hipMemcpy to host") ||
      (Hk && !hip_ok(hipMemcpy(ks, dks, 4 * (size_t)(T * Hk), hipMemcpyDeviceToHost), "hipMemcpy to host")))
    goto done;
  {
    FILE* o = fopen(out_path, "wb");
    if (o == NULL) {
      fprintf(stderr, "c_client: cannot create %s\n", out_path);
      goto done;
    }
    const int wrote = fwrite(q8, 1, nq, o) == nq && fwrite(k8, 1, nk, o) == nk &&
                      fwrite(qs, 4, (size_t)(T * Hq), o) == (size_t)(T * Hq) &&
                      fwrite(ks, 4, (size_t)(T * Hk), o) == (size_t)(T * Hk);
    if (fclose(o) != 0 || !wrote) {
      fprintf(stderr, "c_client: short write to %s\n", out_path);
      goto done;
    }
  }
  rc = 0;
done:
  free(hq); free(hk); free(hwq); free(hwk); free(hc); free(hs);
  free(q8); free(k8); free(qs); free(ks);
  hipFree(dq); hipFree(dk); hipFree(dwq); hipFree(dwk); hipFree(dc); hipFree(ds);
  hipFree(dq8); hipFree(dk8); hipFree(dqs); hipFree(dks);
  return rc;
}

/* statuses of invalid calls: validated on the host before anything is enqueued
 * (the pointers are never dereferenced) */
static int check_errors(void) {
  uint8_t* const fake = (uint8_t*)(uintptr_t)0x10000;  /* 16-byte aligned, never touched */
  struct {
    const char* what;
    rnq_status got, want;
  } c[] = {
      {"head_dim 96", rnq_qk_norm_rope_fp8(fake, fake, fake, fake, (float*)fake, (float*)fake, fake, fake, (float*)fake,
                                           (float*)fake, NULL, NULL, 4, 2, 1, 96, 32, 1e-6f, 448.0f, RNQ_BF16, NULL),
       RNQ_ERR_UNSUPPORTED},
      {"odd rope_dim", rnq_qk_norm_rope_fp8(fake, fake, fake, fake, (float*)fake, (float*)fake, fake, fake, (float*)fake,
                                            (float*)fake, NULL, NULL, 4, 2, 1, 128, 33, 1e-6f, 448.0f, RNQ_BF16, NULL),
       RNQ_ERR_SHAPE},
      {"missing q", rnq_qk_norm_rope_fp8(NULL, fake, fake, fake, (float*)fake, (float*)fake, fake, fake, (float*)fake,
                                         (float*)fake, NULL, NULL, 4, 2, 1, 128, 64, 1e-6f, 448.0f, RNQ_BF16, NULL),
       RNQ_ERR_NULL},
      {"fp8_max 500", rnq_qk_norm_rope_fp8(fake, fake, fake, fake, (float*)fake, (float*)fake, fake, fake, (float*)fake,
                                           (float*)fake, NULL, NULL, 4, 2, 1, 128, 64, 1e-6f, 500.0f, RNQ_BF16, NULL),
       RNQ_ERR_ARG},
      {"zero rows", rnq_qk_norm_rope_fp8(fake, fake, fake, fake, (float*)fake, (float*)fake, fake, fake, (float*)fake,
                                         (float*)fake, NULL, NULL, 0, 2, 1, 128, 64, 1e-6f, 448.0f, RNQ_BF16, NULL),
       RNQ_OK},
  };
  int bad = 0;
  for (size_t i = 0; i < sizeof c / sizeof c[0]; ++i) {
    printf("%s: %s\n", c[i].what, rnq_status_string(c[i].got));
    if (c[i].got != c[i].want) {
      fprintf(stderr, "c_client: %s gave %s, expected %s\n", c[i].what, rnq_status_string(c[i].got),
              rnq_status_string(c[i].want));
      bad = 1;
    }
  }
  return bad;
}

int main(int argc, char** argv) {
  if (argc == 4 && strcmp(argv[1], "qk") == 0) return run_qk(argv[2], argv[3]);
  if (argc == 2 && strcmp(argv[1], "errors") == 0) return check_errors();
  fprintf(stderr, "usage: c_client qk IN OUT | c_client errors\n");
  return 2;
}
