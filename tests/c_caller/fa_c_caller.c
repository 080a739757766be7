/*
 * A plain C caller of the attention library: device memory from the HIP
 * runtime, no Python and no torch.  Reads q, k, v, dout (bf16, contiguous
 * (batch, seqlen, heads, headdim)) from <dir>/{q,k,v,do}.bin, runs fa_fwd and
 * fa_bwd on the null stream, and writes <dir>/{o,dq,dk,dv}.bin (bf16) and
 * <dir>/lse.bin (float32).  Exit status 0 on success; on any error the status
 * name and fa_last_error() are printed.
 *
 * usage: fa_c_caller DIR BATCH SEQLEN NHEADS_Q NHEADS_KV HEADDIM CAUSAL
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fa.h"

static int read_file(const char* dir, const char* name, void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return -1;
  const size_t n = fread(buf, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  const size_t n = fwrite(buf, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

#define HIP_OK(x)                                                     \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
      return 2;                                                       \
    }                                                                 \
  } while (0)

#define FA_OK_OR_FAIL(x)                                                                           \
  do {                                                                                            \
    fa_status s_ = (x);                                                                           \
    if (s_ != FA_OK) {                                                                            \
      fprintf(stderr, "%s: %s (%s)\n", #x, fa_status_string(s_), fa_last_error());                \
      return 3;                                                                                   \
    }                                                                                             \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s DIR BATCH SEQLEN NHEADS_Q NHEADS_KV HEADDIM CAUSAL\n", argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  const int64_t b = atoll(argv[2]), n = atoll(argv[3]), hq = atoll(argv[4]), hkv = atoll(argv[5]),
                d = atoll(argv[6]);
  const int causal = atoi(argv[7]);
  const size_t qn = (size_t)(b * n * hq * d), kn = (size_t)(b * n * hkv * d), ln = (size_t)(b * hq * n);

  uint16_t* hq_ = malloc(qn * 2);
  uint16_t* hk = malloc(kn * 2);
  uint16_t* hv = malloc(kn * 2);
  uint16_t* hdo = malloc(qn * 2);
  float* hl = malloc(ln * 4);
  if (!hq_ || !hk || !hv || !hdo || !hl) return 2;
  if (read_file(dir, "q.bin", hq_, qn * 2) || read_file(dir, "k.bin", hk, kn * 2) ||
      read_file(dir, "v.bin", hv, kn * 2) || read_file(dir, "do.bin", hdo, qn * 2)) {
    fprintf(stderr, "cannot read the inputs in %s\n", dir);
    return 1;
  }

  void *q, *k, *v, *o, *dout, *dq, *dk, *dv, *ws;
  float* lse;
  HIP_OK(hipMalloc(&q, qn * 2));
  HIP_OK(hipMalloc(&k, kn * 2));
  HIP_OK(hipMalloc(&v, kn * 2));
  HIP_OK(hipMalloc(&o, qn * 2));
  HIP_OK(hipMalloc(&dout, qn * 2));
  HIP_OK(hipMalloc(&dq, qn * 2));
  HIP_OK(hipMalloc(&dk, kn * 2));
  HIP_OK(hipMalloc(&dv, kn * 2));
  HIP_OK(hipMalloc((void**)&lse, ln * 4));
  HIP_OK(hipMemcpy(q, hq_, qn * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, kn * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, kn * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dout, hdo, qn * 2, hipMemcpyHostToDevice));

  fa_params p;
  memset(&p, 0, sizeof p);
  p.batch = b;
  p.seqlen_q = p.seqlen_k = n;
  p.nheads_q = hq;
  p.nheads_kv = hkv;
  p.headdim = d;
  const int64_t qs[3] = {n * hq * d, hq * d, d}, ks[3] = {n * hkv * d, hkv * d, d};
  memcpy(p.q_strides, qs, sizeof qs);
  memcpy(p.o_strides, qs, sizeof qs);
  memcpy(p.k_strides, ks, sizeof ks);
  memcpy(p.v_strides, ks, sizeof ks);
  p.dtype = FA_BF16;
  p.scale = 1.0f / __builtin_sqrtf((float)d);
  p.causal = causal;
  p.window_left = p.window_right = -1;

  FA_OK_OR_FAIL(fa_fwd(&p, q, k, v, o, lse, NULL));
  size_t ws_bytes = 0;
  FA_OK_OR_FAIL(fa_bwd_workspace_size(&p, &ws_bytes));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  FA_OK_OR_FAIL(fa_bwd(&p, dout, q, k, v, o, lse, dq, dk, dv, ws, ws_bytes, NULL));
  HIP_OK(hipDeviceSynchronize());

  uint16_t* out = malloc(qn * 2 > kn * 2 ? qn * 2 : kn * 2);
  if (!out) return 2;
  HIP_OK(hipMemcpy(out, o, qn * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "o.bin", out, qn * 2)) return 1;
  HIP_OK(hipMemcpy(hl, lse, ln * 4, hipMemcpyDeviceToHost));
  if (write_file(dir, "lse.bin", hl, ln * 4)) return 1;
  HIP_OK(hipMemcpy(out, dq, qn * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "dq.bin", out, qn * 2)) return 1;
  HIP_OK(hipMemcpy(out, dk, kn * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "dk.bin", out, kn * 2)) return 1;
  HIP_OK(hipMemcpy(out, dv, kn * 2, hipMemcpyDeviceToHost));
  if (write_file(dir, "dv.bin", out, kn * 2)) return 1;
  printf("fa_c_caller: ok (B=%lld N=%lld Hq=%lld Hkv=%lld d=%lld causal=%d, library version %d)\n", (long long)b,
         (long long)n, (long long)hq, (long long)hkv, (long long)d, causal, fa_version());
  return 0;
}
