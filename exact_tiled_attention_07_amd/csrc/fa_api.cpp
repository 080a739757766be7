// C ABI of the attention library (declared in include/fa.h): argument
// validation, device capability check and dispatch to the HIP launchers.
//
// Every argument is checked on the host before the first HIP call, so an
// invalid call returns its status without touching the device.  No C++
// exception crosses the boundary.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <climits>
#include <mutex>
#include <string>

#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

size_t elem_bytes(fa_dtype d) { return d == FA_F32 ? 4 : 2; }

constexpr int64_t kMaxSeq = int64_t(1) << 30;
constexpr int64_t kMaxHeads = int64_t(1) << 16;
constexpr int64_t kMaxBatch = int64_t(1) << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa_status check_params(const fa_params* p) {
  if (!p) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 0 || p->seqlen_q < 0 || p->seqlen_k < 0)
    return fail(FA_ERR_INVALID_ARG, "batch/seqlen must be >= 0 (got %lld, %lld, %lld)",
                (long long)p->batch, (long long)p->seqlen_q, (long long)p->seqlen_k);
  if (p->nheads_q < 1 || p->nheads_kv < 1 || p->headdim < 1)
    return fail(FA_ERR_INVALID_ARG, "nheads_q, nheads_kv and headdim must be >= 1");
  if (p->nheads_q % p->nheads_kv != 0)
    return fail(FA_ERR_INVALID_ARG, "nheads_q (%lld) must be a multiple of nheads_kv (%lld)",
                (long long)p->nheads_q, (long long)p->nheads_kv);
  // A C caller can store any int in the enum field; reading it as the C++
  // enum before it is known to be valid is undefined, so take its raw bits.
  static_assert(sizeof(p->dtype) == sizeof(int32_t), "fa_dtype is a 32-bit enum");
  int32_t dtype_raw;
  std::memcpy(&dtype_raw, &p->dtype, sizeof dtype_raw);
  if (dtype_raw != FA_F32 && dtype_raw != FA_F16 && dtype_raw != FA_BF16)
    return fail(FA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype_raw);
  if (!(std::isfinite(p->scale) && p->scale > 0.f))
    return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (p->causal != 0 && p->causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p->window_left < -1 || p->window_right < -1)
    return fail(FA_ERR_INVALID_ARG, "window bounds must be >= -1 (got %d, %d)", p->window_left,
                p->window_right);
  if (!(std::isfinite(p->softcap) && p->softcap >= 0.f))
    return fail(FA_ERR_INVALID_ARG, "softcap must be finite and >= 0 (0 = off)");
  if (p->alibi_batch_stride < 0) return fail(FA_ERR_INVALID_ARG, "alibi_batch_stride must be >= 0");
  if (p->reserved_mod != 0) return fail(FA_ERR_INVALID_ARG, "reserved_mod must be 0");
  if (p->alibi_slopes && (reinterpret_cast<uintptr_t>(p->alibi_slopes) & 3u) != 0)
    return fail(FA_ERR_UNSUPPORTED, "alibi_slopes is not 4-byte aligned");
  if (p->seqlen_q > kMaxSeq || p->seqlen_k > kMaxSeq || p->nheads_q > kMaxHeads || p->batch > kMaxBatch)
    return fail(FA_ERR_UNSUPPORTED, "sizes exceed this build's limits");
  if (p->batch * p->nheads_q * ((p->seqlen_q + 31) / 32) >= (int64_t(1) << 31) ||
      p->batch * p->nheads_kv * ((p->seqlen_k + 31) / 32) >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "launch grid would exceed 2^31 workgroups");
  if (p->dtype == FA_F32) {
    if (p->headdim > 128 || p->headdim % 4 != 0)
      return fail(FA_ERR_UNSUPPORTED, "fp32 headdim must be a multiple of 4 in [4, 128] (got %lld)",
                  (long long)p->headdim);
  } else if (p->headdim > 128 || p->headdim % 8 != 0) {
    return fail(FA_ERR_UNSUPPORTED, "fp16/bf16 headdim must be a multiple of 8 in [8, 128] (got %lld)",
                (long long)p->headdim);
  }
  // Kernels address a tile of up to 128 rows with 32-bit byte offsets.
  if (p->q_strides[1] > (int64_t(1) << 22) || p->k_strides[1] > (int64_t(1) << 22) ||
      p->v_strides[1] > (int64_t(1) << 22) || p->o_strides[1] > (int64_t(1) << 22))
    return fail(FA_ERR_UNSUPPORTED, "sequence strides above 2^22 elements are not supported");
  const int64_t* strides[4] = {p->q_strides, p->k_strides, p->v_strides, p->o_strides};
  const char* names[4] = {"q", "k", "v", "o"};
  const int64_t eb = (int64_t)elem_bytes(p->dtype);
  for (int t = 0; t < 4; ++t) {
    for (int i = 0; i < 3; ++i) {
      const int64_t s = strides[t][i];
      if (s < 0) return fail(FA_ERR_UNSUPPORTED, "%s_strides[%d] is negative", names[t], i);
      if ((s * eb) % 16 != 0)
        return fail(FA_ERR_UNSUPPORTED, "%s_strides[%d]=%lld is not a multiple of 16 bytes", names[t], i,
                    (long long)s);
    }
  }
  // Rows of one head must not overlap: the tile loads bound a tile by
  // rows * row stride bytes, and outputs written through overlapping rows race.
  const int64_t rows[4] = {p->seqlen_q, p->seqlen_k, p->seqlen_k, p->seqlen_q};
  for (int t = 0; t < 4; ++t) {
    if (rows[t] > 1 && strides[t][1] < p->headdim)
      return fail(FA_ERR_UNSUPPORTED, "%s_strides[1]=%lld is below headdim (%lld): rows would overlap", names[t],
                  (long long)strides[t][1], (long long)p->headdim);
  }
  return FA_OK;
}

bool empty_problem(const fa_params* p) { return p->batch == 0 || p->seqlen_q == 0; }

fa_status check_ptr(const void* ptr, const char* name, bool nonempty) {
  if (!nonempty) return FA_OK;
  if (!ptr) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(FA_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  return FA_OK;
}

// Per-device "is this a gfx950" cache (hipGetDeviceProperties is slow).
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::mutex g_arch_mu;

fa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_arch_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (g_arch_ok[dev] < 0)
      return fail(FA_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  }
  if (g_arch_ok[dev] < 0) return fail(FA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return FA_OK;
}

// Scratch of fa_bwd_noalloc: the backward's row statistics (two float32
// arrays of batch * nheads_q * Nq_pad entries, as in a fa_bwd workspace) live
// in this static device array, so that the call takes no workspace and
// allocates nothing.  Each GPU holds its own copy until the process ends; its
// device address is resolved once per device, with that device current, and
// only that address is handed to kernels (the array's name is a host-side
// stand-in).  The preprocess stage writes every entry the other two stages
// read, so nothing in it needs clearing between calls.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

fa_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

fa::AttnArgs make_args(const fa_params* p) {
  fa::AttnArgs a{};
  a.q_sb = p->q_strides[0]; a.q_sn = p->q_strides[1]; a.q_sh = p->q_strides[2];
  a.k_sb = p->k_strides[0]; a.k_sn = p->k_strides[1]; a.k_sh = p->k_strides[2];
  a.v_sb = p->v_strides[0]; a.v_sn = p->v_strides[1]; a.v_sh = p->v_strides[2];
  a.o_sb = p->o_strides[0]; a.o_sn = p->o_strides[1]; a.o_sh = p->o_strides[2];
  a.B = (int32_t)p->batch;
  a.Nq = (int32_t)p->seqlen_q;
  a.Nk = (int32_t)p->seqlen_k;
  a.Hq = (int32_t)p->nheads_q;
  a.Hkv = (int32_t)p->nheads_kv;
  a.G = (int32_t)(p->nheads_q / p->nheads_kv);
  a.D = (int32_t)p->headdim;
  a.dtype = p->dtype == FA_F32 ? fa::kF32 : (p->dtype == FA_F16 ? fa::kF16 : fa::kBF16);
  a.scale = p->scale;
  a.scale_log2 = p->scale * fa::kLog2e;
  a.causal = p->causal;
  a.wl = p->window_left;
  a.wr = p->window_right;
  a.delta = (int32_t)(p->seqlen_k - p->seqlen_q);
  a.xcd_remap = 1;
  a.alibi = p->alibi_slopes;
  a.alibi_sb = p->alibi_batch_stride;
  a.cap = p->softcap > 0.f ? p->softcap / p->scale : INFINITY;
  a.inv_scale = 1.f / p->scale;
  a.softcap = p->softcap;
  a.mod = (p->alibi_slopes != nullptr || p->softcap > 0.f) ? 1 : 0;
  const int64_t nq_pad = (p->seqlen_q + 127) / 128 * 128;
  a.lse_sb = p->nheads_q * p->seqlen_q;
  a.lse_sh = p->seqlen_q;
  a.ws_sb = p->nheads_q * nq_pad;
  a.ws_sh = nq_pad;
  return a;
}

// Two float32 arrays (row sums D_i and log2-scaled LSE) of batch * nheads_q *
// Nq_pad entries, Nq_pad = seqlen_q rounded up to a multiple of 128.
size_t workspace_rows(const fa_params* p) {
  return (size_t)p->batch * (size_t)p->nheads_q * (size_t)((p->seqlen_q + 127) / 128 * 128);
}
size_t workspace_bytes_for(const fa_params* p) {
  const size_t n = 2 * workspace_rows(p) * sizeof(float);
  return ((n + 255) / 256) * 256;
}


// ----------------------------------------------------------------------------
// Attention against a KV cache.
// ----------------------------------------------------------------------------
constexpr int64_t kMaxKvParts = 1024;

fa_status check_kv_params(const fa_kvcache_params* kp) {
  if (!kp) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  const fa_params* p = &kp->base;
  fa_status s = check_params(p);
  if (s != FA_OK) return s;
  if (kp->num_splits < 0) return fail(FA_ERR_INVALID_ARG, "num_splits must be >= 0 (got %d)", kp->num_splits);
  if (kp->reserved != 0) return fail(FA_ERR_INVALID_ARG, "reserved must be 0");
  if (p->dtype == FA_F32) return fail(FA_ERR_UNSUPPORTED, "fa_fwd_kvcache supports fp16 and bf16 only");
  const int64_t* strides[2] = {kp->knew_strides, kp->vnew_strides};
  const char* names[2] = {"knew", "vnew"};
  for (int t = 0; t < 2; ++t) {
    for (int i = 0; i < 3; ++i) {
      const int64_t st = strides[t][i];
      if (st < 0) return fail(FA_ERR_UNSUPPORTED, "%s_strides[%d] is negative", names[t], i);
      if ((st * 2) % 16 != 0)
        return fail(FA_ERR_UNSUPPORTED, "%s_strides[%d]=%lld is not a multiple of 16 bytes", names[t], i,
                    (long long)st);
    }
  }
  return FA_OK;
}

// Key-range parts per (batch, K/V head, block of 32 packed query rows).
int64_t kv_parts(const fa_kvcache_params* kp) {
  const fa_params* p = &kp->base;
  const int64_t G = p->nheads_q / p->nheads_kv;
  const int64_t n_rb = (G * p->seqlen_q + 31) / 32;
  const int64_t tiles = std::max<int64_t>(1, (p->seqlen_k + 31) / 32);
  int64_t s;
  if (kp->num_splits > 0) {
    s = kp->num_splits;
  } else {
    // About two single-wave parts per SIMD of a 256-CU GPU, with at least 4
    // key tiles per part over a full cache.
    const int64_t units = std::max<int64_t>(1, p->batch * p->nheads_kv * n_rb);
    s = std::min<int64_t>((2048 + units - 1) / units, std::max<int64_t>(1, tiles / 4));
  }
  return std::max<int64_t>(1, std::min<int64_t>({s, tiles, kMaxKvParts}));
}

// Head dim of the kernels that run a head dim (64 or 128; smaller ones are masked).
int64_t kernel_headdim(int64_t d) { return d <= 64 ? 64 : 128; }

size_t kv_workspace_bytes(const fa_kvcache_params* kp) {
  const fa_params* p = &kp->base;
  const size_t rows = (size_t)p->batch * (size_t)p->nheads_q * (size_t)p->seqlen_q;
  const size_t n = rows * (size_t)kv_parts(kp) * (size_t)(kernel_headdim(p->headdim) + 1) * sizeof(float);
  return ((n + 255) / 256) * 256;
}


// ----------------------------------------------------------------------------
// Packed variable-length batches.
// ----------------------------------------------------------------------------
fa_status check_varlen(const fa_varlen_params* vp, fa_params* base) {
  if (!vp) return fail(FA_ERR_INVALID_ARG, "params is NULL");
  *base = vp->base;
  base->q_strides[0] = base->k_strides[0] = base->v_strides[0] = base->o_strides[0] = 0;  // ignored
  fa_status s = check_params(base);
  if (s != FA_OK) return s;
  if (vp->total_q < 0 || vp->total_k < 0)
    return fail(FA_ERR_INVALID_ARG, "total_q / total_k must be >= 0 (got %lld, %lld)", (long long)vp->total_q,
                (long long)vp->total_k);
  if (vp->total_q > INT32_MAX || vp->total_k > INT32_MAX)
    return fail(FA_ERR_UNSUPPORTED, "packed tensors above 2^31 - 1 rows are not supported");
  return FA_OK;
}

fa_status check_offsets(const int32_t* cu, const char* name, bool needed) {
  if (!needed) return FA_OK;
  if (!cu) return fail(FA_ERR_INVALID_ARG, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(cu) & 3u) != 0) return fail(FA_ERR_UNSUPPORTED, "%s is not 4-byte aligned", name);
  return FA_OK;
}

// Row statistics of the backward: nheads_q * (total_q + 128 * batch) floats
// per array (every sequence keeps up to 127 padding rows after its own).
size_t varlen_ws_rows(const fa_params* p, const fa_varlen_params* vp) {
  return (size_t)p->nheads_q * (size_t)(vp->total_q + 128 * p->batch);
}
size_t varlen_ws_bytes(const fa_params* p, const fa_varlen_params* vp) {
  const size_t n = 2 * varlen_ws_rows(p, vp) * sizeof(float);
  return ((n + 255) / 256) * 256;
}

fa::AttnArgs make_varlen_args(const fa_params* p, const fa_varlen_params* vp, const int32_t* cu_q,
                              const int32_t* cu_k) {
  fa::AttnArgs a = make_args(p);
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.total_q = (int32_t)vp->total_q;
  a.total_k = (int32_t)vp->total_k;
  a.lse_sb = 0;
  a.lse_sh = vp->total_q;
  a.ws_sb = 0;
  a.ws_sh = vp->total_q + 128 * p->batch;
  return a;
}
}  // namespace

extern "C" {

fa_status fa_fwd(const fa_params* params, const void* q, const void* k, const void* v, void* o, float* lse,
                 void* stream) {
  fa_status s = check_params(params);
  if (s != FA_OK) return s;
  const bool nonempty = !empty_problem(params);
  const bool kv_nonempty = nonempty && params->seqlen_k > 0;  // K/V are read only if there are queries
  if ((s = check_ptr(q, "q", nonempty)) != FA_OK) return s;
  if ((s = check_ptr(k, "k", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(v, "v", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(o, "o", nonempty)) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse", nonempty)) != FA_OK) return s;
  if (nonempty && (o == q || o == k || o == v)) return fail(FA_ERR_INVALID_ARG, "o must not alias q, k or v");
  if (!nonempty) return FA_OK;
  if ((s = check_device()) != FA_OK) return s;
  fa::AttnArgs a = make_args(params);
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = (params->dtype == FA_F32) ? fa::launch_fwd_f32(a, st) : fa::launch_fwd_mfma(a, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_bwd_workspace_size(const fa_params* params, size_t* bytes) {
  fa_status s = check_params(params);
  if (s != FA_OK) return s;
  if (!bytes) return fail(FA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = workspace_bytes_for(params);
  return FA_OK;
}

}  // extern "C"

namespace {

// noalloc: the row statistics go to this device's static scratch instead of
// a caller's workspace (fa_bwd_noalloc); workspace arguments are ignored.
fa_status run_bwd(const fa_params* params, int stages, const void* dout, const void* q, const void* k,
                  const void* v, const void* o, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, void* stream, bool noalloc = false) {
  fa_status s = check_params(params);
  if (s != FA_OK) return s;
  const bool q_nonempty = !empty_problem(params);
  const bool kv_nonempty = params->batch > 0 && params->seqlen_k > 0;
  if ((s = check_ptr(dout, "dout", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(q, "q", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(k, "k", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(v, "v", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(o, "o", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(dq, "dq", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(dk, "dk", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(dv, "dv", kv_nonempty)) != FA_OK) return s;
  const size_t need = workspace_bytes_for(params);
  if (noalloc) {
    if (need > kNoallocScratchBytes)
      return fail(FA_ERR_UNSUPPORTED,
                  "fa_bwd_noalloc: this problem needs %zu bytes of row statistics, above the %zu bytes of the "
                  "library's static scratch (call fa_bwd with a workspace instead)",
                  need, kNoallocScratchBytes);
  } else if (need > 0) {
    if ((s = check_ptr(workspace, "workspace", true)) != FA_OK) return s;
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  }
  if (q_nonempty || kv_nonempty) {
    const void* outs[3] = {dq, dk, dv};
    const void* ins[6] = {dout, q, k, v, o, lse};
    for (const void* x : outs)
      for (const void* y : ins)
        if (x && x == y) return fail(FA_ERR_INVALID_ARG, "gradient outputs must not alias the inputs");
  }
  if (!q_nonempty && !kv_nonempty) return FA_OK;
  if ((s = check_device()) != FA_OK) return s;
  if (noalloc && (s = device_scratch(&workspace)) != FA_OK) return s;
  fa::AttnArgs a = make_args(params);
  a.q = q; a.k = k; a.v = v; a.o = const_cast<void*>(o); a.lse = const_cast<float*>(lse);
  a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsum = static_cast<float*>(workspace);
  a.lse2 = a.dsum + workspace_rows(params);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      (params->dtype == FA_F32) ? fa::launch_bwd_f32(a, st, stages) : fa::launch_bwd_mfma(a, st, stages);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd(const fa_params* params, const void* dout, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return run_bwd(params, fa::kStageAll, dout, q, k, v, o, lse, dq, dk, dv, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_noalloc(const fa_params* params, const void* dout, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, void* dq, void* dk, void* dv, void* stream) {
  return run_bwd(params, fa::kStageAll, dout, q, k, v, o, lse, dq, dk, dv, nullptr, 0, stream, true);
}

fa_status fa_bwd_stage(const fa_params* params, int stage, const void* dout, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int mask = 0;
  switch (stage) {
    case FA_BWD_PREPARE: mask = fa::kStagePrepare; break;
    case FA_BWD_DKDV: mask = fa::kStageDkdv; break;
    case FA_BWD_DQ: mask = fa::kStageDq; break;
    default: return fail(FA_ERR_INVALID_ARG, "unknown backward stage %d", stage);
  }
  return run_bwd(params, mask, dout, q, k, v, o, lse, dq, dk, dv, workspace, workspace_bytes, stream);
}

fa_status fa_fwd_varlen(const fa_varlen_params* params, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* o, float* lse,
                        void* stream) {
  fa_params p;
  fa_status s = check_varlen(params, &p);
  if (s != FA_OK) return s;
  const bool nonempty = p.batch > 0 && params->total_q > 0 && p.seqlen_q > 0;
  const bool kv_nonempty = nonempty && params->total_k > 0 && p.seqlen_k > 0;
  if ((s = check_ptr(q, "q", nonempty)) != FA_OK) return s;
  if ((s = check_ptr(k, "k", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(v, "v", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(o, "o", nonempty)) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse", nonempty)) != FA_OK) return s;
  if ((s = check_offsets(cu_seqlens_q, "cu_seqlens_q", nonempty)) != FA_OK) return s;
  if ((s = check_offsets(cu_seqlens_k, "cu_seqlens_k", nonempty)) != FA_OK) return s;
  if (nonempty && (o == q || o == k || o == v)) return fail(FA_ERR_INVALID_ARG, "o must not alias q, k or v");
  if (!nonempty) return FA_OK;
  if ((s = check_device()) != FA_OK) return s;
  fa::AttnArgs a = make_varlen_args(&p, params, cu_seqlens_q, cu_seqlens_k);
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = (p.dtype == FA_F32) ? fa::launch_fwd_f32(a, st) : fa::launch_fwd_mfma(a, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_bwd_varlen_workspace_size(const fa_varlen_params* params, size_t* bytes) {
  fa_params p;
  fa_status s = check_varlen(params, &p);
  if (s != FA_OK) return s;
  if (!bytes) return fail(FA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = varlen_ws_bytes(&p, params);
  return FA_OK;
}

fa_status fa_bwd_varlen(const fa_varlen_params* params, const void* dout, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, void* stream) {
  fa_params p;
  fa_status s = check_varlen(params, &p);
  if (s != FA_OK) return s;
  const bool q_nonempty = p.batch > 0 && params->total_q > 0 && p.seqlen_q > 0;
  const bool kv_nonempty = p.batch > 0 && params->total_k > 0 && p.seqlen_k > 0;
  if ((s = check_ptr(dout, "dout", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(q, "q", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(k, "k", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(v, "v", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(o, "o", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(dq, "dq", q_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(dk, "dk", kv_nonempty)) != FA_OK) return s;
  if ((s = check_ptr(dv, "dv", kv_nonempty)) != FA_OK) return s;
  if ((s = check_offsets(cu_seqlens_q, "cu_seqlens_q", q_nonempty || kv_nonempty)) != FA_OK) return s;
  if ((s = check_offsets(cu_seqlens_k, "cu_seqlens_k", q_nonempty || kv_nonempty)) != FA_OK) return s;
  const size_t need = varlen_ws_bytes(&p, params);
  if (need > 0) {
    if ((s = check_ptr(workspace, "workspace", true)) != FA_OK) return s;
    if (workspace_bytes < need)
      return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  }
  if (q_nonempty || kv_nonempty) {
    const void* outs[3] = {dq, dk, dv};
    const void* ins[6] = {dout, q, k, v, o, lse};
    for (const void* x : outs)
      for (const void* y : ins)
        if (x && x == y) return fail(FA_ERR_INVALID_ARG, "gradient outputs must not alias the inputs");
  }
  if (!q_nonempty && !kv_nonempty) return FA_OK;
  if ((s = check_device()) != FA_OK) return s;
  fa::AttnArgs a = make_varlen_args(&p, params, cu_seqlens_q, cu_seqlens_k);
  a.q = q; a.k = k; a.v = v; a.o = const_cast<void*>(o); a.lse = const_cast<float*>(lse);
  a.dout = dout; a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsum = static_cast<float*>(workspace);
  a.lse2 = a.dsum + varlen_ws_rows(&p, params);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      (p.dtype == FA_F32) ? fa::launch_bwd_f32(a, st, fa::kStageAll) : fa::launch_bwd_mfma(a, st, fa::kStageAll);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status fa_fwd_kvcache_workspace_size(const fa_kvcache_params* params, size_t* bytes) {
  fa_status s = check_kv_params(params);
  if (s != FA_OK) return s;
  if (!bytes) return fail(FA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = kv_workspace_bytes(params);
  return FA_OK;
}

}  // extern "C"

namespace {

// Shared by the contiguous and the paged entry points; page_size 0 means a
// contiguous (batch, capacity, nheads_kv, headdim) cache.
fa_status run_kvcache(const fa_kvcache_params* params, int32_t page_size, int64_t num_pages,
                      const int32_t* block_table, int64_t block_table_stride, const void* q, void* k_cache,
                      void* v_cache, const int32_t* cache_seqlens, const void* k_new, const void* v_new, void* o,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  fa_status s = check_kv_params(params);
  if (s != FA_OK) return s;
  const fa_params* p = &params->base;
  if (page_size != 0) {
    if (page_size < 0 || page_size % 32 != 0)
      return fail(FA_ERR_INVALID_ARG, "page_size must be a positive multiple of 32 (got %d)", page_size);
    if (p->seqlen_k % page_size != 0)
      return fail(FA_ERR_INVALID_ARG, "the capacity (seqlen_k = %lld) must be a whole number of pages",
                  (long long)p->seqlen_k);
    if (num_pages < 1 || num_pages > INT32_MAX)
      return fail(FA_ERR_INVALID_ARG, "num_pages must be in [1, 2^31 - 1] (got %lld)", (long long)num_pages);
    if (block_table_stride < p->seqlen_k / page_size)
      return fail(FA_ERR_INVALID_ARG, "block_table_stride (%lld) is below the pages per entry (%lld)",
                  (long long)block_table_stride, (long long)(p->seqlen_k / page_size));
  }

  const bool nonempty = p->batch > 0 && p->seqlen_q > 0;
  if (!nonempty) return FA_OK;
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(FA_ERR_INVALID_ARG, "k_new and v_new must both be given or both be NULL");
  const bool has_cache = p->seqlen_k > 0;
  if ((s = check_ptr(q, "q", true)) != FA_OK) return s;
  if ((s = check_ptr(k_cache, "k_cache", has_cache)) != FA_OK) return s;
  if ((s = check_ptr(v_cache, "v_cache", has_cache)) != FA_OK) return s;
  if ((s = check_ptr(o, "o", true)) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse", true)) != FA_OK) return s;
  if ((s = check_ptr(k_new, "k_new", k_new != nullptr)) != FA_OK) return s;
  if ((s = check_ptr(v_new, "v_new", v_new != nullptr)) != FA_OK) return s;
  if (k_new && p->seqlen_q > 1) {  // new rows must not overlap (as in check_params)
    const int64_t* ns[2] = {params->knew_strides, params->vnew_strides};
    const char* nn[2] = {"knew", "vnew"};
    for (int t = 0; t < 2; ++t)
      if (ns[t][1] < p->headdim)
        return fail(FA_ERR_UNSUPPORTED, "%s_strides[1]=%lld is below headdim (%lld): rows would overlap", nn[t],
                    (long long)ns[t][1], (long long)p->headdim);
  }
  if (!cache_seqlens) return fail(FA_ERR_INVALID_ARG, "cache_seqlens is NULL");
  if (page_size != 0) {
    if (!block_table) return fail(FA_ERR_INVALID_ARG, "block_table is NULL");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
      return fail(FA_ERR_UNSUPPORTED, "block_table is not 4-byte aligned");
  }
  if ((reinterpret_cast<uintptr_t>(cache_seqlens) & 3u) != 0)
    return fail(FA_ERR_UNSUPPORTED, "cache_seqlens is not 4-byte aligned");
  const size_t need = kv_workspace_bytes(params);
  if ((s = check_ptr(workspace, "workspace", true)) != FA_OK) return s;
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  {
    const void* ins[5] = {q, k_cache, v_cache, k_new, v_new};
    for (const void* y : ins)
      if (y && (y == o || y == lse)) return fail(FA_ERR_INVALID_ARG, "o and lse must not alias the inputs");
  }
  const int64_t G = p->nheads_q / p->nheads_kv;
  const int64_t n_rb = (G * p->seqlen_q + 31) / 32;
  const int64_t S = kv_parts(params);
  const int64_t n_split = p->batch * p->nheads_kv * n_rb * S;
  const int64_t n_append =
      k_new ? (2 * p->batch * p->seqlen_q * p->nheads_kv * (p->headdim / 8) + 63) / 64 : 0;
  if (n_split + n_append >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "launch grid would exceed 2^31 workgroups");
  if ((s = check_device()) != FA_OK) return s;

  fa::KvArgs k{};
  k.q = q; k.k_cache = k_cache; k.v_cache = v_cache; k.k_new = k_new; k.v_new = v_new;
  k.o = o; k.lse = lse; k.cache_seqlens = cache_seqlens;
  const size_t rows = (size_t)p->batch * (size_t)p->nheads_q * (size_t)p->seqlen_q;
  k.ws_o = static_cast<float*>(workspace);
  k.ws_lse = k.ws_o + rows * (size_t)S * (size_t)kernel_headdim(p->headdim);
  k.q_sb = p->q_strides[0]; k.q_sn = p->q_strides[1]; k.q_sh = p->q_strides[2];
  k.kc_sb = p->k_strides[0]; k.kc_sn = p->k_strides[1]; k.kc_sh = p->k_strides[2];
  k.vc_sb = p->v_strides[0]; k.vc_sn = p->v_strides[1]; k.vc_sh = p->v_strides[2];
  k.kn_sb = params->knew_strides[0]; k.kn_sn = params->knew_strides[1]; k.kn_sh = params->knew_strides[2];
  k.vn_sb = params->vnew_strides[0]; k.vn_sn = params->vnew_strides[1]; k.vn_sh = params->vnew_strides[2];
  k.o_sb = p->o_strides[0]; k.o_sn = p->o_strides[1]; k.o_sh = p->o_strides[2];
  k.B = (int32_t)p->batch; k.Nq = (int32_t)p->seqlen_q; k.cap = (int32_t)p->seqlen_k;
  k.Hq = (int32_t)p->nheads_q; k.Hkv = (int32_t)p->nheads_kv; k.G = (int32_t)G; k.D = (int32_t)p->headdim;
  k.dtype = p->dtype == FA_F16 ? fa::kF16 : fa::kBF16;
  k.scale = p->scale;
  k.scale_log2 = p->scale * fa::kLog2e;
  k.causal = p->causal; k.wl = p->window_left; k.wr = p->window_right;
  k.append = k_new != nullptr;
  k.alibi = p->alibi_slopes;
  k.alibi_sb = p->alibi_batch_stride;
  k.score_cap = p->softcap > 0.f ? p->softcap / p->scale : INFINITY;
  k.inv_scale = 1.f / p->scale;
  k.mod = (p->alibi_slopes != nullptr || p->softcap > 0.f) ? 1 : 0;
  k.S = (int32_t)S;
  k.n_rb = (int32_t)n_rb;
  k.n_split = (int32_t)n_split;
  k.n_append = (int32_t)n_append;
  k.block_table = block_table;
  k.bt_sb = block_table_stride;
  k.page_size = page_size;
  k.num_pages = (int32_t)num_pages;
  const hipError_t e = fa::launch_kvcache(k, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kv-cache launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_kvcache(const fa_kvcache_params* params, const void* q, void* k_cache, void* v_cache,
                         const int32_t* cache_seqlens, const void* k_new, const void* v_new, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return run_kvcache(params, 0, 0, nullptr, 0, q, k_cache, v_cache, cache_seqlens, k_new, v_new, o, lse, workspace,
                     workspace_bytes, stream);
}

fa_status fa_fwd_kvcache_paged(const fa_kvcache_params* params, int32_t page_size, int64_t num_pages,
                               const int32_t* block_table, int64_t block_table_stride, const void* q, void* k_cache,
                               void* v_cache, const int32_t* cache_seqlens, const void* k_new, const void* v_new,
                               void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (page_size == 0) return fail(FA_ERR_INVALID_ARG, "page_size must be a positive multiple of 32 (got 0)");
  return run_kvcache(params, page_size, num_pages, block_table, block_table_stride, q, k_cache, v_cache,
                     cache_seqlens, k_new, v_new, o, lse, workspace, workspace_bytes, stream);
}

const char* fa_status_string(fa_status status) {
  // Any int may arrive from C; take the raw bits (see check_params).
  int32_t raw;
  static_assert(sizeof status == sizeof raw, "fa_status is a 32-bit enum");
  std::memcpy(&raw, &status, sizeof raw);
  switch (raw) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_STATUS_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error.c_str(); }

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
