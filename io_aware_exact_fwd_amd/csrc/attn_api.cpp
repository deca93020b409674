// attn_api.cpp -- the C ABI declared in include/attn.h.
//
// Validation happens first and makes no HIP call, so every argument error
// comes back before any device work and without a device present.  There is
// no fallback path: an unsupported case is an error code, never a slower
// kernel (page "从“算力黑洞”到“效率革命”：大模型Attention的演进之路", §7, pitfall 1:
// a silent fallback to an inefficient implementation).
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"
#include "attn_launch.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded on this thread";

int hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d (%s) in %s", (int)e,
                hipGetErrorString(e), where);
  return ATTN_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_problem(int B, int Hq, int Hkv, int N, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if ((long long)N * d > INT_MAX) return ATTN_ERR_SHAPE;
  if ((long long)B * Hq * N > INT_MAX) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int check_scale(float scale) {
  return (std::isfinite(scale) && scale > 0.f) ? ATTN_OK : ATTN_ERR_SCALE;
}

// Per-device architecture cache: 0 unknown, 1 gfx950, 2 something else.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int device_check_impl(int device) {
  if (device < 0) return ATTN_ERR_UNSUPPORTED;
  if (device < kMaxDevices) {
    const int c = g_arch_ok[device].load(std::memory_order_relaxed);
    if (c == 1) return ATTN_OK;
    if (c == 2) return ATTN_ERR_UNSUPPORTED;
  }
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
  if (device >= count) return ATTN_ERR_UNSUPPORTED;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (device < kMaxDevices) g_arch_ok[device].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

int current_device_check() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return device_check_impl(dev);
}

int check_window(int window) { return window >= 0 ? ATTN_OK : ATTN_ERR_SHAPE; }

// window < 0: no window (the plain entry points); >= 0: checked by callers.
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int N, int d, int causal, int window, float scale, void* stream,
             const char* where) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_problem(B, Hq, Hkv, N, d);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_UNSUPPORTED;
  if ((rc = check_scale(scale))) return rc;
  if ((rc = current_device_check())) return rc;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, d, causal != 0, scale, window};
  hipError_t e = attn::launch_fwd(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, where);
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
             int window, float scale, void* stream, const char* where) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return ATTN_ERR_NULL;
  int rc = check_problem(B, Hq, Hkv, N, d);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if (workspace_bytes < attn::bwd_workspace_bytes(B, Hq, Hkv, N, d)) return ATTN_ERR_WORKSPACE;
  if ((rc = check_scale(scale))) return rc;
  if ((rc = current_device_check())) return rc;
  attn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace,
                  B, Hq, Hkv, N, d, causal != 0, scale, window};
  // the head split's partial sums follow D in the workspace
  a.kv_splits = attn::bwd_kv_splits(B, Hq, Hkv, N, causal != 0, window);
  a.part = (float*)((char*)workspace + attn::bwd_delta_bytes(B, Hq, N));
  hipError_t e = attn::launch_bwd(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, where);
}

}  // namespace

ATTN_EXPORT int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                         void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, -1, scale, stream,
                  "attn_fwd launch");
}

ATTN_EXPORT int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int N, int d, int causal, int window,
                                float scale, void* stream) {
  if (check_window(window)) return ATTN_ERR_SHAPE;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, stream,
                  "attn_fwd_window launch");
}

ATTN_EXPORT size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  if (check_problem(B, Hq, Hkv, N, d)) return 0;
  return attn::bwd_workspace_bytes(B, Hq, Hkv, N, d);
}

ATTN_EXPORT int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                         int N, int d, int causal, float scale, void* stream) {
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N,
                  d, causal, -1, scale, stream, "attn_bwd launch");
}

ATTN_EXPORT int attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                                int N, int d, int causal, int window, float scale, void* stream) {
  if (check_window(window)) return ATTN_ERR_SHAPE;
  return bwd_impl(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N,
                  d, causal, window, scale, stream, "attn_bwd_window launch");
}

ATTN_EXPORT int attn_bwd_preprocess(const void* o, const void* dout, float* delta, int B, int Hq,
                                    int N, int d, void* stream) {
  if (!o || !dout || !delta) return ATTN_ERR_NULL;
  int rc = check_problem(B, Hq, Hq, N, d);
  if (rc) return rc;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return ATTN_ERR_UNSUPPORTED;
  if ((rc = current_device_check())) return rc;
  attn::BwdArgs a{};
  a.o = o;
  a.dout = dout;
  a.delta = delta;
  a.B = B, a.Hq = Hq, a.Hkv = Hq, a.N = N, a.d = d;
  hipError_t e = attn::launch_bwd_pre(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_preprocess launch");
}

// Shared checks of the recomputing stages (out1..out3 are their outputs).
static int check_stage(const void* q, const void* k, const void* v, const void* dout,
                       const float* lse, const float* delta, const void* out1, const void* out2,
                       const void* out3, int B, int Hq, int Hkv, int N, int d, float scale) {
  if (!q || !k || !v || !dout || !lse || !delta || !out1 || !out2 || !out3) return ATTN_ERR_NULL;
  int rc = check_problem(B, Hq, Hkv, N, d);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, dout, lse, delta, out1, out2, out3};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if ((rc = check_scale(scale))) return rc;
  return current_device_check();
}

ATTN_EXPORT int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, const float* delta, void* dk, void* dv, int B,
                              int Hq, int Hkv, int N, int d, int causal, float scale,
                              void* stream) {
  int rc = check_stage(q, k, v, dout, lse, delta, dk, dv, dv, B, Hq, Hkv, N, d, scale);
  if (rc) return rc;
  attn::BwdArgs a{q, k, v, nullptr, lse, dout, nullptr, dk, dv, (float*)delta,
                  B, Hq, Hkv, N, d, causal != 0, scale};
  hipError_t e = attn::launch_bwd_dkdv(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_dkdv launch");
}

ATTN_EXPORT int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, const float* delta, void* dq, int B, int Hq,
                            int Hkv, int N, int d, int causal, float scale, void* stream) {
  int rc = check_stage(q, k, v, dout, lse, delta, dq, dq, dq, B, Hq, Hkv, N, d, scale);
  if (rc) return rc;
  attn::BwdArgs a{q, k, v, nullptr, lse, dout, dq, nullptr, nullptr, (float*)delta,
                  B, Hq, Hkv, N, d, causal != 0, scale};
  hipError_t e = attn::launch_bwd_dq(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_dq launch");
}

ATTN_EXPORT int attn_bwd_grads(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, const float* delta, void* dq, void* dk,
                               void* dv, int B, int Hq, int Hkv, int N, int d, int causal,
                               float scale, void* stream) {
  int rc = check_stage(q, k, v, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, N, d, scale);
  if (rc) return rc;
  attn::BwdArgs a{q, k, v, nullptr, lse, dout, dq, dk, dv, (float*)delta,
                  B, Hq, Hkv, N, d, causal != 0, scale};
  hipError_t e = attn::launch_bwd_grads(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_grads launch");
}

ATTN_EXPORT int attn_bwd_grads_window(const void* q, const void* k, const void* v,
                                      const void* dout, const float* lse, const float* delta,
                                      void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                                      int N, int d, int causal, int window, float scale,
                                      void* stream) {
  if (check_window(window)) return ATTN_ERR_SHAPE;
  int rc = check_stage(q, k, v, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, N, d, scale);
  if (rc) return rc;
  attn::BwdArgs a{q, k, v, nullptr, lse, dout, dq, dk, dv, (float*)delta,
                  B, Hq, Hkv, N, d, causal != 0, scale, window};
  hipError_t e = attn::launch_bwd_grads(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_grads_window launch");
}

// Shapes of a decode call: Nq queries (the last Nq positions) against Nk keys.
static int check_decode(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || Nq > Nk) return ATTN_ERR_SHAPE;
  if ((long long)Nk * d > INT_MAX) return ATTN_ERR_SHAPE;
  if ((long long)B * Hq * Nq * (d + 1) > INT_MAX) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

ATTN_EXPORT size_t attn_fwd_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                                   int num_splits) {
  if (check_decode(B, Hq, Hkv, Nq, Nk, d)) return 0;
  int chunk = 0;
  const int splits = attn::decode_splits(B, Hq, Hkv, Nq, Nk, num_splits, &chunk);
  return attn::decode_workspace_bytes(B, Hq, Nq, d, splits);
}

ATTN_EXPORT int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                                int window, float scale, int num_splits, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return ATTN_ERR_NULL;
  int rc = check_decode(B, Hq, Hkv, Nq, Nk, d);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, o, lse, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  int chunk = 0;
  const int splits = attn::decode_splits(B, Hq, Hkv, Nq, Nk, num_splits, &chunk);
  if (workspace_bytes < attn::decode_workspace_bytes(B, Hq, Nq, d, splits)) return ATTN_ERR_WORKSPACE;
  if ((rc = check_scale(scale))) return rc;
  if ((rc = current_device_check())) return rc;
  attn::DecodeArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal != 0, scale,
                     window < 0 ? -1 : window, splits, chunk, (float*)workspace};
  hipError_t e = attn::launch_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_fwd_decode launch");
}

ATTN_EXPORT int attn_fwd_decode_static(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                       int causal, int window, float scale, int num_splits,
                                       void* stream) {
  static_assert(attn::kDecodeStaticScratchBytes == ATTN_DECODE_STATIC_SCRATCH_BYTES,
                "header and library agree on the static scratch size");
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_decode(B, Hq, Hkv, Nq, Nk, d);
  if (rc) return rc;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  int chunk = 0;
  const int splits = attn::decode_splits(B, Hq, Hkv, Nq, Nk, num_splits, &chunk);
  if (attn::decode_workspace_bytes(B, Hq, Nq, d, splits) > attn::kDecodeStaticScratchBytes)
    return ATTN_ERR_SCRATCH;
  if ((rc = check_scale(scale))) return rc;
  if ((rc = current_device_check())) return rc;
  float* scratch = nullptr;
  hipError_t e = attn::decode_static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "attn_fwd_decode_static scratch lookup");
  attn::DecodeArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal != 0, scale,
                     window < 0 ? -1 : window, splits, chunk, scratch};
  e = attn::launch_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_fwd_decode_static launch");
}

// Shapes of a packed variable-length call: B sequences, `total` packed rows per
// head, none longer than max_seqlen.  total == 0 is an empty batch.
static int check_varlen(int B, int total, int max_seqlen, int Hq, int Hkv, int d) {
  if (B <= 0 || total < 0 || max_seqlen < 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || max_seqlen > total || (total > 0 && max_seqlen == 0)) return ATTN_ERR_SHAPE;
  if ((long long)total * d > INT_MAX || (long long)Hq * total > INT_MAX) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

ATTN_EXPORT int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* cu_seqlens, int B, int total, int max_seqlen, int Hq,
                                int Hkv, int d, int causal, int window, float scale,
                                void* stream) {
  int rc = check_varlen(B, total, max_seqlen, Hq, Hkv, d);
  if (rc) return rc;
  if ((rc = check_scale(scale))) return rc;
  if (total == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return ATTN_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if ((rc = current_device_check())) return rc;
  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen, d, causal != 0, scale,
                  window < 0 ? -1 : window};
  a.pack = attn::Packing{cu_seqlens, total};
  hipError_t e = attn::launch_fwd(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_fwd_varlen launch");
}

ATTN_EXPORT size_t attn_bwd_varlen_workspace_bytes(int Hq, int total, int d) {
  if (Hq <= 0 || total < 0 || (long long)Hq * total > INT_MAX || (d != 64 && d != 128)) return 0;
  return (size_t)Hq * total * sizeof(float);
}

ATTN_EXPORT size_t attn_bwd_varlen_split_workspace_bytes(int B, int total, int max_seqlen, int Hq,
                                                         int Hkv, int d) {
  if (check_varlen(B, total, max_seqlen, Hq, Hkv, d)) return 0;
  return attn::bwd_varlen_workspace_bytes(
      total, Hq, Hkv, d, attn::bwd_kv_splits_packed_max(total, max_seqlen, Hq, Hkv));
}

ATTN_EXPORT int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                const int* cu_seqlens, void* workspace, size_t workspace_bytes,
                                int B, int total, int max_seqlen, int Hq, int Hkv, int d,
                                int causal, int window, float scale, void* stream) {
  int rc = check_varlen(B, total, max_seqlen, Hq, Hkv, d);
  if (rc) return rc;
  if ((rc = check_scale(scale))) return rc;
  if (total == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens || !workspace)
    return ATTN_ERR_NULL;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if (workspace_bytes < (size_t)Hq * total * sizeof(float)) return ATTN_ERR_WORKSPACE;
  if ((rc = current_device_check())) return rc;
  attn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace,
                  B, Hq, Hkv, max_seqlen, d, causal != 0, scale, window < 0 ? -1 : window};
  a.pack = attn::Packing{cu_seqlens, total};
  // the head split, when the workspace has room for its partials after D
  const int S = attn::bwd_kv_splits_packed(total, max_seqlen, Hq, Hkv, causal != 0, a.window);
  if (S > 1 && workspace_bytes >= attn::bwd_varlen_workspace_bytes(total, Hq, Hkv, d, S)) {
    a.kv_splits = S;
    a.part = (float*)((char*)workspace + attn::bwd_delta_bytes(1, Hq, total));
  }
  hipError_t e = attn::launch_bwd(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_varlen launch");
}

ATTN_EXPORT int attn_bwd_grads_varlen(const void* q, const void* k, const void* v,
                                      const void* dout, const float* lse, const float* delta,
                                      void* dq, void* dk, void* dv, const int* cu_seqlens, int B,
                                      int total, int max_seqlen, int Hq, int Hkv, int d,
                                      int causal, int window, float scale, void* stream) {
  int rc = check_varlen(B, total, max_seqlen, Hq, Hkv, d);
  if (rc) return rc;
  if ((rc = check_scale(scale))) return rc;
  if (total == 0) return ATTN_OK;
  if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv || !cu_seqlens)
    return ATTN_ERR_NULL;
  const void* ptrs[] = {q, k, v, dout, lse, delta, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if ((rc = current_device_check())) return rc;
  attn::BwdArgs a{q, k, v, nullptr, lse, dout, dq, dk, dv, (float*)delta,
                  B, Hq, Hkv, max_seqlen, d, causal != 0, scale, window < 0 ? -1 : window};
  a.pack = attn::Packing{cu_seqlens, total};
  hipError_t e = attn::launch_bwd_grads(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_bwd_grads_varlen launch");
}

ATTN_EXPORT int attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                             const float* k_descale, const float* v_descale, void* o, float* lse,
                             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                             void* stream) {
  if (!q || !k || !v || !q_descale || !k_descale || !v_descale || !o || !lse) return ATTN_ERR_NULL;
  int rc = check_problem(B, Hq, Hkv, N, d);
  if (rc) return rc;
  if (d != 128) return ATTN_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_UNSUPPORTED;
  if ((rc = check_scale(scale))) return rc;
  if ((rc = current_device_check())) return rc;
  attn::Fp8FwdArgs a{q, k, v, q_descale, k_descale, v_descale, o, lse, B, Hq, Hkv, N, d,
                     causal != 0, scale};
  hipError_t e = attn::launch_fwd_fp8(a, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e, "attn_fwd_fp8 launch");
}

ATTN_EXPORT const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape: B, Hq, Hkv, N, d must be >= 1, Hq % Hkv == 0, N*d < 2^31";
    case ATTN_ERR_UNSUPPORTED: return "unsupported: d must be 64 or 128, pointers 16-byte aligned, device gfx950";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_bwd_workspace_bytes()";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_HIP: return g_hip_msg;
    case ATTN_ERR_SCRATCH:
      return "the problem needs more than ATTN_DECODE_STATIC_SCRATCH_BYTES (32 MiB) of decode "
             "partials: call attn_fwd_decode with a workspace, or ask for fewer splits";
    default: return "unknown attn error code";
  }
}

ATTN_EXPORT int attn_device_check(int device) { return device_check_impl(device); }
