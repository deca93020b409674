// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdint>

namespace attn {

// Packed variable-length batches: tensors are [H, T, d] with the B sequences
// concatenated along T, and sequence b is rows cu[b] .. cu[b+1]-1 of every
// head (LSE and D: [H, T]).  cu == nullptr means fixed-length [B, H, N, d]
// tensors.  With a packing, N is the longest sequence (it sizes the grid).
struct Packing {
  const int* cu = nullptr;  // B + 1 boundaries, device memory
  int T = 0;                // packed rows per head
};

// Allows `bytes` of dynamic LDS (more than the default 64 KB) for `kern` on
// the current device.  The attribute is set once per device; `done` is the
// caller's per-kernel mask of devices already set (devices 0..63).
inline hipError_t allow_lds_on_device(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Whether a grid over `units` (batch, head) pairs keeps all blocks of a pair
// on one XCD (workgroup w runs on XCD w % 8).  That keeps a pair's K/V tiles in
// one L2 and balances the XCDs when every pair carries the same work.  Packed
// batches do not (pairs of a long sequence carry more), so they keep the plain
// order, where block w goes to XCD (w mod units) mod 8: with units a multiple
// of 8 each XCD then gets the same heads of every sequence.
inline int xcd_remap(int units, const Packing& p) { return (units % 8 == 0 && !p.cu) ? 1 : 0; }

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  int window = -1;  // sliding window: keys with |i - j| <= window; < 0 = none
  Packing pack;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: D_i = rowsum(dO * O), fp32 [B, Hq, N] (packed: [Hq, T])
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  int window = -1;  // sliding window: keys with |i - j| <= window; < 0 = none
  Packing pack;
  // query rows over all heads: B*Hq*N, or Hq*T when packed
  size_t rows() const { return pack.cu ? (size_t)Hq * pack.T : (size_t)B * Hq * N; }
};

// Bytes of workspace the backward uses (fp32 D per query row).
inline size_t bwd_workspace_bytes(int B, int Hq, int N) {
  return (size_t)B * Hq * N * sizeof(float);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// Forward over 8-bit (OCP E4M3) Q, K, V [B, H, N, d=128] with fp32 descales
// [B, Hq] (q) and [B, Hkv] (k, v); O bf16, LSE fp32 as launch_fwd.
struct Fp8FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
};

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);

// Decoding against a KV cache: q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d], Nq <= Nk,
// queries at the last Nq positions.  Keys are split into n_splits chunks of
// `chunk` keys (a multiple of 128); workspace holds the per-chunk partials.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  bool causal;
  float scale;
  int window;      // < 0: none
  int n_splits;
  int chunk;
  float* workspace;
};
// The chunking the decode launch uses for a requested split count (<= 0: pick
// one); returns the number of chunks and sets *chunk.
int decode_splits(int B, int Hq, int Hkv, int Nq, int Nk, int requested, int* chunk);
inline size_t decode_workspace_bytes(int B, int Hq, int Nq, int d, int n_splits) {
  return (size_t)n_splits * B * Hq * Nq * (d + 1) * sizeof(float);
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// The backward's stages.  Each reads the BwdArgs fields it needs (delta must
// be set for all of them).  launch_bwd_grads runs dK/dV and dQ in one launch;
// launch_bwd is launch_bwd_pre followed by launch_bwd_grads.
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace attn
