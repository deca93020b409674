// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>

namespace attn {

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
  float* delta;  // workspace: D_i = rowsum(dO * O), fp32 [B, Hq, N]
  int B, Hq, Hkv, N, d;
  bool causal;
  float scale;
  int window = -1;  // sliding window: keys with |i - j| <= window; < 0 = none
};

// Bytes of workspace the backward uses (fp32 D per query row).
inline size_t bwd_workspace_bytes(int B, int Hq, int N) {
  return (size_t)B * Hq * N * sizeof(float);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

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
