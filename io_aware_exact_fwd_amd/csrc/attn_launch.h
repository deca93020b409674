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

// Packed batches of up to this many sequences are launched over their real
// blocks only (the kernels enumerate them from the boundary table, heaviest
// first); larger ones take the plain (batch, head, block) grid.
constexpr int kMaxPackedSeqs = 512;

// Workgroups for `heads` x blocks of BS rows over B sequences: `plain` (every
// sequence as long as the longest), or for a packed batch of at most
// kMaxPackedSeqs sequences the smaller bound heads * (ceil(T / BS) + B) on its
// real blocks (sum over b of ceil(len_b / BS) <= T / BS + B whenever the
// boundaries rise; rows a malformed table would add past that are not
// computed, as with any malformed table).
inline long long packed_grid(const Packing& p, int B, int heads, int BS, long long plain) {
  if (!p.cu || B > kMaxPackedSeqs) return plain;
  const long long bound = (long long)heads * (((long long)p.T + BS - 1) / BS + B);
  return bound < plain ? bound : plain;
}

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
  // dK/dV head split: the Hq/Hkv query heads of a K/V head are shared out
  // over kv_splits workgroups per key block, each writing fp32 partial sums
  // [kv_splits, 2 (dK unscaled, dV), B*Hkv*N (packed: Hkv*T), d] to `part`;
  // a reduction adds them in split order.  1 = one workgroup sums all heads
  // and writes bf16.
  int kv_splits = 1;
  float* part = nullptr;
  // query rows over all heads: B*Hq*N, or Hq*T when packed
  size_t rows() const { return pack.cu ? (size_t)Hq * pack.T : (size_t)B * Hq * N; }
};

// Keys per 8-wave dK/dV workgroup of the backward (d = 128; d = 64 runs
// 4-wave workgroups of half as many keys, two of them per CU).
constexpr int kBwdKeysPerBlock = 128;

// dK/dV head splits for a fixed-length problem.  Each dK/dV workgroup sums
// over all G = Hq/Hkv query heads of its K/V head, so with few K/V heads the
// U = B*Hkv*ceil(N/128) workgroups (counted in 128-key blocks, one resident
// per CU; at d = 64 twice as many 64-key ones, two per CU, the same ratio)
// are too few to fill 256 CUs, or their longest outlast the rest of the
// launch.  Splitting the heads S ways makes S*U workgroups of 1/S the work,
// at the price of 16*d bytes of fp32 partial sums written and read back per
// key row, K/V head and split.
//  - Causal, no window: block sizes fall linearly (heaviest first), and the
//    idle tail of the launch is about a fifth of the work times 256 / (S*U).
//    With the partials' traffic (both grow as N*d) the cost is, up to one
//    factor, S + 16 G / (B*Hkv*S) whatever N and d -- least at
//    S^2 = 16 G / (B*Hkv) -- and S is the divisor of G that minimises it
//    (the smaller one on a tie).  Splits past 2048 blocks (eight per CU)
//    are not taken once the chip is full: there the tail is already short
//    and the partials and per-block set-up cost more than the model's tail
//    term says (every measured shape's best S kept S*U <= 2048).
//  - Otherwise every block carries the same work and one full wave of
//    blocks suffices: the smallest divisor of G with S*U >= 256.
// The rule over bh = B*Hkv (independent K/V heads of the longest length) and
// U dK/dV blocks of 128 keys.
inline int bwd_kv_splits_rule(int G, long long bh, long long units, bool causal_plain) {
  if (G < 2) return 1;
  int S = 1;
  if (causal_plain) {
    // cost(s) * B*Hkv = s*B*Hkv + 16 G / s, compared as s^2*B*Hkv + 16 G over s
    long long best_num = bh + 16LL * G, best_den = 1;
    for (int s = 2; s <= G; ++s) {
      if (G % s != 0 || (units * s > 2048 && units * S >= 256)) continue;
      const long long num = (long long)s * s * bh + 16LL * G;
      if (num * best_den < best_num * s) {
        best_num = num;
        best_den = s;
        S = s;
      }
    }
  } else {
    for (int s = 2; s <= G && units * S < 256; ++s)
      if (G % s == 0) S = s;
  }
  return S;
}

inline int bwd_kv_splits(int B, int Hq, int Hkv, int N, bool causal, int window) {
  const long long bh = (long long)B * Hkv;
  const long long units = bh * ((N + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock);
  const bool local = window >= 0 && window < N - 1;
  return bwd_kv_splits_rule(Hq / Hkv, bh, units, causal && !local);
}

// A packed batch of `total` rows whose longest sequence has max_seqlen: about
// Hkv*total/128 dK/dV blocks (one more per sequence at most, for ragged
// ends), and the causal model takes it as ceil(total / max_seqlen)
// sequences of the longest length.
inline int bwd_kv_splits_packed(int total, int max_seqlen, int Hq, int Hkv, bool causal,
                                int window) {
  if (total <= 0 || max_seqlen <= 0) return 1;
  const long long seqs = ((long long)total + max_seqlen - 1) / max_seqlen;
  const long long units = (long long)Hkv * (((long long)total + kBwdKeysPerBlock - 1) / kBwdKeysPerBlock);
  const bool local = window >= 0 && window < max_seqlen - 1;
  return bwd_kv_splits_rule(Hq / Hkv, seqs * Hkv, units, causal && !local);
}

// The most splits any mask takes for this shape: the workspace holds that many.
inline int bwd_kv_splits_max(int B, int Hq, int Hkv, int N) {
  const int a = bwd_kv_splits(B, Hq, Hkv, N, true, -1);
  const int b = bwd_kv_splits(B, Hq, Hkv, N, false, -1);
  return a > b ? a : b;
}

// Bytes of the fp32 D rows at the head of the backward's workspace, rounded
// up so that the partial sums after them start 256-byte aligned.
inline size_t bwd_delta_bytes(int B, int Hq, int N) {
  return ((size_t)B * Hq * N * sizeof(float) + 255) & ~(size_t)255;
}

// Bytes of workspace the backward uses: fp32 D per query row, then the head
// split's partial sums (2 fp32 d-vectors per key row and split).
inline size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
  const int S = bwd_kv_splits_max(B, Hq, Hkv, N);
  const size_t part = S > 1 ? (size_t)S * 2 * B * Hkv * N * d * sizeof(float) : 0;
  return bwd_delta_bytes(B, Hq, N) + part;
}

// A packed batch: D over Hq*total rows (rounded to 256 bytes), and the
// partials of S splits over Hkv*total key rows.
inline size_t bwd_varlen_workspace_bytes(int total, int Hq, int Hkv, int d, int S) {
  const size_t part = S > 1 ? (size_t)S * 2 * Hkv * total * d * sizeof(float) : 0;
  return bwd_delta_bytes(1, Hq, total) + part;
}
inline int bwd_kv_splits_packed_max(int total, int max_seqlen, int Hq, int Hkv) {
  const int a = bwd_kv_splits_packed(total, max_seqlen, Hq, Hkv, true, -1);
  const int b = bwd_kv_splits_packed(total, max_seqlen, Hq, Hkv, false, -1);
  return a > b ? a : b;
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
// Bytes of the library's static decode scratch (one copy per GPU).
constexpr size_t kDecodeStaticScratchBytes = size_t{32} << 20;
// Device address of the current GPU's static decode scratch, looked up on the
// first call on each device and cached.  The scratch needs no clearing: every
// decode launch writes each partial it later reads.
hipError_t decode_static_scratch(float** out);
// The backward's stages.  Each reads the BwdArgs fields it needs (delta must
// be set for all of them).  launch_bwd_grads runs dK/dV and dQ in one launch,
// followed by the reduction of the partial sums when kv_splits > 1
// (launch_bwd_dkdv ignores kv_splits); launch_bwd is launch_bwd_pre followed
// by launch_bwd_grads.
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_grads(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace attn
