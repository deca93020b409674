/*
 * attn.h -- C ABI of an IO-aware exact attention library for AMD MI355X (gfx950).
 *
 * The library computes exact scaled dot-product attention
 *
 *     O = softmax(scale * Q K^T + mask) V
 *
 * by tiling Q, K and V along the sequence: each block of query rows streams
 * K/V tiles through on-chip memory while it keeps a running row maximum and
 * row sum, so the N x N score matrix never reaches device memory.  The forward
 * stores only O and the per-row log-sum-exp; the backward recomputes block
 * scores from that log-sum-exp.
 *
 * Sources (web pages, cited by title and section):
 *   [EVOL]    "从“算力黑洞”到“效率革命”：大模型Attention的演进之路" (mhpn.cn)
 *               §2  softmax(QK^T / sqrt(d_k)) V;
 *               §3  multi-query / grouped-query heads sharing K and V;
 *               §4  Flash Attention: tiling, online softmax statistics,
 *                   recomputation in the backward, O(N) memory;
 *               §6  the scaled_dot_product_attention call (query, key, value,
 *                   is_causal) whose problem statement these entry points take;
 *               §7  pitfall 1: a silent fallback to a slow path -- this
 *                   library never falls back; it returns an error instead.
 *   [LONGCTX] "6.1 2023 年代：長上下文擴展技術：FlashAttention、RoPE 與稀疏注意力"
 *             (cccbook) §2.2 tiling plus recomputation, only O and the
 *             log-sum-exp kept by the forward; §2.3 exact, not approximate.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, contiguous, row-major [B, H, N, d] (batch, heads,
 *    sequence, head dim), the tensor layout of the example in [EVOL] §6.
 *    Q, O, dO, dQ have H = Hq heads; K, V, dK, dV have H = Hkv.
 *  - bf16 tensors hold IEEE-style bfloat16 bit patterns (uint16 storage).
 *    The log-sum-exp and the backward's workspace are fp32.
 *  - Grouped heads: query head h reads K/V head h / (Hq / Hkv); Hkv = 1 is
 *    multi-query attention, Hkv = Hq is plain multi-head attention.
 *  - causal != 0 applies the lower-triangular mask: query i attends keys
 *    j <= i (one sequence length N for queries and keys).
 *  - scale multiplies the fp32 scores; the usual value is 1/sqrt(d).
 *  - Every pointer is a device pointer (hipMalloc'd or a torch CUDA tensor),
 *    16-byte aligned.  The caller allocates and owns every buffer, including
 *    the workspace; the library allocates and frees nothing and keeps no
 *    per-call state.
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).
 *    Arguments are validated synchronously, before any HIP call; kernels are
 *    then enqueued on the stream and the call returns without synchronising.
 *    Outputs are valid once the stream has reached that point.
 *  - Supported: d in {64, 128}, N >= 1 (any length, ragged tails included),
 *    B, Hq, Hkv >= 1 with Hq % Hkv == 0, gfx950 devices only.
 */
#ifndef IO_AWARE_ATTN_H
#define IO_AWARE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ATTN_OK              0  /* success (work enqueued)                          */
#define ATTN_ERR_NULL        1  /* a required pointer is NULL                       */
#define ATTN_ERR_SHAPE       2  /* B, Hq, Hkv, N or d <= 0, Hq % Hkv != 0, or one
                                   head's N*d elements would not fit in 2^31 - 1    */
#define ATTN_ERR_UNSUPPORTED 3  /* d not in {64,128}, a pointer not 16-byte aligned,
                                   or the current device is not gfx950              */
#define ATTN_ERR_WORKSPACE   4  /* workspace smaller than attn_bwd_workspace_bytes  */
#define ATTN_ERR_SCALE       5  /* scale not finite or not > 0                      */
#define ATTN_ERR_HIP         6  /* a HIP runtime call or kernel launch failed; the
                                   message is available from attn_strerror(6)       */
#define ATTN_ERR_SCRATCH     7  /* attn_fwd_decode_static: the problem's partials
                                   exceed ATTN_DECODE_STATIC_SCRATCH_BYTES         */

/*
 * Forward pass ([EVOL] §4, [LONGCTX] §2.2).
 *   q    [B, Hq,  N, d] bf16, read
 *   k, v [B, Hkv, N, d] bf16, read
 *   o    [B, Hq,  N, d] bf16, written: softmax(scale*QK^T + mask) V, rounded
 *        to nearest-even bf16
 *   lse  [B, Hq,  N]    fp32, written: LSE_i = ln sum_{j visible} exp(scale*q_i.k_j),
 *        natural log of the scaled scores, masked keys excluded
 * o and lse must not alias the inputs.  Returns ATTN_OK or an error code; on
 * an error nothing is enqueued and no output is touched.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
             void* stream);

/*
 * Bytes of device workspace attn_bwd and attn_bwd_window need for this
 * problem: linear in N, never O(N^2) ([EVOL] §4: memory goes from O(N^2) to
 * O(N)).  It holds D = rowsum(dO * O), one fp32 per query row (B*Hq*N*4 bytes,
 * rounded up to a multiple of 256), and, when Hq > Hkv and the library shares
 * the Hq/Hkv query heads of each K/V head out over S workgroups, their fp32
 * partial dK and dV (S*2*B*Hkv*N*d*4 more bytes).  Returns 0 when the arguments
 * are invalid.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/*
 * Backward pass with recomputation from the saved log-sum-exp ([LONGCTX] §2.2,
 * [EVOL] §4): consumes only the inputs, the forward's O and LSE, and dO.
 *   q, o, dout [B, Hq,  N, d] bf16, read (o and lse from attn_fwd with the
 *                                  same inputs, causal flag and scale)
 *   k, v       [B, Hkv, N, d] bf16, read
 *   lse        [B, Hq,  N]    fp32, read
 *   dq         [B, Hq,  N, d] bf16, written: dL/dQ for L = sum(dO * O)
 *   dk, dv     [B, Hkv, N, d] bf16, written: dL/dK, dL/dV, summed over the
 *                                  Hq/Hkv query heads that share each K/V head
 *   workspace  device buffer of workspace_bytes >= attn_bwd_workspace_bytes();
 *              its contents on entry are ignored and on exit are unspecified.
 * Outputs must not alias inputs or each other.  Deterministic: the same
 * inputs give bitwise the same outputs.  With the head split (workspace bytes
 * beyond the rounded B*Hq*N*4), dK and dV are the fp32 per-split sums added in
 * split order, then rounded to bf16.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
             void* stream);

/*
 * The stages of attn_bwd, for callers that schedule them themselves.  attn_bwd
 * is attn_bwd_preprocess followed by attn_bwd_grads, bitwise, whenever
 * attn_bwd_workspace_bytes is the rounded B*Hq*N*4 (no head split); otherwise
 * dQ is still bitwise equal, and dK and dV, which the stages sum over all
 * query heads in one workgroup, differ from attn_bwd's by fp32 rounding of the
 * summation order (at most about one bf16 unit in the last place).
 * attn_bwd_grads computes bitwise what attn_bwd_dkdv and attn_bwd_dq compute,
 * in one launch.  The
 * gradient stages read only the inputs, the LSE and delta, so they may run on
 * different streams once delta is written.  Same conventions and errors as
 * attn_bwd.
 *
 * attn_bwd_preprocess: delta [B, Hq, N] fp32 (caller-owned, e.g. the first
 *   B*Hq*N*4 bytes of attn_bwd's workspace) = rowsum(dO * O), which equals the
 *   softmax-Jacobian term sum_k P_ik dP_ik of each query row.
 * attn_bwd_dkdv: dK, dV [B, Hkv, N, d] bf16, each summed over the Hq/Hkv query
 *   heads of its group, recomputing probabilities from lse ([LONGCTX] §2.2).
 * attn_bwd_dq: dQ [B, Hq, N, d] bf16, recomputing probabilities from lse.
 * attn_bwd_grads: dQ, dK and dV as the two calls above give them.
 */
int attn_bwd_preprocess(const void* o, const void* dout, float* delta,
                        int B, int Hq, int N, int d, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                  const float* lse, const float* delta, void* dk, void* dv,
                  int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                  void* stream);
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                const float* lse, const float* delta, void* dq,
                int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                void* stream);
int attn_bwd_grads(const void* q, const void* k, const void* v, const void* dout,
                   const float* lse, const float* delta, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   void* stream);

/*
 * Sliding-window attention (page "6.1 2023 年代：長上下文擴展技術：FlashAttention、
 * RoPE 與稀疏注意力", §4): query i attends to key j only when |i - j| <= window,
 * intersected with j <= i when causal != 0.  window counts keys on each side,
 * the query's own key excluded: window = 0 leaves only key i, window >= N - 1
 * gives exactly the plain call.  Arguments, layouts, ownership and errors are
 * those of attn_fwd / attn_bwd / attn_bwd_grads, plus ATTN_ERR_SHAPE for
 * window < 0.  Tiles of keys outside every row's band are neither loaded nor
 * computed, so the work grows with N * window instead of N^2.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, int causal, int window,
                    float scale, void* stream);
int attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes,
                    int B, int Hq, int Hkv, int N, int d, int causal, int window,
                    float scale, void* stream);
int attn_bwd_grads_window(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, const float* delta, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int N, int d, int causal, int window,
                          float scale, void* stream);

/*
 * Forward for decoding against a KV cache (pages "从“算力黑洞”到“效率革命”：
 * 大模型Attention的演进之路", §1 and §3, and "6.1 … 長上下文擴展技術", §1.5): a
 * few new queries attend to a long cached K/V history.  The Nq queries are the
 * last Nq positions of a sequence of Nk (query i at position i + Nk - Nq); the
 * causal mask and the window are taken between positions, so with causal the
 * last query sees every key.  The key axis is split into chunks processed in
 * parallel, and the per-chunk (O, LSE) partials are merged by their
 * log-sum-exp (page "6.1 …", §2.2: the online softmax makes that exact).
 *
 *   q      [B, Hq,  Nq, d] bf16, read;  o [B, Hq, Nq, d] bf16, written
 *   k, v   [B, Hkv, Nk, d] bf16, read (the cache; Nk >= Nq)
 *   lse    [B, Hq, Nq] fp32, written (natural log of the scaled scores)
 *   window < 0: none; >= 0: keys with |pos - j| <= window
 *   num_splits: <= 0 lets the library choose; otherwise an upper bound
 *     (a chunk is a whole number of 128-key tiles, so fewer may be used)
 *   workspace: device buffer of workspace_bytes >= the value
 *     attn_fwd_decode_workspace_bytes returns for the same shapes and
 *     num_splits; contents on entry ignored, on exit unspecified.
 * Errors as attn_fwd, with ATTN_ERR_SHAPE also for Nq > Nk and ATTN_ERR_WORKSPACE
 * for a short workspace.  Deterministic for a fixed num_splits.
 */
size_t attn_fwd_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                       int num_splits);
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int window,
                    float scale, int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * attn_fwd_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It computes exactly what attn_fwd_decode computes (same
 * kernels, same chunking for the same num_splits, bitwise the same outputs),
 * taking the per-chunk partials from a static buffer that the library holds in
 * device memory for the life of the process: ATTN_DECODE_STATIC_SCRATCH_BYTES
 * per GPU, reserved on every GPU the library runs on.  The call allocates
 * nothing and frees nothing.
 *   - Problems whose partials (attn_fwd_decode_workspace_bytes for the same
 *     arguments) exceed that size return ATTN_ERR_SCRATCH before any device
 *     work.
 *   - Every call on one GPU uses that GPU's one buffer: calls that can overlap
 *     on one GPU (different streams, or different host threads without an
 *     ordering between them) race on it and give undefined results; order them
 *     on one stream or with events.  Calls on different GPUs do not interact.
 *   - The buffer needs no initialisation: each call writes every partial it
 *     reads, so the previous call's contents never leak into a result.
 * Arguments, layouts and the other errors are those of attn_fwd_decode.
 */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_fwd_decode_static(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, int window,
                           float scale, int num_splits, void* stream);

/*
 * Packed variable-length batches (page "从“算力黑洞”到“效率革命”：大模型Attention的
 * 演进之路", §6, scenario 2: long-context training data is built by
 * concatenating and packing sequences).  B sequences of different lengths are
 * stored back to back without padding; each is its own attention problem (its
 * queries see only its own keys, positions counted from its first token), so
 * the result equals B separate attn_fwd / attn_bwd calls.
 *
 *   q, o, dout, dq  [Hq,  total, d] bf16    k, v, dk, dv  [Hkv, total, d] bf16
 *   lse             [Hq,  total]   fp32     (natural log of the scaled scores)
 *   cu_seqlens      B + 1 int32 in DEVICE memory: sequence b is rows
 *                   cu_seqlens[b] .. cu_seqlens[b+1] - 1 of every head;
 *                   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[B] = total
 *                   (empty sequences allowed)
 *   max_seqlen      the longest sequence (bounds the grid): 1 <= max_seqlen <= total
 *   window < 0: none; >= 0: as attn_fwd_window, within each sequence
 *   workspace       attn_bwd_varlen: >= attn_bwd_varlen_workspace_bytes(Hq, total, d)
 *                   bytes (fp32 D per packed query row); contents on exit unspecified.
 *                   With at least attn_bwd_varlen_split_workspace_bytes(B, total,
 *                   max_seqlen, Hq, Hkv, d) bytes, attn_bwd_varlen may share the
 *                   Hq/Hkv query heads of each K/V head out over several workgroups
 *                   (as attn_bwd does, with the fp32 partial dK/dV after D in the
 *                   workspace) when the packed dK/dV grid is too short for the chip;
 *                   dQ is the same either way and dK, dV then differ from the
 *                   smaller workspace's by one bf16 unit in the last place at most.
 *                   Either way the result is deterministic for a given workspace
 *                   size class (below or at least the split size).
 *
 * The boundaries live on the device and are not read by the host; with up to
 * 512 sequences each workgroup finds its own (sequence, head, block) among the
 * table's real blocks, heaviest first.  A table that breaks the rules above
 * (or a sequence longer than max_seqlen) cannot make the kernels access memory
 * outside the [H, total, d] tensors -- every boundary is clamped to
 * [0, total] and every length to max_seqlen -- but the rows it describes
 * wrongly are left unspecified.  total = 0 is an empty batch
 * and returns ATTN_OK without touching memory.  Other errors as attn_fwd /
 * attn_bwd (ATTN_ERR_SHAPE also for max_seqlen > total, or total * d or
 * Hq * total beyond 2^31 - 1).  Deterministic, like the fixed-length calls.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int B, int total, int max_seqlen, int Hq, int Hkv,
                    int d, int causal, int window, float scale, void* stream);
size_t attn_bwd_varlen_workspace_bytes(int Hq, int total, int d);
/* Workspace bytes that let attn_bwd_varlen split query heads over workgroups
 * (see `workspace` above): D rounded up to 256 bytes, plus S*2*Hkv*total*d*4
 * for the split count S the shape takes (the larger of the causal and full
 * masks' counts; no extra when S = 1).  Returns 0 for invalid arguments
 * (the rules of attn_bwd_varlen). */
size_t attn_bwd_varlen_split_workspace_bytes(int B, int total, int max_seqlen, int Hq, int Hkv,
                                             int d);
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    const int* cu_seqlens, void* workspace, size_t workspace_bytes,
                    int B, int total, int max_seqlen, int Hq, int Hkv, int d, int causal,
                    int window, float scale, void* stream);
/* The gradient stage of attn_bwd_varlen alone (dK/dV and dQ in one launch), for
 * callers that run the D pre-pass themselves: over packed rows that pass is
 * attn_bwd_preprocess with B = 1, N = total (delta is fp32 [Hq, total]). */
int attn_bwd_grads_varlen(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, const float* delta, void* dq, void* dk, void* dv,
                          const int* cu_seqlens, int B, int total, int max_seqlen, int Hq,
                          int Hkv, int d, int causal, int window, float scale, void* stream);

/*
 * Forward over 8-bit inputs (page "6.1 2023 年代：長上下文擴展技術：FlashAttention、
 * RoPE 與稀疏注意力", §2.3: FlashAttention-3's low-bit path; the method stays
 * exact).  Q, K, V hold OCP E4M3 codes (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; largest value 448; S.1111.111 is NaN), one byte per
 * element; element x of head (b, h) stands for decode(x) * descale[b, h].
 * The result is the attention of those values, computed on the 8-bit matrix
 * unit:
 *
 *   q          [B, Hq,  N, 128] E4M3, read       o   [B, Hq, N, 128] bf16, written
 *   k, v       [B, Hkv, N, 128] E4M3, read       lse [B, Hq, N] fp32, written
 *   q_descale  [B, Hq]  fp32, device, read;  k_descale, v_descale [B, Hkv] fp32, device, read
 *
 * The scores and their softmax statistics are fp32 (LSE as exact as the bf16
 * forward's); the probabilities enter the P V product rounded to E4M3 after
 * scaling by 2^8 (relative error <= 2^-4, absolute <= 2^-18 of the row's
 * largest probability in the subnormal range), so |O - O_exact| <=
 * sum_j max(2^-4 P_ij, 2^-18 max_k P_ik) |v_j| plus O's own bf16 rounding.
 * A NaN code is not an error: it propagates into the outputs of the rows that
 * read it.  Descales live in device memory and are not read by the host: each
 * must be finite, and q_descale * k_descale >= 0 for every head.  A zero
 * descale stands for an all-zero head (zero scores: uniform attention over the
 * visible keys; zero values from v) and is computed exactly; a head whose
 * q_descale * k_descale is negative or not finite gets NaN in its O and LSE
 * rows instead of a silently wrong result.  Errors as attn_fwd, with
 * ATTN_ERR_UNSUPPORTED for d != 128.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                 const float* k_descale, const float* v_descale, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale, void* stream);

/* Static description of a return code; for ATTN_ERR_HIP, the HIP error text
 * of the last failure on the calling thread.  Never NULL.  ([EVOL] §7,
 * pitfall 1: a request the fast path cannot serve must surface as an error the
 * caller can read, not turn silently into a slow fallback; every entry point
 * therefore returns a code, and this call names it.) */
const char* attn_strerror(int code);

/* ATTN_OK when device `device` exists and is a gfx950 part this library was
 * built for; ATTN_ERR_UNSUPPORTED for another architecture; ATTN_ERR_HIP when
 * the device cannot be queried.  ([EVOL] §7: check that the fast kernel is
 * really the one that can run, instead of falling back.) */
int attn_device_check(int device);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* IO_AWARE_ATTN_H */
