/*
 * jfa.h -- C ABI of libjfa.so: jagged exact-softmax attention on AMD MI355X
 * (gfx950), forward and backward.
 *
 * The operation ("Jagged Flash Attention (JFA)", sysdesign-wiki, section
 * "Definition"; tiling and online softmax as in "TLX-Optimized Jagged Flash
 * Attention: Approaching FA4-Level Performance on Blackwell", section "Why
 * Jagged Flash Attention Deserves Attention"): B variable-length sequences are
 * packed back to back with no padding and addressed by prefix-sum offsets.
 * Query and key/value lengths may differ per sequence. For sequence b, head h,
 * local query row i and key row j:
 *
 *   S_ij   = (Q_i . K_j) / sqrt(D) + bias[h][clamp(i - j, -128, 128) + 128]
 *   causal : key j is visible to query i iff j <= i (top-left alignment)
 *   O_i    = sum_j softmax_j(S_ij) V_j,   lse_i = ln sum_j exp(S_ij)
 *   a sequence with no keys gives O_i = 0 and lse_i = -inf.
 *
 * Layouts (all row-major, D contiguous, device memory):
 *   q, out, dout, dq      [total_q,  H, D]   element type T
 *   k, v, dk, dv          [total_kv, H, D]   element type T
 *   lse                   [total_q,  H]      fp32, natural log
 *   q_offsets, kv_offsets [B + 1]            int32, offsets[0] = 0,
 *                                            non-decreasing, offsets[B] = total
 *   bias                  [H, 257]           fp32, or NULL for no bias
 * T is bf16 for jfa_fwd / jfa_bwd and fp32 for jfa_fwd_f32 / jfa_bwd_f32.
 * Accumulation is fp32 in every variant. D must be 32, 64 or 128; H must be
 * 1 .. JFA_MAX_HEADS.
 * Each sequence's slice of one tensor (length * H * D * sizeof(T)) must be
 * below 4 GiB. kv_offsets may alias q_offsets.
 *
 * Ownership: the caller owns every buffer. The library allocates no device
 * memory; scratch space is the caller's `workspace` (size from the
 * *_workspace_bytes queries, 256-byte aligned). All calls are asynchronous on
 * `stream` (a hipStream_t, NULL = default stream): no host synchronisation
 * and no device-to-host reads. Concurrent calls must use distinct
 * workspaces.
 *
 * max_kv_len (jfa_fwd, jfa_bwd and their fp32 twins): an upper bound on every
 * sequence's key count when the caller knows one, else 0 (a negative value
 * is an invalid argument). With a bound of at most 1024 no sequence can take
 * the short-query path described below, whose launches are then skipped and
 * every sequence takes the query-tile and key-tile passes. Those are exact
 * for any lengths, so a bound that is wrong costs speed, never correctness.
 *
 * Errors: every call returns a jfa_status. Invalid arguments are detected on
 * the host before anything is launched (nothing is written then);
 * jfa_last_error() gives a thread-local description of the last failure.
 * Device-side faults surface at the caller's next synchronisation. Offsets
 * that break the preconditions above are not detected; if they make the work
 * list larger than the workspace, no output is written and the list header's
 * status word is set to 1.
 */
#ifndef JFA_H
#define JFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARGUMENT = 1,
  JFA_ERR_WORKSPACE = 2,
  JFA_ERR_UNSUPPORTED = 3,
  JFA_ERR_HIP = 4
} jfa_status;

#define JFA_BIAS_RADIUS 128 /* bias table is [H][2 * JFA_BIAS_RADIUS + 1] */
#define JFA_BIAS_LEN (2 * JFA_BIAS_RADIUS + 1)
#define JFA_MAX_BATCH 8192  /* largest B accepted by one call */
#define JFA_MAX_HEADS 65535 /* largest H accepted by one call */
#define JFA_PLAN_QUEUES 8   /* work-list queues, one per XCD */
#define JFA_PLAN_HEADER_BYTES 2048

/* Kernel ids for jfa_tile_config / jfa_build_plan. */
#define JFA_KERNEL_FWD 0       /* forward: tiles of query rows            */
#define JFA_KERNEL_BWD_DKDV 1  /* backward dK/dV pass: tiles of keys       */
#define JFA_KERNEL_BWD_DQ 2    /* backward dQ pass: tiles of query rows    */
#define JFA_KERNEL_BWD_SQ 3    /* backward of short-query sequences (Lq <= 64 < 1024 < Lk): chunks of keys */
#define JFA_KERNEL_FWD_SQ 4    /* forward of short-query sequences (Lq <= 64 < 1024 < Lk): chunks of keys  */

/* Element types for jfa_tile_config / jfa_build_plan. */
#define JFA_DTYPE_BF16 0
#define JFA_DTYPE_F32 1

/* Bytes of workspace jfa_fwd / jfa_fwd_f32 need. total_q, total_kv are the
 * row counts of q and k. Returns 0 for invalid sizes. */
size_t jfa_fwd_workspace_bytes(int B, int H, int64_t total_q, int64_t total_kv, int D, int causal);

/* Bytes of workspace jfa_bwd / jfa_bwd_f32 need. */
size_t jfa_bwd_workspace_bytes(int B, int H, int64_t total_q, int64_t total_kv, int D, int causal);

/* Forward pass (bf16 q/k/v/out). Writes out and lse for every valid row;
 * rows are never written outside their sequence. The softmax scale is
 * 1/sqrt(D). Jagged edges are handled by zero-filled loads and a subtraction
 * of the extra exponent terms ("Jagged Flash Attention (JFA)", section "Four
 * generations", item 1); a row whose valid terms the fp32 subtraction would
 * cancel (every valid score far below the pad keys' score) has its last
 * block's valid terms summed again instead. Work is scheduled longest-first over persistent
 * workgroups (same section, item 3). A sequence with at most 64 queries and
 * more than 1024 keys is split over its keys instead, one workgroup per
 * chunk of 1024 keys; each chunk's rows, normalised over its keys, and their
 * log-sum-exp are combined per (b, h) in a fixed order, so the result is
 * deterministic (asymmetric query/key lengths, section "Definition"). */
jfa_status jfa_fwd(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                   const int32_t* kv_offsets, int B, int H, int D, int64_t total_q, int64_t total_kv,
                   int max_kv_len, const float* bias, int causal, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Backward pass (bf16). Takes the forward's out and lse and the upstream
 * gradient dout; writes dq, dk, dv (same layout and type as q, k, v). dK/dV
 * and dQ are computed in two passes with no atomics ("Jagged Flash Attention
 * (JFA)", section "Four generations", item 2). A sequence with at most 64
 * queries and more than 1024 keys is instead owned whole by one workgroup
 * per chunk of 1024 keys, which forms S and dP once and reads K, V once; its
 * dQ is the sum, in a fixed order, of the chunks' partial results
 * (asymmetric query/key lengths, section "Definition").
 *
 * dbias: NULL, or an fp32 [H][JFA_BIAS_LEN] array (caller-owned, device
 * memory) that receives the gradient of sum(dout * out) with respect to the
 * bias table: dbias[h][r] is the sum, over every sequence and visible
 * (query i, key j) pair of head h with clip(i - j) + JFA_BIAS_RADIUS = r, of
 * the gradient with respect to that pair's score, dS = P * (dP - Delta)
 * (the bias is one of the custom attention biases of "Definition"). Needs
 * `bias` (JFA_ERR_INVALID_ARGUMENT otherwise). Computed in a fixed order,
 * so it is bit-identical run to run. */
jfa_status jfa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                   const void* dout, const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H,
                   int D, int64_t total_q, int64_t total_kv, int max_kv_len, const float* bias, int causal,
                   void* dq, void* dk, void* dv, float* dbias, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same parameters and results as jfa_fwd
 * (bit-identical outputs: the same kernels) without workspace and
 * workspace_bytes: the scratch is a fixed JFA_NOALLOC_SCRATCH_BYTES device
 * array inside the library, one per GPU, held until the process ends. The
 * call allocates nothing (no hipMalloc, no allocating library routine).
 * A call whose work list needs more scratch than that returns
 * JFA_ERR_WORKSPACE with the size it needs: the list takes 16 bytes per item
 * (at most H * (ceil(total_q / 128) + B) items), and, unless max_kv_len is in
 * 1 .. 1024, the short-query chunk rows add about
 * H * (ceil(total_kv / 1024) + B) * (256 * D + 272) bytes. Every call on one
 * GPU uses that GPU's one array: calls that overlap on one GPU (several
 * streams, several host threads) race and must be serialised by the
 * caller. */
#define JFA_NOALLOC_SCRATCH_BYTES (32u << 20)
jfa_status jfa_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                           const int32_t* kv_offsets, int B, int H, int D, int64_t total_q, int64_t total_kv,
                           int max_kv_len, const float* bias, int causal, void* out, float* lse, void* stream);

/* fp32 twins: identical parameters, every tensor of element type fp32;
 * D must be 32 or 64 (JFA_ERR_UNSUPPORTED for 128). */
jfa_status jfa_fwd_f32(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                       const int32_t* kv_offsets, int B, int H, int D, int64_t total_q, int64_t total_kv,
                       int max_kv_len, const float* bias, int causal, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);
jfa_status jfa_bwd_f32(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H,
                       int D, int64_t total_q, int64_t total_kv, int max_kv_len, const float* bias, int causal,
                       void* dq, void* dk, void* dv, float* dbias, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Padded-dense baseline (bf16), the comparison the method is measured
 * against: padding every sequence to a common length wastes compute
 * ("Jagged Flash Attention (JFA)", sections "Definition" and "Why standard
 * FlashAttention falls short"), and the speedup and memory reduction over
 * dense attention are the paper's headline figures ("Enhancing Performance
 * and Scalability of Large-Scale Recommendation Systems with Jagged Flash
 * Attention", section "Abstract"). Every sequence b occupies a fixed-length
 * slot:
 *   q, out, dout, dq  [B, q_slot,  H, D] bf16     lse [B, q_slot, H] fp32
 *   k, v, dk, dv      [B, kv_slot, H, D] bf16
 *   kv_lens           [B] int32 (device): the true key count of each slot,
 *                     in [0, kv_slot] (values outside are clamped)
 * The forward visits every block of every slot (query rows and keys up to the
 * slot length) and masks keys j >= kv_lens[b] with -inf, element by element on
 * every block, as a conventional kernel over padded tensors does; the causal
 * mask and the bias are those of jfa_fwd. Rows of out and lse that lie past a
 * sequence's true query length are computed like any other row and are the
 * caller's to ignore. The backward visits every block as well; its dQ pass
 * masks keys j >= kv_lens[b] element by element on the blocks that hold them.
 * It needs the rows of q, k, v and dout past each sequence's true lengths to
 * be zero (as a jagged batch copied into zeroed slots has them) and the lse
 * of jfa_fwd_padded: then every product of the dK/dV pass that involves a
 * pad row is zero, and the rows of dq, dk, dv inside the true lengths are
 * exact (that pass applies no mask, so it is no slower than a conventional
 * masked one). The softmax scale is 1/sqrt(D); no bias gradient. B * q_slot and
 * B * kv_slot must be below 2^31. Workspace: jfa_padded_workspace_bytes, for
 * either pass. Same ownership, asynchrony and error rules as jfa_fwd. */
size_t jfa_padded_workspace_bytes(int B, int H, int q_slot, int kv_slot, int D);
jfa_status jfa_fwd_padded(const void* q, const void* k, const void* v, const int32_t* kv_lens, int B, int q_slot,
                          int kv_slot, int H, int D, const float* bias, int causal, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);
jfa_status jfa_bwd_padded(const void* q, const void* k, const void* v, const void* out, const float* lse,
                          const void* dout, const int32_t* kv_lens, int B, int q_slot, int kv_slot, int H, int D,
                          const float* bias, int causal, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* stream);

/* offsets[0] = 0, offsets[b+1] = offsets[b] + lengths[b] for b < B (device
 * int32 arrays, lengths [B], offsets [B+1]); the prefix-sum addressing of
 * jagged tensors ("Jagged Flash Attention (JFA)", section "Definition"). */
jfa_status jfa_offsets_from_lengths(const int32_t* lengths, int B, int32_t* offsets, void* stream);

/* Tile shape of a kernel: *tile_m query rows and *tile_n keys. Tiles are
 * the work items of the persistent, longest-first scheduling ("Jagged Flash
 * Attention (JFA)", sections "Why standard FlashAttention falls short", on
 * short sequences leaving compute units idle, and "Four generations", item 3,
 * persistent kernels). For
 * JFA_KERNEL_FWD and JFA_KERNEL_BWD_DQ an item is one tile of tile_m query
 * rows and its cost counts tile_n-key blocks; for JFA_KERNEL_BWD_DKDV an item
 * is one tile of tile_n keys and its cost counts tile_m-row query blocks; for
 * JFA_KERNEL_BWD_SQ and JFA_KERNEL_FWD_SQ an item is one chunk of tile_n keys
 * of a sequence with at most tile_m queries. */
jfa_status jfa_tile_config(int kernel, int D, int dtype, int* tile_m, int* tile_n);

/* Builds the longest-first work lists the given kernel runs on (the
 * scheduling of "Jagged Flash Attention (JFA)", sections "Why standard
 * FlashAttention falls short" and "Four generations", item 3), into
 * `workspace`: a JFA_PLAN_HEADER_BYTES header of int32 {count, status, nq,
 * pad, start[8], qcount[8], ...; queue q's ticket at int32 index 32 * (q + 1)}
 * followed by `count` items of four
 * int32 (b, h, tile, cost). The items of one (b, h) form a group whose cost
 * is the sum of its items' costs; groups are ranked by cost descending, then
 * b, then h, and group rank g goes to queue g mod 16 < 8 ? g mod 8 :
 * 15 - g mod 16 (one queue per XCD; a workgroup drains its own queue, then
 * the others). Inside a queue groups follow their rank; inside a group items
 * follow cost descending, then tile ascending. Queue q holds items
 * [start[q], start[q] + qcount[q]). The lists of JFA_KERNEL_FWD,
 * JFA_KERNEL_BWD_DKDV and JFA_KERNEL_BWD_DQ skip sequences with at most 64
 * queries and more than 1024 keys; the lists of JFA_KERNEL_BWD_SQ and
 * JFA_KERNEL_FWD_SQ (the same list) have only those, one item per chunk of
 * 1024 keys (cost = keys in the chunk, causal or not), and the last
 * align(B * H * 4, 256) bytes of the workspace then receive, per (b, h), the
 * list position of its chunk 0 (-1 for other sequences). Exposed so that the
 * lists can be checked against an independent builder. */
jfa_status jfa_build_plan(const int32_t* q_offsets, const int32_t* kv_offsets, int B, int H, int D, int dtype,
                          int causal, int kernel, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes jfa_build_plan needs for that kernel: the list header and
 * at most H * (ceil(total / tile) + B) items of the work list above (same
 * passages). Returns 0 for invalid sizes. */
size_t jfa_plan_workspace_bytes(int B, int H, int64_t total_q, int64_t total_kv, int D, int dtype, int kernel);

/* Launch timing, for benchmarks and profiling. While enabled, every kernel
 * launch of this library is bracketed by two HIP events recorded on its
 * stream (a few microseconds of host overhead per launch). */
#define JFA_TIMING_KINDS 9 /* 0 work lists (forward, jfa_build_plan, padded slot offsets), 1 forward (with the short-query \
                             chunk merge), 2 backward work lists with Delta (one launch), 3 dK/dV, \
                             4 dQ (with the short-query dQ sum), 5 offsets scan, 6 short-query backward chunks, \
                             7 short-query forward chunks, 8 bias-gradient sum */
jfa_status jfa_timing_enable(int enable);

/* Waits for every recorded launch, writes the summed kernel milliseconds and
 * the launch count per kind (arrays of n_kinds entries), and forgets them. */
jfa_status jfa_timing_collect(double* total_ms, int64_t* launches, int n_kinds);

const char* jfa_status_string(jfa_status status);
const char* jfa_last_error(void);

/* Version of the argument lists above; a binding compares it with the one it
 * was written for before calling anything else. */
#define JFA_ABI_VERSION 5
int jfa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H */
