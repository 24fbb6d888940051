/*
 * lsh.h - exact long-sequence multi-head attention (forward and backward)
 * for AMD MI355X (gfx950). C ABI of liblsh.so.
 *
 * What the library computes. For every batch entry b and head h, with
 * scores s_ij = scale * <q_i, k_j>, the forward pass of softmax attention
 *     LSE_i = log( sum_j exp(s_ij) )                (natural log)
 *     O_i   = sum_j exp(s_ij - LSE_i) * v_j
 * (definition: "LLM Lab Notes 05: Attention Tensor Parallelism - Splitting
 * QKV by Head, Megatron Style", sections 2 and 3: per-head scaled dot
 * products, softmax over the keys, weighted sum of the values; heads never
 * interact). O is returned in float32, LSE in float32. The computation is
 * exact up to floating-point rounding: a blockwise online softmax over key
 * tiles of 64, with QK^T and PV on the matrix cores and fp32 accumulation.
 * lsh_attn_bwd gives the gradients of the dense forward (see there).
 *
 * Conventions shared by every entry point.
 *  - Pointers named q, k, v, o, lse, src, dst, o_parts, lse_parts,
 *    block_mask, dout, dq, dk, dv and workspace are DEVICE pointers owned
 *    by the caller. No call allocates device memory and none keeps
 *    per-call state; the one static device array of the library (see
 *    lsh_attn_fwd_blocksparse_noalloc) is part of its loaded code.
 *  - Streams are hipStream_t values passed as void*; NULL is the null
 *    stream. Every function only enqueues work and returns; results are
 *    ready when the stream(s) reach that point.
 *  - Tensors use element strides; the innermost (head_dim) stride is 1.
 *    Q is [B, Sq, H, D] and K, V are [B, Skv, H, D] as seen through
 *    (b, s, h) strides; O is float32 [B, Sq, H, D] through its own strides;
 *    LSE is float32 [B, H, Sq], contiguous.
 *  - Base pointers must be 16-byte aligned and every stride times the
 *    element size must be a multiple of 16 bytes. D must be 128.
 *  - Outputs must not overlap inputs or each other.
 *  - Errors: every argument is validated before the first HIP call, so a
 *    call that returns an error has enqueued nothing. A failed kernel
 *    launch returns LSH_ERR_HIP. lsh_last_error() gives a message for the
 *    last failing call on the calling thread.
 *  - Determinism: the result for one (b, h) depends only on that head's
 *    q, k, v, the dtype, D, Sq, Skv and scale - never on H, on the head
 *    chunking, on strides, on streams or on the run. Repeated runs are
 *    bit-identical; no floating-point atomics are used.
 *  - Thread safety: all entry points may be called concurrently.
 */
#ifndef LSH_H
#define LSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSH_ABI_VERSION 1
#define LSH_HEAD_DIM 128     /* the only supported head_dim */
#define LSH_MASK_BLOCK 128   /* block edge of the block-sparse mask, tokens */

typedef enum lsh_status {
  LSH_OK = 0,
  LSH_ERR_INVALID = 1,      /* bad argument (null pointer, bad size, stride, alignment) */
  LSH_ERR_UNSUPPORTED = 2,  /* valid but not implemented (D != 128, huge offsets) */
  LSH_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  LSH_ERR_NO_DEVICE = 4,    /* no gfx950 device is current */
  LSH_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} lsh_status;

typedef enum lsh_dtype {
  LSH_F32 = 0,   /* float32 Q, K, V */
  LSH_BF16 = 1   /* bfloat16 Q, K, V (fp32 accumulation and output) */
} lsh_dtype;

typedef void* lsh_stream;   /* a hipStream_t */

/*
 * Arguments of one attention forward.
 * Validation (before any HIP call): pointers 16-byte aligned, strides
 * non-negative and multiples of 16 bytes, D = 128, B, Sq, Skv, H below
 * 2^30, B*Sq*H below 2^31; for bf16, one head's K (and V) rows must span
 * less than 2 GiB ((Skv - 1) * key stride * 2 + 256 bytes). Violations
 * return LSH_ERR_INVALID or LSH_ERR_UNSUPPORTED.
 */
typedef struct lsh_attn_args {
  const void* q;          /* [B, Sq, H, D] elements of `dtype` */
  const void* k;          /* [B, Skv, H, D] */
  const void* v;          /* [B, Skv, H, D] */
  float* o;               /* float32 [B, Sq, H, D] */
  float* lse;             /* float32 [B, H, Sq], contiguous */
  int32_t dtype;          /* lsh_dtype */
  int32_t reserved;       /* must be 0 */
  int64_t B, Sq, Skv, H, D;
  int64_t q_stride[3];    /* element strides of (b, s, h) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  float scale;            /* score multiplier; 1/sqrt(D) for standard attention */
} lsh_attn_args;

/* Version of this header the library was built from (LSH_ABI_VERSION). */
int lsh_abi_version(void);

/* Static text for a status code. */
const char* lsh_status_str(int status);

/* Message for the last failing call on this thread ("" if none). */
const char* lsh_last_error(void);

/* LSH_OK when a gfx950 device is current on the calling thread, else
 * LSH_ERR_NO_DEVICE. */
lsh_status lsh_device_check(void);

/*
 * Dense attention forward over all keys, launched on one stream.
 * Reads Q, K, V through their strides, writes O and LSE. Skv >= 1.
 * Source: the TP page above, sections 2-3 (per-head local attention).
 */
lsh_status lsh_attn_fwd(const lsh_attn_args* args, lsh_stream stream);

/*
 * Head-chunked multi-stream forward.
 * Source: "HCMS: Head-Chunked Multi-Stream Pipeline for Communication-
 * Computation Overlap in Long-Sequence Parallel Attention", Abstract: the
 * heads are split into chunks, possibly of unequal size; the re-layout of
 * one chunk (an all-to-all across GPUs there, a local head-major copy here)
 * runs on a second stream while the attention of the previous chunk runs,
 * and the result is the same as the unchunked computation.
 *
 * head_chunks[0..n_chunks-1] >= 1 and sum to H; chunk c covers heads
 * [sum_{c'<c}, sum_{c'<=c}) in ascending order. For each chunk, Q, K and V
 * of its heads are copied by lsh_head_permute into the workspace as
 * [B, hc, S, D] (on `permute_stream`), then attention runs on that copy
 * (on `compute_stream`) and writes the chunk's heads of O and LSE.
 * Ordering: the permute stream first waits for all work previously
 * enqueued on the compute stream; chunk c's attention waits for chunk c's
 * copy; all the call's work is ordered before later work on the compute
 * stream. The two streams may be the same stream. Requires Sq == Skv.
 * O and LSE are bit-identical to lsh_attn_fwd on the same inputs.
 * workspace: device memory of at least lsh_attn_fwd_chunked_workspace(args)
 * bytes; it must not be reused before the compute stream has passed this
 * call's work.
 */
lsh_status lsh_attn_fwd_chunked(const lsh_attn_args* args,
                                const int32_t* head_chunks, int32_t n_chunks,
                                void* workspace, size_t workspace_bytes,
                                lsh_stream compute_stream,
                                lsh_stream permute_stream);

/* Workspace bytes of lsh_attn_fwd_chunked: the head-major copies of Q, K
 * and V (3 * B * H * S * D elements), 256-byte aligned. 0 on bad args. */
size_t lsh_attn_fwd_chunked_workspace(const lsh_attn_args* args);

/*
 * Attention of the queries against ONE block of keys (one Ring Attention
 * round). Source: "CHARM+: How Cross-Hardware Attention Breaks Through
 * Distributed Communication Bottlenecks", section on where the bottleneck
 * comes from: in Ring Attention each device keeps its queries, receives the
 * KV blocks in turn and combines per-block partial results.
 * O is normalised over the block's keys and LSE is the block's log-sum-exp,
 * so lsh_lse_merge over all blocks yields attention over all keys.
 * Skv may be 0 (an empty block): O = 0 and LSE = -inf; k and v may then be
 * NULL.
 */
lsh_status lsh_attn_partial(const lsh_attn_args* args, lsh_stream stream);

/*
 * One Ring Attention round folded into a running result (same page and
 * section as lsh_attn_partial; the per-block results are combined as they
 * arrive rather than all at the end). On entry o and lse hold attention
 * over the key blocks folded in so far: O normalised over their keys, LSE
 * their log-sum-exp; before the first block, O = 0 and LSE = -inf. On
 * return they hold attention over those blocks and this one, merged row by
 * row as lsh_lse_merge merges two parts (a row whose two LSE are both -inf
 * is left as it is). Folding a block into O = 0, LSE = -inf gives exactly
 * lsh_attn_partial's result for it. Arguments as for lsh_attn_partial;
 * Skv = 0 returns LSH_OK and leaves o and lse untouched. o and lse are read
 * and written in place: nothing else may use them until the call's work on
 * the stream has finished, and the call must not overlap another that
 * writes them.
 */
lsh_status lsh_attn_partial_accumulate(const lsh_attn_args* args, lsh_stream stream);

/*
 * Merge n partial results over disjoint key sets (same page as above; the
 * "Re-Merge" of "CHARM+: Cross-Hardware Attention with Re-Merge Multistream
 * Mechanism", read as this merge):
 *   M = max_k LSE_k, w_k = exp(LSE_k - M), Z = sum_k w_k,
 *   LSE = M + log Z,  O = sum_k (w_k / Z) * O_k.
 * Rows whose n LSE values are all -inf get O = 0 and LSE = -inf.
 * o_parts: float32 [n, B, Sq, H, D] contiguous; lse_parts: float32
 * [n, B, H, Sq] contiguous; o: float32 [B, Sq, H, D] contiguous; lse:
 * float32 [B, H, Sq] contiguous. 1 <= n <= 4096. D must be 128.
 */
lsh_status lsh_lse_merge(const float* o_parts, const float* lse_parts,
                         int32_t n, int64_t B, int64_t Sq, int64_t H,
                         int64_t D, float* o, float* lse, lsh_stream stream);

/*
 * Head-major copy of heads [h0, h0 + hc): src [B, S, H, D] (contiguous) ->
 * dst [B, hc, S, D] (contiguous), dst[b, h - h0, s, :] = src[b, s, h, :].
 * A bit copy. It stands in, on one GPU, for the all-to-all that turns a
 * sequence-sharded layout into a head-sharded one (HCMS page, Abstract;
 * "db-SP: Accelerating Sparse Attention for Visual Generative Models with
 * Dual-Balanced Sequence Parallelism", Abstract: Ulysses parallelises
 * along the head dimension). D * element size must be a multiple of 16.
 */
lsh_status lsh_head_permute(const void* src, void* dst, int32_t dtype,
                            int64_t B, int64_t S, int64_t H, int64_t D,
                            int32_t h0, int32_t hc, lsh_stream stream);

/*
 * Block-sparse attention forward. Source: the db-SP page, Abstract:
 * block-wise sparse attention computes only the dense blocks of a sparse
 * mask; sparsity differs between heads and dense blocks sit irregularly.
 * block_mask: device uint8 [B, H, ceil(Sq/128), ceil(Skv/128)]; query i
 * attends key j iff block_mask[b, h, i/128, j/128] != 0. Masked pairs are
 * excluded from the softmax. A query row with no kept block gets O = 0 and
 * LSE = -inf. Requires a bf16 or f32 args as lsh_attn_fwd, Skv >= 1.
 * workspace: at least lsh_attn_fwd_blocksparse_workspace(args) bytes; it
 * holds the launch schedule, readable after the call for diagnostics. With
 * n = B * H * ceil(Sq/128) items (item = (b * H + h) * ceil(Sq/128) + query
 * block), G = B * H heads, nk = ceil(Skv/128), R = n * 4, T = G * 8 and
 * K = n * nk * 2, each rounded up to 256 bytes:
 *   int32 counts[n]      at byte 0:             kept blocks of each item's mask row;
 *   int32 order[n]       at byte R:             item of each launch slot;
 *   int64 totals[G]      at byte 2 * R:         kept blocks of each head;
 *   uint16 kept[n][nk]   at byte 2 * R + T:     each item's kept key blocks,
 *                                               ascending (counts[item] of them);
 *   int32 place[G + 8]   at byte 2 * R + T + K: XCD placement of the heads.
 * Launch slot s runs on XCD s mod 8. Heads are dealt to the 8 XCDs whole:
 * in descending total (ties: lower index first), each to the XCD with the
 * smallest total so far among those holding fewer than ceil(G / 8) heads
 * (ties: lowest XCD); place[g] = x + 8 * k for the k-th head dealt to XCD x,
 * place[G + x] = heads of XCD x. XCD x's list is its heads in the order
 * dealt, each head's items in descending count (ties: lower index first);
 * position j of that list (lists of L_x = place[G + x] * ceil(Sq/128)
 * items) takes slot sum_x' min(L_x', j) + #{x' < x : L_x' > j}. So each
 * head's K/V streams through one XCD's L2, one head at a time per XCD, and
 * the heaviest rows of a head start first. Same reuse rule as the chunked
 * workspace.
 */
lsh_status lsh_attn_fwd_blocksparse(const lsh_attn_args* args,
                                    const uint8_t* block_mask,
                                    void* workspace, size_t workspace_bytes,
                                    lsh_stream stream);

/* Workspace bytes of lsh_attn_fwd_blocksparse. 0 on bad args. */
size_t lsh_attn_fwd_blocksparse_workspace(const lsh_attn_args* args);

/*
 * lsh_attn_fwd_blocksparse without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid allocation). Same arguments, kernels and
 * results (bit-identical) as lsh_attn_fwd_blocksparse; the launch schedule
 * goes to a static device array of LSH_NOALLOC_SCRATCH_BYTES instead of a
 * workspace. The call allocates nothing. Each GPU holds its own array from
 * the library's load until the process ends; the schedule kernels overwrite
 * every byte they use, so nothing needs clearing between calls, and the
 * schedule of the last call stays readable there only by the library.
 * Calls that overlap on one GPU (two streams, or two threads) share the
 * array and race: order them on one stream. Returns LSH_ERR_WORKSPACE,
 * before any HIP call, when lsh_attn_fwd_blocksparse_workspace(args)
 * exceeds LSH_NOALLOC_SCRATCH_BYTES.
 */
#define LSH_NOALLOC_SCRATCH_BYTES (16u << 20)
lsh_status lsh_attn_fwd_blocksparse_noalloc(const lsh_attn_args* args,
                                            const uint8_t* block_mask,
                                            lsh_stream stream);

/*
 * Arguments of one attention backward (bf16 only).
 * The forward is lsh_attn_fwd on the same q, k, v and scale; o and lse
 * are its outputs. Validation (before any HIP call) as for
 * lsh_attn_args; in addition dtype must be LSH_BF16 (LSH_F32 returns
 * LSH_ERR_UNSUPPORTED), and one head's Q (and dO) rows must span less
 * than 2 GiB, like K and V.
 */
typedef struct lsh_attn_bwd_args {
  const void* q;          /* bf16 [B, Sq, H, D] */
  const void* k;          /* bf16 [B, Skv, H, D] */
  const void* v;          /* bf16 [B, Skv, H, D] */
  const void* dout;       /* bf16 [B, Sq, H, D]: gradient of the loss w.r.t. O */
  const float* o;         /* float32 [B, Sq, H, D]: the forward's O */
  const float* lse;       /* float32 [B, H, Sq], contiguous: the forward's LSE */
  float* dq;              /* float32 [B, Sq, H, D] */
  float* dk;              /* float32 [B, Skv, H, D] */
  float* dv;              /* float32 [B, Skv, H, D] */
  int32_t dtype;          /* lsh_dtype; only LSH_BF16 */
  int32_t reserved;       /* must be 0 */
  int64_t B, Sq, Skv, H, D;
  int64_t q_stride[3];    /* element strides of (b, s, h) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t do_stride[3];
  int64_t o_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  float scale;            /* the forward's score multiplier */
} lsh_attn_bwd_args;

/*
 * Attention backward: gradients of the dense forward (lsh_attn_fwd) with
 * respect to q, k and v for a loss whose gradient with respect to O is
 * dout. With P = exp(scale q k^T - LSE) per (b, h):
 *   dV = P^T dO,   dP = dO V^T,   Delta = rowsum(dO * O),
 *   dS = P * (dP - Delta),   dQ = scale dS K,   dK = scale dS^T Q.
 * Source: the forward's definition (the TP page above, sections 2-3)
 * differentiated; CHARM+ ("CHARM+: How Cross-Hardware Attention Breaks
 * Through Distributed Communication Bottlenecks", section "Measured
 * Speedups") reports the backward pass beside the forward.
 * dQ, dK, dV are written in float32 (every element, no accumulation into
 * prior contents). Skv >= 1. Deterministic: no atomics; dK/dV and dQ come
 * from separate kernels that each rebuild P.
 * workspace: device memory of at least lsh_attn_bwd_workspace(args)
 * bytes, 256-byte aligned (per-row LSE * log2(e) and Delta); same reuse
 * rule as the chunked workspace.
 */
lsh_status lsh_attn_bwd(const lsh_attn_bwd_args* args, void* workspace,
                        size_t workspace_bytes, lsh_stream stream);

/* Workspace bytes of lsh_attn_bwd: B * H * ceil(Sq / 64) * 512. 0 on bad
 * args. */
size_t lsh_attn_bwd_workspace(const lsh_attn_bwd_args* args);

#ifdef __cplusplus
}
#endif

#endif /* LSH_H */
