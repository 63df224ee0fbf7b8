/*
 * fcp.h -- C ABI of the block-level variable-length attention library for MI355X
 * (gfx950). One worker's share of FCP-style context-parallel attention: fixed-size
 * Q blocks attend to local or pulled KV blocks, every block pair yields a partial
 * output with its log-sum-exp, and partials of the same query rows are combined by an
 * associative LSE merge. A backward pass produces dQ, dK and dV.
 *
 * Sources. "Unleashing Scalable Context Parallelism for Foundation Models
 * Pre-Training via FCP" (arXiv 2605.08524): Sec. 2.2 (attention over [H, L, D]
 * tensors, causal and non-causal masks only, forward and backward both implemented,
 * grouped-query attention so KV rather than Q moves between workers, per-slice
 * results of one sequence reduce to the final output); Sec. 4.1 (fixed-size blocks,
 * short sequences packed into blocks and computed through the kernel's
 * variable-length interface); Sec. 4.2 (a worker computes pulled KV blocks with its
 * local Q blocks one block, or c coalesced blocks, at a time). The attention formula
 * itself is legible only on the paper's review page (xllm-io paper review of
 * 2605.08524, section "核心公式与建模"): O = Softmax(QK^T / sqrt(D) (.) M) V; the mask
 * M is read as excluding masked keys from the softmax.
 *
 * Conventions shared by every call
 *  - Tensors are caller-owned device memory, token-major and contiguous:
 *      q, dout, o        bf16  [q_rows,  num_q_heads,  head_dim]
 *      k, v              bf16  [kv_rows, num_kv_heads, head_dim]
 *      lse               fp32  [q_rows,  num_q_heads]      natural logarithm
 *      o_part            fp32  [part_rows, num_q_heads, head_dim]
 *      lse_part          fp32  [part_rows, num_q_heads]    natural logarithm
 *      dq                fp32  [q_rows,  num_q_heads,  head_dim]
 *      dk, dv            fp32  [kv_rows, num_kv_heads, head_dim]
 *    bf16 is IEEE bfloat16 stored as 16-bit words.
 *  - Query head h reads KV head h / (num_q_heads / num_kv_heads) (contiguous groups).
 *  - `pairs` is HOST memory, read only during the call; it may be reused on return.
 *  - `ws` is caller-owned device scratch of at least fcp_workspace_bytes(...) bytes for
 *    the same op and arguments; it must stay untouched until the stream passes the
 *    call. The library allocates no device memory; it owns only pinned host staging
 *    buffers used to upload its work lists (at most 8, each reused once its copy has
 *    completed; with more than 8 uploads still in flight a call waits for the oldest)
 *    and two small static device arrays (the 4 MiB work-list array of
 *    fcp_block_attn_fwd_fused_noalloc and the timing hook's clock samples).
 *  - Calls enqueue work on `stream` and return without waiting for it. They may be
 *    issued concurrently from several threads on distinct streams. Calls that share a
 *    workspace or output buffers must be ordered by the caller.
 *  - Return value: FCP_OK or an FCP_ERR_* code. No exception crosses the ABI and the
 *    library prints nothing; fcp_last_error() gives a thread-local message. Device
 *    faults surface at the caller's next synchronisation.
 *  - n_pairs == 0 is a no-op that returns FCP_OK.
 */
#ifndef FCP_H_
#define FCP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FCP_ABI_VERSION 1

/* Status codes. */
#define FCP_OK 0
#define FCP_ERR_INVALID_ARG 1 /* null pointer, bad dims, pair out of range, overlap  */
#define FCP_ERR_UNSUPPORTED 2 /* head_dim not 64/128, heads not grouped evenly, ... */
#define FCP_ERR_WORKSPACE 3   /* ws missing or smaller than fcp_workspace_bytes()   */
#define FCP_ERR_HIP 4         /* a HIP runtime call failed (text in last_error)     */
#define FCP_ERR_INTERNAL 5    /* host-side failure inside the library (e.g. no memory) */

/* Ops, for fcp_workspace_bytes() and fcp_validate(). */
#define FCP_OP_FWD 0
#define FCP_OP_MERGE 1
#define FCP_OP_BWD 2
#define FCP_OP_FWD_FUSED 3

/* Pair flags. */
#define FCP_PAIR_CAUSAL 1

/*
 * One block pair: the Q rows [q_start, q_start + q_len) of one sequence attend to the
 * KV rows [kv_start, kv_start + kv_len) of the same sequence (FCP paper Sec. 2.2 and
 * Sec. 4.2: a worker computes local Q blocks against local or pulled KV blocks; Sec.
 * 4.1: a packed block holds several sequences, so one block pair may become several
 * descriptors, one per same-sequence segment pair).
 *   seq_id       informational; not used by the kernels.
 *   q_start      first row in q / dout / o / lse / dq.            q_len  >= 1
 *   kv_start     first row in k / v / dk / dv.                    kv_len >= 1
 *   mask_offset  in-sequence position of Q row 0 minus that of KV row 0. With the
 *                causal flag, key j (0-based within the pair) is visible to query i iff
 *                j - i <= mask_offset; a query that sees no key of the pair gets an
 *                empty partial (O = 0, LSE = -inf). Any int32 value is accepted.
 *                Ignored without the causal flag.
 *   out_row      first row of this pair's partial in o_part / lse_part (fwd only).
 *   flags        bit 0: causal. Other bits must be zero.
 */
typedef struct fcp_pair_t {
  int32_t seq_id;
  int32_t q_start;
  int32_t q_len;
  int32_t kv_start;
  int32_t kv_len;
  int32_t mask_offset;
  int32_t out_row;
  int32_t flags;
} fcp_pair_t;

/*
 * Problem shape. num_q_heads must be a multiple of num_kv_heads, and the group size
 * G = num_q_heads / num_kv_heads must be 1, 2, 4 or a multiple of 8. head_dim is 64
 * or 128. softmax_scale 0 means 1/sqrt(head_dim) (the scale of the attention formula);
 * otherwise it must be finite and positive. The row extents bound every pair.
 */
typedef struct fcp_dims_t {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float softmax_scale;
  int64_t q_rows;    /* rows of q, dout, o, lse, dq      */
  int64_t kv_rows;   /* rows of k, v, dk, dv             */
  int64_t part_rows; /* rows of o_part, lse_part (fwd, merge) */
} fcp_dims_t;

/* ABI version of the loaded library (FCP_ABI_VERSION at build time). */
int fcp_abi_version(void);

/* Static text for a status code. Never NULL. */
const char* fcp_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* fcp_last_error(void);

/*
 * Host-only check of dims and pairs for `op` (no HIP call). Returns the status the
 * corresponding entry point would return for these arguments before touching the GPU.
 * FWD: pairs in range; partial-output ranges [out_row, out_row + q_len) disjoint.
 * MERGE, BWD, FWD_FUSED: any two pairs' Q ranges are identical or disjoint.
 * MERGE reads no K/V, so it does not check KV ranges against kv_rows.
 */
int fcp_validate(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op);

/*
 * Device workspace that `op` needs for these dims and pairs, in bytes (host-only).
 * Returns 0 when the arguments are invalid (fcp_last_error() says why) or nothing is
 * needed (n_pairs == 0).
 */
size_t fcp_workspace_bytes(const fcp_dims_t* dims, const fcp_pair_t* pairs,
                           int32_t n_pairs, int op);

/*
 * Host-only summary of the work lists that `op` builds for these dims and pairs (the
 * varlen tile scheduler's output; no HIP call), for tests and tools. Writes n_out int64
 * values to `out` (entries past FCP_PLAN_INFO_COUNT are 0):
 *   FCP_PLAN_QITEMS                  forward / dQ work items (Q tiles; each runs on
 *                                    num_q_heads / min(G, 8) workgroups)
 *   FCP_PLAN_KVITEMS                 dK/dV work items (BWD), after head splitting
 *   FCP_PLAN_SPLIT_TILES             dK/dV key tiles split by query heads (BWD)
 *   FCP_PLAN_SLOTS                   partial dK/dV slots of the split tiles (BWD)
 *   FCP_PLAN_MULTIHEAD_PARTS         parts of split tiles holding more than one head
 *   FCP_PLAN_MULTIHEAD_OFFSET_PARTS  of those, parts whose first head is not the first
 *                                    of the group
 *   FCP_PLAN_WS_BYTES                fcp_workspace_bytes() for the same arguments
 *   FCP_PLAN_Q_WORKGROUPS            launched workgroups of the forward / dQ kernel
 *   FCP_PLAN_KV_WORKGROUPS           launched workgroups of the dK/dV kernel (BWD)
 *   FCP_PLAN_EMPTY_WORKGROUPS        of those, empty ones (placement padding)
 *   FCP_PLAN_Q_KVHEADS_PER_XCD       the most distinct KV heads that the forward / dQ
 *                                    workgroups placed on one XCD use
 *   FCP_PLAN_KV_KVHEADS_PER_XCD      the same for the dK/dV workgroups
 * Placement: workgroup b of a launch is taken to run on XCD b % 8 (round-robin dispatch
 * over the 8 XCDs); the scheduler orders workgroups so that each KV head's work stays on
 * its own XCDs (one XCD per head at 8 KV heads, 8 / num_kv_heads XCDs per head below
 * that), heaviest first and balanced by cost. It affects locality only, never results.
 * Returns the status fcp_validate would return, or FCP_ERR_INVALID_ARG for a bad `out`.
 */
#define FCP_PLAN_QITEMS 0
#define FCP_PLAN_KVITEMS 1
#define FCP_PLAN_SPLIT_TILES 2
#define FCP_PLAN_SLOTS 3
#define FCP_PLAN_MULTIHEAD_PARTS 4
#define FCP_PLAN_MULTIHEAD_OFFSET_PARTS 5
#define FCP_PLAN_WS_BYTES 6
#define FCP_PLAN_Q_WORKGROUPS 7
#define FCP_PLAN_KV_WORKGROUPS 8
#define FCP_PLAN_EMPTY_WORKGROUPS 9
#define FCP_PLAN_Q_KVHEADS_PER_XCD 10
#define FCP_PLAN_KV_KVHEADS_PER_XCD 11
#define FCP_PLAN_INFO_COUNT 12

int fcp_plan_info(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs, int op,
                  int64_t* out, int32_t n_out);

/*
 * Forward, one partial per pair (FCP paper Sec. 2.2: per-slice intermediate results).
 * For every pair and query head, writes the pair's own normalised attention output
 * over its visible keys to o_part rows [out_row, out_row + q_len) and its natural-log
 * LSE to lse_part; queries with no visible key get O = 0 and LSE = -inf. Other rows of
 * o_part / lse_part are left untouched. Arithmetic: bf16 products, fp32 accumulation
 * and softmax.
 */
int fcp_block_attn_fwd(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                       const fcp_pair_t* pairs, int32_t n_pairs, float* o_part,
                       float* lse_part, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Partial formats for the _ex variants. FCP_PART_F32: o_part is fp32, as above.
 * FCP_PART_BF16: o_part holds the same normalised partial outputs rounded to bf16 (round
 * to nearest even; [part_rows, num_q_heads, head_dim] 16-bit words), halving the bytes a
 * pair writes and the merge reads; lse_part stays fp32. fcp_block_attn_fwd and
 * fcp_merge_partials are the FCP_PART_F32 cases. An unknown format is
 * FCP_ERR_INVALID_ARG.
 */
#define FCP_PART_F32 0
#define FCP_PART_BF16 1

int fcp_block_attn_fwd_ex(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                          const fcp_pair_t* pairs, int32_t n_pairs, void* o_part,
                          float* lse_part, int32_t part_format, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * LSE merge of partials (FCP paper Sec. 2.2: per-slice results reduce to the final
 * output). Pairs with identical (q_start, q_len) form a group; for every row and head
 * of a group, LSE = ln sum_i exp(LSE_i) and O = sum_i exp(LSE_i - LSE) O_i over the
 * group's partials, written as bf16 `o` and fp32 `lse` at rows q_start... A row whose
 * partials are all empty gets O = 0, LSE = -inf. Rows no pair covers are untouched.
 * Partially overlapping Q ranges are an error.
 */
int fcp_merge_partials(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs,
                       const float* o_part, const float* lse_part, void* o, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* fcp_merge_partials over partials in `part_format` (FCP_PART_F32 or FCP_PART_BF16). */
int fcp_merge_partials_ex(const fcp_dims_t* dims, const fcp_pair_t* pairs, int32_t n_pairs,
                          const void* o_part, const float* lse_part, int32_t part_format,
                          void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Forward with the merge folded in: for every group of pairs with identical Q range,
 * one pass over all of the group's KV ranges writes the final bf16 O and fp32 LSE
 * directly (same result as fcp_block_attn_fwd followed by fcp_merge_partials, without
 * the fp32 partials; the execution side of the bottom-up coalescer, FCP paper Sec.
 * 4.2). out_row is ignored. Partially overlapping Q ranges are an error.
 */
int fcp_block_attn_fwd_fused(const fcp_dims_t* dims, const void* q, const void* k,
                             const void* v, const fcp_pair_t* pairs, int32_t n_pairs,
                             void* o, float* lse, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * For callers that cannot allocate memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): fcp_block_attn_fwd_fused without a workspace
 * argument. Same arguments, checks and results as fcp_block_attn_fwd_fused (bitwise:
 * same kernel, same work lists); the work lists go to a static device array of 4 MiB
 * that the library holds on each GPU it runs on until the process ends, instead of `ws`.
 * The call allocates no device or pinned memory (the host planner uses ordinary heap
 * memory) and uploads the lists from pageable host memory with one hipMemcpyAsync on
 * `stream`. Tables whose work lists exceed 4 MiB (about 130 000 tiles of 32 query rows,
 * i.e. some 4 million query rows at 8 heads per KV head) return FCP_ERR_WORKSPACE before
 * any HIP call. Every call on one GPU shares that GPU's array, which keeps the last
 * call's lists: calls on one stream are ordered, but calls that overlap on one GPU
 * (different streams or threads without ordering) race on the array and must not be
 * issued.
 */
int fcp_block_attn_fwd_fused_noalloc(const fcp_dims_t* dims, const void* q, const void* k,
                                     const void* v, const fcp_pair_t* pairs, int32_t n_pairs,
                                     void* o, float* lse, hipStream_t stream);

/*
 * Backward (FCP paper Sec. 2.2 states that a backward is implemented; the gradient
 * here is the exact one of the forward). Takes the MERGED o (bf16) and lse (fp32) of
 * the rows the pairs cover and the upstream gradient dout, and ADDS each pair's
 * contribution to fp32 dq, dk and dv (the caller zeroes them first). With
 * Delta_i = sum_d dout_i o_i, P_ij = exp(S_ij - lse_i) and dS_ij = P_ij (dP_ij - Delta_i):
 * dv_j += sum_i P_ij dout_i, dk_j += scale sum_i dS_ij q_i, dq_i += scale sum_j dS_ij k_j,
 * summed over the query heads of each KV head's group. Any two pairs' Q ranges must be
 * identical or disjoint. Results are deterministic (no atomics).
 */
int fcp_block_attn_bwd(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* dout,
                       const fcp_pair_t* pairs, int32_t n_pairs, float* dq, float* dk,
                       float* dv, void* ws, size_t ws_bytes, hipStream_t stream);

/* fcp_block_attn_bwd_ex flag: write the gradients instead of adding to them. */
#define FCP_BWD_OVERWRITE 1

/*
 * fcp_block_attn_bwd with `flags`: 0 behaves exactly as fcp_block_attn_bwd; with
 * FCP_BWD_OVERWRITE the rows of dq that some pair's Q range covers, and the rows of dk
 * and dv that some pair's KV range covers, are WRITTEN with the gradient (every such row
 * has exactly one writer, so the result equals zeroing them and adding), and every other
 * row is left as it was. A caller that does not accumulate gradients across calls skips
 * the zero-fill and the kernels' read of the old values. Other flag bits:
 * FCP_ERR_INVALID_ARG.
 */
int fcp_block_attn_bwd_ex(const fcp_dims_t* dims, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout,
                          const fcp_pair_t* pairs, int32_t n_pairs, float* dq, float* dk,
                          float* dv, int32_t flags, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Block-level pipelined forward (FCP paper Sec. 4.2, "Block-level pipelining", Figure 7:
 * a worker's pull, compute and push are split into block-grained sub-stages that
 * interleave, each stage's transfer overlapping the previous stage's computation; the
 * bottom-up coalescer of the same section lets a stage carry c blocks).
 *
 * A stage brings KV rows into k / v (the worker's KV buffer, kv_rows rows) by copying
 * them from k_src / v_src (src_rows rows, same row layout; on one GPU they stand in for
 * the memory of the workers the blocks are pulled from) and then computes its block
 * pairs' partials. `stages[s]` takes the next n_copies entries of `copies` and the next
 * n_pairs entries of `pairs`, in table order. With depth R >= 1 (the number of KV
 * regions the caller rotates through):
 *  - stage s's copies run on copy_stream after the work enqueued on `stream` before this
 *    call, and after stage s-R's pairs have been computed;
 *  - stage s's pairs are computed on `stream` (as by fcp_block_attn_fwd: fp32 partials at
 *    out_row) once stage s's copies are done;
 *  - after the last stage every pair's partial is merged into o / lse on `stream` (as by
 *    fcp_merge_partials); `stream` has then also passed every copy.
 * So the copies of stages s+1 .. s+R-1 may overlap the computation of stage s (R = 2:
 * double buffering). The KV rows that stage s's copies write must not be read by the
 * pairs of stages s-R+1 .. s-1 (FCP_ERR_INVALID_ARG otherwise).
 * copy_stream == stream runs everything in order with no overlap. Copies use a DMA
 * engine (no compute units) unless flags has FCP_PIPE_COPY_SHADER (copy kernel). With
 * FCP_PIPE_PART_BF16 the partials in o_part are bf16 (FCP_PART_BF16 layout; o_part then
 * points at part_rows * num_q_heads * head_dim 16-bit words).
 * k_src / v_src must not overlap k / v. Tables are host memory read during the call;
 * o_part / lse_part have dims->part_rows rows; all pairs together must satisfy the
 * checks of both FCP_OP_FWD and FCP_OP_MERGE. `ws` holds at least
 * fcp_pipeline_workspace_bytes(...) bytes. A stage may have no copies or no pairs.
 */
typedef struct fcp_copy_t {
  int64_t src_row; /* first row in k_src / v_src */
  int64_t dst_row; /* first row in k / v */
  int64_t n_rows;  /* >= 1 */
} fcp_copy_t;

typedef struct fcp_stage_t {
  int32_t n_copies;
  int32_t n_pairs;
} fcp_stage_t;

#define FCP_PIPE_COPY_SHADER 1
#define FCP_PIPE_PART_BF16 2

int fcp_pipeline_fwd(const fcp_dims_t* dims, const void* q, void* k, void* v,
                     const void* k_src, const void* v_src, int64_t src_rows,
                     const fcp_stage_t* stages, int32_t n_stages, const fcp_copy_t* copies,
                     const fcp_pair_t* pairs, int32_t depth, float* o_part, float* lse_part,
                     void* o, float* lse, int32_t flags, void* ws, size_t ws_bytes,
                     hipStream_t stream, hipStream_t copy_stream);

/* Workspace of fcp_pipeline_fwd for these tables (host-only; 0 when invalid, with
 * fcp_last_error() set, or when there are no pairs). */
size_t fcp_pipeline_workspace_bytes(const fcp_dims_t* dims, const fcp_stage_t* stages,
                                    int32_t n_stages, const fcp_copy_t* copies,
                                    const fcp_pair_t* pairs, int32_t depth, int64_t src_rows);

/*
 * Optional per-kernel timing, for measurement tools (not needed for computing).
 * Kernel ids: FCP_KERNEL_FWD (per-pair forward), FCP_KERNEL_FWD_FUSED, FCP_KERNEL_MERGE,
 * FCP_KERNEL_DELTA (reserved: the backward's Delta now runs inside the dQ kernel, so this
 * id records no launches), FCP_KERNEL_DQ, FCP_KERNEL_DKDV,
 * FCP_KERNEL_DKDV_REDUCE (sums the parts of dK/dV tiles the scheduler split by head),
 * FCP_KERNEL_PIPE_COPY (all copies of one pipeline stage, timed on copy_stream).
 * fcp_timing_enable(1): from now on every kernel launch, from any thread, is bracketed by
 * a pair of HIP events recorded on the call's stream. fcp_timing_enable(0) stops that.
 * fcp_timing_read(): waits for every recorded pair, adds each pair's elapsed time to
 * total_ms[id] and 1 to launches[id] for id < n (arrays of n >= FCP_KERNEL_COUNT entries,
 * zeroed by the call first), then forgets the pairs. Returns FCP_OK or FCP_ERR_HIP.
 * fcp_kernel_name(id) gives the kernel's name ("" for an unknown id).
 */
#define FCP_KERNEL_FWD 0
#define FCP_KERNEL_FWD_FUSED 1
#define FCP_KERNEL_MERGE 2
#define FCP_KERNEL_DELTA 3
#define FCP_KERNEL_DQ 4
#define FCP_KERNEL_DKDV 5
#define FCP_KERNEL_DKDV_REDUCE 6
#define FCP_KERNEL_PIPE_COPY 7
#define FCP_KERNEL_COUNT 8

int fcp_timing_enable(int on);
int fcp_timing_read(double* total_ms, int32_t* launches, int32_t n);

/*
 * fcp_timing_read, and in sclk_mhz[id] (n entries, or NULL) the average shader clock of
 * the timed launches of kernel id on the calling thread's current device, in MHz (0 when
 * none ran or the kernel takes no samples: the merge, the reduce and the copies). While
 * timing is on, the forward, dQ and dK/dV kernels sample the shader-clock counter and a
 * 100 MHz reference counter when each workgroup starts and ends; the value is the ratio
 * of the summed differences times 100 MHz (a workgroup-lifetime-weighted average). The
 * samples are reset by every read.
 */
int fcp_timing_read_clock(double* total_ms, int32_t* launches, double* sclk_mhz, int32_t n);
const char* fcp_kernel_name(int id);

/*
 * Congestion-free communication plan (FCP paper Sec. 4.2, "Congestion-free solver",
 * Lemmas 1 and 2). Host only: no GPU, no stream, callable anywhere. The n_edges block
 * transfers among n_workers workers form a bipartite multigraph (edge e: worker src[e]
 * sends one block to worker dst[e]; src[e] == dst[e] is allowed and counts once on each
 * side). Writes stage[e] for every edge so that within one stage no worker sends more
 * than one block and none receives more than one (each stage is a matching), using the
 * minimum possible number of stages, the maximal send-or-receive degree Delta, returned
 * in *n_stages. Stages are numbered 0..Delta-1 and each is non-empty. Host arrays of
 * n_edges int32 each, owned by the caller; n_edges == 0 gives *n_stages = 0. A worker id
 * outside [0, n_workers) or a NULL array is FCP_ERR_INVALID_ARG. Coalescing c sub-stages
 * into one (the pages' knob for launch overhead) is stage[e] / c.
 */
int fcp_comm_plan(int32_t n_workers, int32_t n_edges, const int32_t* src, const int32_t* dst,
                  int32_t* stage, int32_t* n_stages);

#ifdef __cplusplus
}
#endif

#endif /* FCP_H_ */
