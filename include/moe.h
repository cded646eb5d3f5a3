/*
 * moe.h -- one MoE layer's token dispatch, expert FFN and combine on a single
 * AMD Instinct MI355X (gfx950), behind a plain C ABI.
 *
 * What the layer computes (MindSpeed Chunk MoE article, sections "核心原理"
 * (core principle) and the timing-diagram section): routing metadata, then a
 * permute of hidden_states into an expert-contiguous buffer, then the expert
 * computation, then an unpermute that returns every token's output to its
 * original position as the top_k_weights-weighted sum over its k experts.  The
 * Chunk MoE variant cuts the tokens into N chunks of T_chunk = ceil(T/N)
 * (same article, "一组关键公式", key formulas) and runs adjacent chunks as a
 * pair so one chunk's data movement overlaps its neighbour's expert compute.
 *
 *   out[t] = sum_{j<k} top_k_weights[t][j] * FFN_{top_k_index[t][j]}(hidden_states[t])
 *   FFN_e(x) = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)),  silu(z) = z / (1 + e^-z)
 *
 * The expert FFN form (SwiGLU, no bias) is not spelled out on the pages; it is
 * the reading this library takes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named as tensors are DEVICE memory owned by the caller.  The
 *    library allocates no device memory and keeps no pointer after it returns.
 *    Its only state is a per-thread cache of three HIP events per device, used
 *    by moe_chunked_forward(_schedule) to order its two streams.
 *  - Calls only enqueue work on the given stream(s) and return.  No call waits
 *    on the device or copies anything back to the host.
 *  - Row-major, dense layouts:
 *      hidden_states, out       [T][H]
 *      top_k_index              [T][k]  int32
 *      top_k_weights            [T][k]  float32 (kept in fp32 for every dtype)
 *      w_gate_up                [E][2I][H]  rows 0..I-1 gate, rows I..2I-1 up
 *      w_down                   [E][H][I]
 *    Flat assignment index f = t*k + j.
 *  - dtype MOE_BF16: hidden_states, weights, out and the intermediates are
 *    bf16, products accumulate in fp32, and act, y and out are each rounded to
 *    bf16 (nearest even) exactly once; silu uses the hardware exponential and
 *    reciprocal (relative error about 1e-7 * (1 + |z|), far below the bf16
 *    rounding).  dtype MOE_F32: fp32 everywhere.  Forward results do not depend
 *    on N, on the schedule or on the entry point used: every path gives the
 *    same bits (the backward's fp32 weight gradients add the chunk pairs'
 *    contributions in turn, so those depend on N within rounding).
 *  - Errors: the status comes from host-side checks of the arguments and of the
 *    kernel launches; nothing throws across the ABI.  Expert ids outside [0, E)
 *    are a device-side condition: such slots are dropped (no row, zero
 *    contribution) and counted into *dev_error.
 *  - Alignment: tensors of hidden/weight/intermediate/out type and the
 *    workspace need 16-byte alignment (the workspace 256); int32/float32 arrays
 *    need 4 bytes.
 *  - Limits: T >= 0, 1 <= k <= 64, 1 <= E <= 1024, E % G == 0, T*k < 2^31.
 *    MOE_BF16 needs H % 64 == 0 and I % 64 == 0; MOE_F32 needs H % 4 == 0 and
 *    I % 4 == 0.  Anything else returns MOE_ERR_UNSUPPORTED or
 *    MOE_ERR_INVALID_ARG.
 *  - The library is thread-safe; calls that share output or workspace memory
 *    must be ordered by the caller.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,          /* null/misaligned pointer, bad size, chunk out of range */
  MOE_ERR_UNSUPPORTED = 2,          /* valid but outside the library's shape limits */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,  /* ws_bytes below what the *_workspace_size call returns */
  MOE_ERR_HIP = 4                   /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Stream schedule of moe_chunked_forward_schedule (see there). */
typedef enum moe_schedule {
  MOE_SCHEDULE_PAIR_FUSED = 0,  /* one expert-GEMM launch pair per chunk pair (default) */
  MOE_SCHEDULE_PER_CHUNK = 1,   /* every chunk runs all four steps on its own stream */
  MOE_SCHEDULE_PAIR_FUSED_PREFETCH = 2,  /* pair-fused, plus a weight warm-up on s1 */
  MOE_SCHEDULE_EXPERT_HALVES = 3  /* pair-fused, each expert GEMM split over two expert halves */
} moe_schedule;

/* Problem shape.  Field names follow the pages' notation. */
typedef struct moe_shape {
  int32_t num_tokens;    /* T: tokens of this GPU's share */
  int32_t hidden;        /* H: hidden size */
  int32_t num_experts;   /* E: routed experts */
  int32_t top_k;         /* k: experts per token */
  int32_t intermediate;  /* I: expert FFN intermediate size */
  int32_t num_groups;    /* G: destination groups of E/G contiguous experts (0 means 1) */
  int32_t num_chunks;    /* N: Chunk MoE chunk count (<= 0 means 1; N > T is legal) */
  int32_t dtype;         /* moe_dtype */
} moe_shape;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status status);

/*
 * Chunk count from the two knobs of the Chunk MoE guide (MindSpeed Chunk MoE
 * article, "操作指南" step 3): set only one of num_chunks and chunk_size; if
 * both are > 0, num_chunks wins and *warned (nullable) is set to 1; chunk_size
 * alone gives ceil(T / chunk_size); neither gives 1.  Host-only, no HIP call.
 */
int32_t moe_resolve_num_chunks(int32_t num_tokens, int32_t num_chunks, int32_t chunk_size,
                               int32_t* warned);

/*
 * Token range [*t0, *t1) of chunk `chunk`: T_chunk = ceil(T/N) tokens per chunk
 * (MindSpeed Chunk MoE article, key formulas); trailing chunks may be empty.
 * Host-only, no HIP call.
 */
moe_status moe_chunk_range(const moe_shape* shape, int32_t chunk, int32_t* t0, int32_t* t1);

/* Bytes of scratch moe_route_meta needs: per-segment expert counts of the
 * batched metadata pass (MindSpeed Chunk MoE article, timing-diagram section:
 * one metadata pass for all chunks).  Host-only. */
moe_status moe_route_meta_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * Bytes of workspace moe_chunked_forward needs: the metadata of all chunks plus
 * min(N, 2) slots of ceil(T/N)*k rows of (H + I) elements -- the pair
 * residency W_pair = O(2 x ceil(T/N)) of the Chunk MoE key formulas.  Host-only.
 */
moe_status moe_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * Routing metadata for ALL chunks in one pass (MindSpeed Chunk MoE article,
 * timing-diagram section: the metadata of every chunk is produced at once;
 * MindSpore news page, "# 02 AlltoAllV收发异构复用特性": the per-destination
 * send lists stay on the device and are reused by combine).
 *
 *  top_k_index   [T][k] int32 (in)
 *  counts        [N][E]   int32 (out): assignments of chunk c routed to expert e
 *  offsets       [N][E+1] int32 (out): exclusive prefix of counts; offsets[c][E] = valid rows
 *  group_splits  [N][G]   int32 (out): rows chunk c sends to destination group g
 *  src_row       [T*k]    int32 (out): src_row[t0_c*k + r] = flat index held by chunk row r,
 *                                      -1 past the chunk's valid rows
 *  dst_row       [T*k]    int32 (out): chunk-local row of assignment f, -1 if dropped
 *  dev_error     [1]      int32 (out, nullable): number of dropped (out-of-range) ids
 *  ws, ws_bytes  scratch of moe_route_meta_workspace_size bytes
 *
 * Rows are stable: inside one expert they keep ascending f.  Every output is an
 * exact integer result.
 */
moe_status moe_route_meta(const moe_shape* shape, const int32_t* top_k_index, int32_t* counts,
                          int32_t* offsets, int32_t* group_splits, int32_t* src_row,
                          int32_t* dst_row, int32_t* dev_error, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Permute of chunk `chunk` (MindSpeed Chunk MoE article, core principle):
 * x_perm[dst_row[f]] = hidden_states[f / k] for every assignment f of the chunk
 * with dst_row[f] >= 0.  hidden_states and dst_row are the full [T][H] and
 * [T*k] arrays; x_perm is the chunk's buffer of at least (t1-t0)*k rows of H.
 * Rows past offsets[chunk][E] are not written.  Pure data movement (bit-exact).
 *
 * Implementation choice: the call takes dst_row (token-major: each token row is
 * read once and written to its k expert rows) rather than the inverse src_row
 * (row-major gather, x_perm[r] = hidden_states[src_row[t0*k + r] / k]); both
 * give the same buffer.  The gather form is what moe_expert_gate_up_gather_pair
 * fuses into its row addressing.
 */
moe_status moe_permute(const moe_shape* shape, int32_t chunk, const void* hidden_states,
                       const int32_t* dst_row, void* x_perm, hipStream_t stream);

/*
 * First expert GEMM with the SwiGLU epilogue, grouped by expert (the expert
 * computation on the permuted, expert-contiguous rows of the MindSpeed Chunk
 * MoE article's core principle and timing diagram; the SwiGLU form is this
 * library's reading, the pages do not give the FFN):
 * act[r][i] = silu(g) * u with g = x_perm[r] . w_gate_up[e][i],
 * u = x_perm[r] . w_gate_up[e][I+i], for the rows r in
 * [offsets[chunk][e], offsets[chunk][e+1]).  offsets is the full [N][E+1]
 * array; act is the chunk's [rows][I] buffer.  Group sizes are read on the
 * device; the grid is bounded from (t1-t0)*k.
 */
moe_status moe_expert_gate_up(const moe_shape* shape, int32_t chunk, const void* x_perm,
                              const int32_t* offsets, const void* w_gate_up, void* act,
                              hipStream_t stream);

/*
 * Second expert GEMM, grouped by expert (same passage as moe_expert_gate_up):
 * y[r] = act[r] . w_down[e]^T for the rows [offsets[chunk][e],
 * offsets[chunk][e+1]) of expert e.  act is the chunk's [rows][I] buffer; y is
 * its [rows][H] buffer and may alias x_perm.  Rows past offsets[chunk][E] are
 * not written.
 */
moe_status moe_expert_down(const moe_shape* shape, int32_t chunk, const void* act,
                           const int32_t* offsets, const void* w_down, void* y,
                           hipStream_t stream);

/* moe_expert_gate_up followed by moe_expert_down on the same stream: the whole
 * expert step of one chunk (MindSpeed Chunk MoE article, timing diagram:
 * Expert(c)). */
moe_status moe_expert_ffn(const moe_shape* shape, int32_t chunk, const void* x_perm,
                          const int32_t* offsets, const void* w_gate_up, const void* w_down,
                          void* act, void* y, hipStream_t stream);

/*
 * Expert GEMMs of the two chunks of a pair, chunk and chunk + 1, each as ONE
 * grouped launch over both chunks' rows (the adjacent-chunk pairs of the
 * MindSpeed Chunk MoE article's timing diagram and the pair residency W_pair of
 * its key formulas: both chunks' rows are resident together, so
 * each expert's weights are streamed once for the pair instead of once per
 * chunk).  Row for row the same arithmetic as the single-chunk calls, so the
 * same bits.
 *
 *  x_perm0, y0  chunk `chunk`'s buffers of rows0 = (t1-t0)*k rows of H
 *               (y0 may alias x_perm0)
 *  x_perm1, y1  chunk `chunk+1`'s buffers of rows1 rows of H (y1 may alias
 *               x_perm1); ignored, and may be null, when chunk + 1 == N or that
 *               chunk is empty (then the call is the single-chunk one)
 *  act          [rows0 + rows1][I]: the pair's rows grouped by expert; expert
 *               e's rows start at offsets[chunk][e] + offsets[chunk+1][e], its
 *               chunk-`chunk` rows first (for a lone chunk: that chunk's layout)
 *  offsets      the full [N][E+1] array
 * A pair with no rows is a no-op that needs no pointer.  Rows past each chunk's
 * valid rows are not written.
 */
moe_status moe_expert_gate_up_pair(const moe_shape* shape, int32_t chunk, const void* x_perm0,
                                   const void* x_perm1, const int32_t* offsets,
                                   const void* w_gate_up, void* act, hipStream_t stream);

/*
 * moe_expert_gate_up_pair with the permute fused into the GEMM's row addressing
 * (what moe_chunked_forward's pair-fused schedule runs): row r of chunk c is
 * read straight from hidden_states[src_row[t0_c*k + r] / k] instead of from an
 * x_perm buffer.  src_row is the full [T*k] array from moe_route_meta; act as
 * for moe_expert_gate_up_pair.  Same bits as permute + moe_expert_gate_up_pair.
 */
moe_status moe_expert_gate_up_gather_pair(const moe_shape* shape, int32_t chunk,
                                          const void* hidden_states, const int32_t* src_row,
                                          const int32_t* offsets, const void* w_gate_up,
                                          void* act, hipStream_t stream);

/*
 * Down GEMM of a chunk pair as one grouped launch (same passages as
 * moe_expert_gate_up_pair): act is the pair's joint [rows0 + rows1][I] buffer
 * from moe_expert_gate_up_pair; y0 / y1 receive chunk `chunk`'s and chunk
 * `chunk+1`'s rows at their chunk-local positions (y1 ignored, may be null, when
 * chunk + 1 == N or that chunk is empty).
 */
moe_status moe_expert_down_pair(const moe_shape* shape, int32_t chunk, const void* act,
                                const int32_t* offsets, const void* w_down, void* y0, void* y1,
                                hipStream_t stream);

/* moe_expert_gate_up_pair followed by moe_expert_down_pair on the same stream
 * (same passages). */
moe_status moe_expert_ffn_pair(const moe_shape* shape, int32_t chunk, const void* x_perm0,
                               const void* x_perm1, const int32_t* offsets,
                               const void* w_gate_up, const void* w_down, void* act, void* y0,
                               void* y1, hipStream_t stream);

/*
 * Unpermute and weighted combine of chunk `chunk` (MindSpeed Chunk MoE article,
 * timing-diagram section; the combine reuses dispatch's dst_row, as the
 * MindSpore page's "# 02" reuses the dispatch lists):
 * out[t] = sum_{j<k, dst_row[t*k+j] >= 0} top_k_weights[t][j] * y[dst_row[t*k+j]],
 * summed in fp32 in ascending j and rounded once.  Writes out rows [t0, t1)
 * only; a token whose slots were all dropped gets zeros.
 */
moe_status moe_unpermute_combine(const moe_shape* shape, int32_t chunk, const void* y,
                                 const int32_t* dst_row, const float* top_k_weights, void* out,
                                 hipStream_t stream);

/*
 * The whole layer, Chunk MoE schedule (MindSpeed Chunk MoE article: timing
 * diagram and key formulas; Ascend dual-stream article, "01 Prefill
 * micro-batch" overlap of one micro-batch's compute with another's transfer).
 *
 * Metadata for all chunks runs once on s0.  Adjacent chunks (0,1), (2,3), ...
 * form pairs; at most two chunks are resident (workspace slots 0 and 1), and a
 * last odd chunk runs alone.
 *  MOE_SCHEDULE_PAIR_FUSED: one gate_up launch over the pair's rows, which
 *    gathers each row straight from hidden_states through src_row (the permute
 *    fused into the GEMM's row addressing: same rows, same bits, no x_perm
 *    buffer traffic), one down launch, one combine launch for both chunks, all
 *    on s0 (s1 is not used: on MI355X the joins that would let the second
 *    chunk's steps overlap on s1 cost more than the overlap gains).
 *  MOE_SCHEDULE_PER_CHUNK: chunk c runs permute -> gate_up -> down -> combine on
 *    stream s[c % 2] in slot c % 2, so the two chunks of a pair overlap as whole
 *    pipelines; every chunk streams the expert weights again.
 *  MOE_SCHEDULE_PAIR_FUSED_PREFETCH: the pair-fused schedule on s0, while s1
 *    (after the work already on s0) reads the first 128 bytes of every expert's
 *    gate/up weight rows into the caches during the metadata pass (Ascend
 *    dual-stream article, "02 Weight預取雙流並行": weights prefetched on a second
 *    stream while the first is busy).  Same bits; without a distinct s1 it is the
 *    pair-fused schedule.
 *  MOE_SCHEDULE_EXPERT_HALVES: the pair-fused schedule with each expert GEMM
 *    launched twice, over experts [0, E/2) and [E/2, E): the first half's down on
 *    s1 runs beside the second half's gate_up on s0, so each launch's last,
 *    partly idle moments overlap the other's work (two micro-batches on two
 *    streams, as the Ascend dual-stream article's "01 Prefill micro-batch雙流並行"
 *    splits the work, here by experts, so that no weight is read twice).  Same
 *    bits; without a distinct s1 it is the pair-fused schedule.
 * The overlap also needs s0 and s1 on different hardware queues: HIP runs its
 * streams on a few of them (GPU_MAX_HW_QUEUES, four by default), given out as
 * streams are created, and two streams that share a queue run their launches
 * one after another (same bits, no overlap).
 * Every schedule enqueues only kernels and event record / wait pairs (no
 * memsets, allocations or host reads), and s1 is forked from s0 and joined
 * back within the call, so a call can be captured in a HIP graph on s0 (the
 * library's events are created on a thread's first call on a device: make
 * that call before capturing).
 * s1 == s0 (or null) is legal and gives the same bits without overlap; the
 * result never depends on N or on the schedule.  On return s0 is ordered after
 * all work of the call.  ws must hold moe_workspace_size bytes.  dev_error is
 * nullable.  schedule outside moe_schedule -> MOE_ERR_INVALID_ARG.
 */
moe_status moe_chunked_forward_schedule(const moe_shape* shape, const void* hidden_states,
                                        const int32_t* top_k_index, const float* top_k_weights,
                                        const void* w_gate_up, const void* w_down, void* out,
                                        int32_t* dev_error, void* ws, size_t ws_bytes,
                                        hipStream_t s0, hipStream_t s1, int32_t schedule);

/* moe_chunked_forward_schedule with MOE_SCHEDULE_PAIR_FUSED.  That schedule runs
 * every step on s0; s1 is accepted (and may be null) but not used. */
moe_status moe_chunked_forward(const moe_shape* shape, const void* hidden_states,
                               const int32_t* top_k_index, const float* top_k_weights,
                               const void* w_gate_up, const void* w_down, void* out,
                               int32_t* dev_error, void* ws, size_t ws_bytes, hipStream_t s0,
                               hipStream_t s1);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * layer of moe_chunked_forward (pair-fused schedule, every step on `stream`,
 * same bits) with no workspace argument.  Its workspace is a file-scope device
 * array of 64 MiB (67108864 bytes) inside the library, one per GPU, held from
 * the first call on that GPU until the process ends; the call itself
 * allocates nothing.  Shapes whose moe_workspace_size exceeds 64 MiB return
 * MOE_ERR_WORKSPACE_TOO_SMALL before any work is enqueued (decode-sized
 * batches fit: T = 64, H = 7168, I = 2048, top-8 needs about 10 MB).  All calls
 * on one GPU share that array, which keeps the last call's contents: calls that
 * may overlap in time on one GPU race and must be ordered by the caller.
 * Other arguments and errors as for moe_chunked_forward.
 */
moe_status moe_chunked_forward_noalloc(const moe_shape* shape, const void* hidden_states,
                                       const int32_t* top_k_index, const float* top_k_weights,
                                       const void* w_gate_up, const void* w_down, void* out,
                                       int32_t* dev_error, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward of the same layer (gradient of L = sum(grad_out * out)), chunk pair
 * by chunk pair with each chunk's forward recomputed instead of stored (the
 * MindSpeed Chunk MoE guide's recompute option, "操作指南" step 3; the
 * backward mirrors the forward timing diagram chunk by chunk).
 *
 * Per pair: the permutes, the gate/up GEMM (act plus a saved copy of g and u)
 * and the down GEMM (y) are recomputed; then
 *   grad_top_k_weights[t][j] = grad_out[t] . y[r]          (fp32)
 *   grad_y[r]  = top_k_weights[t][j] grad_out[t]           (r = dst_row[t*k+j])
 *   grad_act   = grad_y W_d[e];  grad_g = grad_act u silu'(g),  grad_u = grad_act silu(g)
 *   grad_x[r]  = grad_g W_g[e] + grad_u W_u[e]
 *   grad_hidden_states[t] = sum_j grad_x[dst_row[t*k+j]]   (fp32 sum, rounded once)
 *   grad_w_down[e]    = sum over e's rows of grad_y^T act    (fp32)
 *   grad_w_gate_up[e] = sum over e's rows of [grad_g grad_u]^T x  (fp32)
 * For MOE_BF16, g, u, act, y, grad_y, grad_g, grad_u and grad_x are bf16 in
 * memory (each rounded once); products accumulate in fp32.
 * --------------------------------------------------------------------------- */

/* Bytes of workspace moe_chunked_backward needs (metadata plus min(N,2) slots of
 * ceil(T/N)*k rows of 2H + 3I elements).  Host-only. */
moe_status moe_backward_workspace_size(const moe_shape* shape, size_t* bytes);

/*
 * The whole backward.  Inputs as for moe_chunked_forward plus grad_out [T][H]
 * (dtype of the layer).  Outputs, all overwritten:
 *   grad_hidden_states [T][H] (layer dtype), grad_top_k_weights [T][k] fp32
 *   (0 for dropped slots), grad_w_gate_up [E][2I][H] fp32, grad_w_down [E][H][I]
 *   fp32 (zero for experts that receive no row).
 * Dropped ids are counted into *dev_error (nullable).  As in the forward's
 * pair-fused schedule every step runs on s0 (s1 may be null and is not used);
 * on return s0 is ordered after all work.  grad_hidden_states and
 * grad_top_k_weights do not depend on N (same bits); the weight gradients sum
 * the pairs' contributions in pair order, so they differ across N by rounding.
 */
moe_status moe_chunked_backward(const moe_shape* shape, const void* hidden_states,
                                const int32_t* top_k_index, const float* top_k_weights,
                                const void* w_gate_up, const void* w_down, const void* grad_out,
                                void* grad_hidden_states, float* grad_top_k_weights,
                                float* grad_w_gate_up, float* grad_w_down, int32_t* dev_error,
                                void* ws, size_t ws_bytes, hipStream_t s0, hipStream_t s1);

/*
 * Combine backward of chunk `chunk`: for every assignment f = t*k + j of the
 * chunk with r = dst_row[f] >= 0, grad_top_k_weights[f] = grad_out[t] . y[r]
 * (fp32) and grad_y[r] = top_k_weights[f] * grad_out[t] (rounded once); dropped
 * slots get grad_top_k_weights[f] = 0.  grad_out is the full [T][H] array, y and
 * grad_y the chunk's [rows][H] buffers (grad_y may alias y).
 */
moe_status moe_unpermute_combine_backward(const moe_shape* shape, int32_t chunk,
                                          const void* grad_out, const void* y,
                                          const int32_t* dst_row, const float* top_k_weights,
                                          void* grad_y, float* grad_top_k_weights,
                                          hipStream_t stream);

/*
 * Permute backward of chunk `chunk`: grad_hidden[t] = sum over kept slots j of
 * grad_x_perm[dst_row[t*k+j]], fp32 in ascending j, rounded once; rows [t0, t1)
 * of grad_hidden only.
 */
moe_status moe_permute_backward(const moe_shape* shape, int32_t chunk, const void* grad_x_perm,
                                const int32_t* dst_row, void* grad_hidden, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
