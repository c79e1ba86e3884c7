/*
 * retention.h -- C ABI of the MI355X (gfx950) multi-scale retention library.
 *
 * Retention per batch b and head h, on query/key rows q'_n, k'_m (after the
 * optional complex rotation) and value rows v_m:
 *
 *     o_n = sum_{m <= n} gamma_h^(n - m) (q'_n . k'_m) v_m
 *
 * ("RetNet Guide: Retentive Networks & The Impossible Triangle", sections
 * "The Parallel Representation", "The Recurrent Representation" and "The
 * Chunkwise Recurrent Representation"; "How RetNet Combines Parallel Training
 * and Constant Inference").
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, contiguous device buffers owned by the
 *     caller: q, k [B, H, N, dk]; v, o [B, H, N, dv]; state [B, H, dk, dv].
 *     Device pointers must be 16-byte aligned.
 *   - dtype selects the element type of q, k, v and o (RET_F32 or RET_BF16).
 *     The recurrent state is always float32; accumulation is always float32.
 *   - gamma: host array of H floats, each in (0, 1], read during the call; NULL
 *     selects gamma_h = 1 - 2^(-5-h), heads counted from 0 ("RetNet Guide"
 *     section "3. Multi-Scale Retention (MSR)").
 *   - theta: host array of dk/2 floats, read during the call, or NULL for no
 *     rotation. With theta, coordinates (2j, 2j+1) of every query and key row
 *     are treated as the complex number x_2j + i x_2j+1 and multiplied by
 *     e^(i n theta_j) at absolute position n ("RetNet Guide" section "2.
 *     Relative Position via Complex Exponential Phase Rotations"). Angles are
 *     formed in float64. Values are never rotated.
 *   - No 1/sqrt(dk) score scale is applied; callers fold it into q.
 *   - Every call validates all arguments before touching the GPU, launches
 *     asynchronously on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns a status. Launch failures reported by hipGetLastError map to
 *     RET_ERR_HIP; faults inside kernels surface at the caller's next
 *     synchronisation. The library allocates no device memory and keeps no
 *     state between calls. Nothing is written when a call returns an error
 *     found during validation. Checks run in this order, and the first
 *     failure is returned: NULL pointers, sizes and dtype, gamma and theta
 *     values, pointer alignment, the implemented set, the workspace.
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RETENTION_ABI_VERSION 4
#define RETENTION_MAX_HEADS 128 /* H limit (per-head constants travel in kernel arguments) */
#define RETENTION_MAX_DK 256

typedef enum { RET_F32 = 0, RET_BF16 = 1 } ret_dtype_t;

typedef enum {
    RET_OK = 0,
    RET_ERR_NULL = 1,        /* a required pointer is NULL */
    RET_ERR_SHAPE = 2,       /* a size is < 1, or dk is odd while theta is given */
    RET_ERR_DTYPE = 3,       /* dtype is not one of ret_dtype_t */
    RET_ERR_GAMMA = 4,       /* a gamma is not in (0, 1] or not finite, or theta not finite */
    RET_ERR_UNSUPPORTED = 5, /* valid request outside the implemented set (see each call) */
    RET_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
    RET_ERR_ALIGN = 7,       /* a device pointer is not 16-byte aligned */
    RET_ERR_HIP = 8          /* the HIP runtime reported a launch error */
} ret_status_t;

/*
 * Parallel form: O = ((Q' K'^T) (.) D) V with D[n, m] = gamma^(n - m) for
 * n >= m, else 0 ("RetNet Guide" section "1. The Parallel Representation for
 * High-Throughput Pretraining"). Positions are pos0 .. pos0 + N - 1.
 * Implemented set: bf16 with dk in {64, 128, 256} and dv a multiple of 64;
 * f32 with dk <= 128 and dv a multiple of 16 (dk a multiple of 4).
 * Work is O(N^2) per head; key blocks whose decay underflows float32 for every
 * entry are skipped (their exact contribution is below float32 resolution).
 */
ret_status_t retention_parallel_fwd(const void* q, const void* k, const void* v, void* o,
                                    int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                    const float* gamma, const float* theta, int64_t pos0,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace retention_parallel_fwd can use for these sizes (0: it
 * uses none). Causal work grows with a query block's position, so when the
 * query blocks alone would leave compute units idle (bf16 without rotation,
 * d_k 64 or 128, at most 512 blocks of 128 queries over heads and value
 * tiles), the key walk of every query block longer than half the longest is
 * split over two workgroups, whose float32 partial outputs meet in this
 * workspace and the later of the two adds them. The workspace follows the
 * chunkwise forward's contract: zero-filled before its first use, left ready
 * by every call, calls sharing it ordered on one stream. With a NULL
 * workspace the call runs every query block's walk in one workgroup (same
 * result up to float32 rounding order); a workspace smaller than this size is
 * RET_ERR_WORKSPACE.
 */
size_t retention_parallel_workspace_size(int B, int H, int N, int dk, int dv, ret_dtype_t dtype);

/*
 * Chunkwise recurrent form ("RetNet Guide" section "3. The Chunkwise Recurrent
 * Representation"): the sequence is cut into chunks of `chunk` tokens (the
 * last may be shorter). Inside a chunk the parallel form is used; between
 * chunks a float32 state S [dk, dv] is carried:
 *     O_X = ((Q_X K_X^T) (.) D) V_X + zeta (.) (Q_X S),   zeta_j = gamma^(j+1)
 *     S  <- gamma^L S + K_X^T (xi (.) V_X),               xi_j   = gamma^(L-1-j)
 * (L = chunk length; the xi weights are the in-chunk key decay implied by the
 * recurrent form). Same result as the parallel form up to rounding.
 *
 * state_in:  device float32 [B, H, dk, dv] state before the first token, or
 *            NULL for zeros. Positions are pos0 .. pos0 + N - 1, so a long
 *            sequence may be processed in pieces by handing state_out of one
 *            call to state_in of the next with pos0 advanced.
 * state_out: device float32 [B, H, dk, dv] receiving the state after the last
 *            token, or NULL. May alias state_in.
 * segments:  0 lets the library choose; s >= 1 asks for s sequence segments
 *            (clamped to the number of chunks and to 4096; ignored when
 *            B*H*(value tiles) exceeds 512). With more than one segment
 *            the sequence of every head is cut into segments that run in
 *            parallel, and the state entering each segment is assembled from
 *            the end states of the segments before it, with factor
 *            gamma^(segment length) per segment. bf16 does this in one launch
 *            (workgroups publish segment states and look back at their
 *            predecessors' through the workspace), except for unrotated
 *            heads with dk of 128 or 256 in 128-token chunks, which run
 *            three kernels like float32 (segment end states, their scan,
 *            the segments).
 * workspace: device buffer of at least retention_chunkwise_workspace_size(...)
 *            bytes (may be NULL when that size is 0). It must be zero-filled
 *            before its first use (one hipMemset after allocation); every
 *            call leaves it ready for the next, so it can be reused without
 *            clearing, by calls of any sizes and from a captured graph.
 *            Calls that share a
 *            workspace must be ordered on one stream (they must not overlap).
 *            The caller owns it; the library keeps no pointer to it.
 * Large chunks ("RetNet Guide" section "3. The Chunkwise Recurrent
 * Representation" suggests 512 or 1024 tokens for long prefill): for bf16,
 * chunk may be any multiple of 128 up to 65536. Inside a chunk the kernel
 * still works in 128-token tiles (the matrix-core tile that fits the register
 * file); the state is exchanged between chunks, which run in parallel as
 * segments (`segments` is then ignored: one segment per chunk, at most 4096).
 * The workspace then grows with N / chunk (one state per chunk).
 * Implemented set: chunk in {64, 128} (and the large chunks above for bf16;
 * f32 also takes 16 and 32); bf16 with dk in {64, 128, 256} and dv a multiple
 * of 64; f32 with chunk*dk <= 8192, dk a multiple of 4, dv a multiple of 16.
 */
ret_status_t retention_chunkwise_fwd(const void* q, const void* k, const void* v, void* o,
                                     int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                     int chunk, const float* gamma, const float* theta,
                                     int64_t pos0, const float* state_in, float* state_out,
                                     int segments, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * retention_chunkwise_fwd with a timing hook for profilers and benchmarks:
 * events points to six hipEvent_t created by the caller, a start/stop pair for
 * each phase in order: segment pre-pass, segment scan, main chunk kernel. Each
 * pair brackets that kernel's execution on `stream` (recorded by the launch
 * itself, so host submission gaps are not included); a phase that does not
 * run records its pair back to back (bf16 runs every form as the one main
 * kernel, so its first two pairs are always empty). Same result and status codes as
 * retention_chunkwise_fwd (RET_ERR_NULL if an event is missing).
 */
ret_status_t retention_chunkwise_fwd_timed(const void* q, const void* k, const void* v, void* o,
                                           int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                           int chunk, const float* gamma, const float* theta,
                                           int64_t pos0, const float* state_in, float* state_out,
                                           int segments, void* workspace, size_t workspace_bytes,
                                           void* stream, void* const* events);

/*
 * retention_chunkwise_fwd for callers that cannot allocate memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call without a workspace argument. The workspace of the segmented
 * form lives in a device array of the library, RETENTION_NOALLOC_SCRATCH_BYTES
 * bytes per GPU, held until the process ends; its address is looked up once
 * per device (the current device of the calling thread, which must be the
 * device of the tensors and the stream). The call allocates nothing.
 * Returns RET_ERR_WORKSPACE when these sizes need more workspace than that
 * (retention_chunkwise_workspace_size tells), RET_ERR_HIP if the array's
 * address cannot be obtained; otherwise the results and status codes of
 * retention_chunkwise_fwd. Every call on one GPU shares that array: calls
 * that overlap on one GPU (concurrent streams, several host threads) race and
 * must be serialised by the caller.
 */
#define RETENTION_NOALLOC_SCRATCH_BYTES (32u << 20)
ret_status_t retention_chunkwise_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                             int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                             int chunk, const float* gamma, const float* theta,
                                             int64_t pos0, const float* state_in, float* state_out,
                                             int segments, void* stream);

/*
 * Bytes of workspace retention_chunkwise_fwd needs for these sizes and this
 * `segments` request. For chunk <= 128 the value does not depend on N (the
 * segment count is bounded independently of the sequence length). Returns 0
 * for sizes the call would reject.
 */
size_t retention_chunkwise_workspace_size(int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                          int chunk, int segments);

/*
 * The plan retention_chunkwise_fwd follows for these sizes (a diagnostic for
 * callers and tests; the pages define no such call): the kernel's token tile,
 * value-tile width and count, how each (batch, head) sequence is cut into
 * segments and grouped for the state look-back, and the byte offsets of the
 * workspace regions the segmented kernels index. "Chains" are the
 * B * H * value_tiles independent (batch, head, value tile) sequences.
 *   ticket counters  [0, flags_off): one 8-byte counter per chain, 128 bytes apart
 *   segment flags    [flags_off, gflags_off): chain * segments + segment, 128 bytes apart
 *   group flags      [gflags_off, agg_off): chain * groups + group, 128 bytes apart
 *   segment states   [agg_off, gagg_off): bf16 look-back: chain * segments + segment,
 *                    dk * dv_tile floats each; the three-kernel form (float32, and
 *                    bf16 unrotated dk 128/256 in 128-token tiles of 128 value
 *                    columns): [B, H, segments, dk, dv] floats
 *   group states     [gagg_off, workspace_bytes): chain * groups + group, dk * dv_tile floats
 * with groups = ceil(segments / group_len). A plan with segments == 1 uses no
 * workspace (workspace_bytes == 0). Returns the status retention_chunkwise_fwd
 * would return for these sizes (RET_OK, RET_ERR_SHAPE, RET_ERR_DTYPE or
 * RET_ERR_UNSUPPORTED); `plan` (host memory, not NULL) is filled on RET_OK.
 */
typedef struct {
    int tile;           /* tokens per kernel chunk tile (16, 32, 64 or 128) */
    int dv_tile;        /* value columns per workgroup */
    int value_tiles;    /* dv / dv_tile */
    int segments;       /* segments per (batch, head) sequence */
    int segment_len;    /* tokens per segment (a multiple of tile) */
    int group_len;      /* segments per look-back group */
    int segments_max;   /* segments the workspace holds per chain */
    int reserved;
    uint64_t flags_off, gflags_off, agg_off, gagg_off, workspace_bytes;
} ret_chunk_plan_t;

ret_status_t retention_chunkwise_plan(int B, int H, int N, int dk, int dv, ret_dtype_t dtype, int chunk,
                                      int segments, ret_chunk_plan_t* plan);

/*
 * Backward of retention_chunkwise_fwd (whose result is that of the parallel
 * form, which is how training evaluates retention: "RetNet Guide" section "1.
 * The Parallel Representation for High-Throughput Pretraining"; "Retentive
 * Networks (RetNet)", "At a glance": training stays parallel over the
 * sequence). For the forward O, S_N of the same q, k, v, gamma, theta, pos0 and
 * state_in, and the gradients d_o = dL/dO and d_state_out = dL/dS_N, it writes
 *     d_q, d_k [B, H, N, dk] and d_v [B, H, N, dv] (dtype): dL/dq, dL/dk, dL/dv
 *     d_state_in [B, H, dk, dv] float32 (when not NULL): dL/d(state_in)
 * Per head, with Q', K' the rotated rows, Z_n = gamma^(n+1), Xi_m = gamma^(N-1-m):
 *     dV  = ((Q' K'^T) (.) D)^T dO + Xi (.) (K' dS)
 *     dQ' = ((dO V^T) (.) D) K' + Z (.) (dO S0^T),   dq = rotation of dQ' by -theta
 *     dK' = ((dO V^T) (.) D)^T Q' + Xi (.) (V dS^T), dk likewise
 *     dS0 = Q'^T (Z (.) dO) + gamma^N dS
 * Each of dQ', dK', dV is computed as one chunkwise forward pass (the last two
 * over the reversed sequence, where the transposed decay matrix is causal);
 * for bf16 the matrix-core kernel reads and writes those two in reverse token
 * order itself, and with dk == dv the three passes share one launch.
 *
 * d_o:         device [B, H, N, dv] in dtype.
 * state_in:    the forward's initial state, or NULL for zeros.
 * d_state_out: device float32 [B, H, dk, dv], or NULL for zeros.
 * d_state_in:  device float32 [B, H, dk, dv] to receive dL/d(state_in), or
 *              NULL. May alias d_state_out or state_in; d_q, d_k, d_v must not
 *              overlap any input or each other.
 * workspace:   device buffer of retention_chunkwise_bwd_workspace_size(...)
 *              bytes (it grows with N: it holds the rotated copies of q and k,
 *              and for float32 reversed copies of q, k, v and d_o). It needs
 *              no initialisation: every call clears
 *              the counters its passes use, in a kernel (so the call can be
 *              captured in a graph). Backward calls of any sizes may share it
 *              when ordered on one stream; a forward workspace must not be the
 *              same memory (the backward's scratch would overwrite the
 *              counters a forward call expects to find). The caller owns it.
 * Implemented set: retention_chunkwise_fwd's chunks; dk and dv multiples of
 * 8, and each of (dk, dv) and (dv, dk) inside retention_chunkwise_fwd's set,
 * except that for bf16 a dv twice a supported key width is taken too (the two
 * passes keyed by dv then run over its halves): bf16 with dk in {64, 128, 256}
 * and dv in {64, 128, 256, 512}; f32 with chunk*dk and chunk*dv <= 8192, both
 * multiples of 16; with d_state_out, every gamma >= 2^-20.
 */
ret_status_t retention_chunkwise_bwd(const void* q, const void* k, const void* v, const void* d_o,
                                     void* d_q, void* d_k, void* d_v, int B, int H, int N, int dk, int dv,
                                     ret_dtype_t dtype, int chunk, const float* gamma, const float* theta,
                                     int64_t pos0, const float* state_in, const float* d_state_out,
                                     float* d_state_in, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Bytes of workspace retention_chunkwise_bwd needs; 0 for sizes it would reject. */
size_t retention_chunkwise_bwd_workspace_size(int B, int H, int N, int dk, int dv, ret_dtype_t dtype,
                                              int chunk);

/*
 * One recurrent decode step for one token per sequence ("RetNet Guide" section
 * "2. The Recurrent Representation for Constant-Memory O(1) Decoding"):
 *     S <- gamma S + k'^T v ;  o = q' S   (with the updated S)
 * q, k: [B, H, dk]; v, o: [B, H, dv] in dtype; state: device float32
 * [B, H, dk, dv], updated in place. pos: device int64 [B] absolute position of
 * each sequence's token (used only with theta; may be NULL without theta).
 * Implemented set: dv a multiple of 4 with dv <= 1024, dk <= 4096.
 */
ret_status_t retention_recurrent_step(const void* q, const void* k, const void* v, void* o,
                                      float* state, int B, int H, int dk, int dv,
                                      ret_dtype_t dtype, const float* gamma, const float* theta,
                                      const int64_t* pos, void* stream);

/*
 * Output stage of multi-scale retention ("RetNet Guide" section "1. The
 * Parallel Representation for High-Throughput Pretraining": MSR(X) =
 * GroupNorm(Concat(R_1, ..., R_H)) W_O; its listing uses one GroupNorm group
 * per head with eps 1e-6 and a bias-free projection; "How RetNet Combines
 * Parallel Training and Constant Inference" adds a gate, with no formula):
 *     Z[b, n, h*dv + j] = ((o[b,h,n,j] - mean) / sqrt(var + eps) * w[h*dv+j]
 *                          + beta[h*dv+j]) * gate[b, n, h*dv+j]
 *     y[b, n, :] = Z[b, n, :] W_O^T
 * with mean and (biased) var over the dv channels of head h of token n.
 *
 * o:         device bf16 [B, H, N, dv], a retention call's output.
 * gate:      device bf16 [B, N, H*dv] or NULL (no gate); the caller applies
 *            whatever activation its gate uses.
 * gn_weight, gn_bias: device float32 [H*dv] or NULL (ones / zeros).
 * eps:       >= 0 and finite (else RET_ERR_GAMMA).
 * w_o:       device bf16 [d_out, H*dv] (the layout of a linear layer's weight).
 * y:         device bf16 [B, N, d_out], written.
 * workspace: retention_msr_epilogue_workspace_size(...) bytes (holds Z); no
 *            initialisation needed.
 * Implemented set: dtype RET_BF16, dv in {64, 128, 256, 512}, d_out a
 * multiple of 128, H*dv a multiple of 64.
 */
ret_status_t retention_msr_epilogue(const void* o, const void* gate, const float* gn_weight,
                                    const float* gn_bias, float eps, const void* w_o, void* y, int B,
                                    int H, int N, int dv, int d_out, ret_dtype_t dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Bytes of workspace retention_msr_epilogue needs; 0 for sizes it would reject. */
size_t retention_msr_epilogue_workspace_size(int B, int H, int N, int dv, int d_out, ret_dtype_t dtype);

/*
 * One decode step of a multi-scale retention layer: retention_recurrent_step
 * (state updated in place, o = q' S written to `o`, device [B, H, dv]) followed
 * by retention_msr_epilogue on that token (o read as [B, H, 1, dv]; gate
 * [B, H*dv] or NULL): y [B, d_out] = (GroupNorm(o) * gate) W_O^T ("RetNet
 * Guide" section "2. The Recurrent Representation for Constant-Memory O(1)
 * Decoding": the listing's recurrent step normalises and projects each
 * token's output). With few tokens the projection splits its contraction over
 * workgroups so the whole of W_O streams from HBM in parallel. When one
 * workgroup of the step owns a whole (sequence, head) row (B*H >= 256, or d_v
 * not a multiple of 128), the step also normalises and gates that row, and no separate
 * GroupNorm pass runs; o and y are the same either way up to float32 rounding
 * order in the statistics.
 * Arguments as in the two calls; workspace:
 * retention_msr_epilogue_workspace_size(B, H, 1, dv, d_out, RET_BF16) bytes.
 * Implemented set: bf16, and each call's own set.
 */
ret_status_t retention_recurrent_step_msr(const void* q, const void* k, const void* v, float* state,
                                          int B, int H, int dk, int dv, ret_dtype_t dtype,
                                          const float* gamma, const float* theta, const int64_t* pos,
                                          const void* gate, const float* gn_weight, const float* gn_bias,
                                          float eps, const void* w_o, int d_out, void* o, void* y,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* retention_status_string(ret_status_t status);

/* RETENTION_ABI_VERSION of the built library. */
int retention_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RETENTION_H */
