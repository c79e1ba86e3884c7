// Host-side launch interface between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <hip/hip_ext.h>

#include "common.hpp"

namespace ret {

// Arguments of the chunkwise forward, already validated by the ABI layer.
struct ChunkArgs {
    const u16* q;  // element type is u16 for bf16 and reinterpreted as float for f32
    const u16* k;
    const u16* v;
    u16* o;
    const float* state_in;  // [B,H,dk,dv] or nullptr
    float* state_out;       // [B,H,dk,dv] or nullptr
    // Workspace regions when nseg > 1 (carved out of the caller's workspace):
    unsigned long long* ctl;    // per chain: ticket counter (low 32 bits) and generation (high 32 bits)
    unsigned long long* flags;  // [B*H*nvt][nseg] publication flags of the bf16 look-back
    float* agg;                 // published per-segment states: bf16 [B*H*nvt][nseg][dk*dvt] in
                                // accumulator order; float32 [B*H][nseg][dk][dv]
    unsigned long long* gflags;  // [B*H*nvt][ngroups] flags of the bf16 segment-group aggregates
    float* gagg;                 // [B*H*nvt][ngroups][dk*dvt] segment-group aggregates
    int B, H, N, dk, dv;
    int chunk;
    int nvt;      // value tiles per head
    int nseg;     // sequence segments per head
    int seg_len;  // tokens per segment, a multiple of chunk
    int grp;      // segments per look-back group (bf16 segmented form)
    long long pos0;
    int rev;      // rows in reverse token order (chunk_bf16_multi_kernel only; no rotation then)
    int orot;     // rotate each output row by minus theta at its token's position before rounding
                  // (chunk_bf16_multi_kernel only, where chunk_orot_fits; output columns are the pairs)
    int rescale;  // chunks per decay group of chunk_wide_kernel (set by launch_chunk_bf16)
    int ldqk;     // row stride of q and k in elements (0: dk; chunk_wide kernels only, which then
                  // read a dk-wide column block of wider rows)
};

// Ticket counters of the segmented bf16 chunk kernel: one per chain, each on a
// 128-byte line of its own (64-bit words apart).
constexpr int kCtlStride = 16;
// Published-state flags (per chain and segment, per chain and segment group)
// likewise sit one per 128-byte line.
constexpr int kFlagStride = 16;

// LDS bytes of the bf16 chunk kernel's tiles (keys, values, state copy), and
// whether the multi-call kernel also holds the output rotation's frequencies
// next to them within a compute unit's 160 KiB.
constexpr int chunk_bf16_tile_lds(int dk, int dvt, int c) { return (c * dk + dvt * c + dvt * dk) * 2; }
constexpr bool chunk_orot_fits(int dk, int dvt, int c) { return chunk_bf16_tile_lds(dk, dvt, c) + dvt * 2 <= 160 * 1024; }

// Several chunkwise calls with one tile and kernel form (different tensors,
// states and workspace regions) run by one launch; `first` and `interleave`
// are filled by launch_chunk_bf16_multi.
constexpr int kMaxChunkCalls = 5;
struct ChunkCalls {
    ChunkArgs a[kMaxChunkCalls];
    int n;
    int first[kMaxChunkCalls + 1];  // workgroup ranges when the calls differ in size
    int interleave;                 // calls of one size: workgroup b serves call b % n
};

struct ParallelArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    u16* o;
    int B, H, N, dk, dv;
    int nvt;
    long long pos0;
    // balanced schedule of parallel_wide_kernel (split_t == 0: none): the key walks of
    // query blocks longer than split_t blocks go to two workgroups, whose float32
    // partials meet in `part` ([split block][2][128 x 128]) under ticket `ctr`
    // ([split block], at most 256)
    int split_t;
    float* part;
    unsigned* ctr;
};

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* state;
    const int64_t* pos;
    int B, H, dk, dv;
    int bf16;
    int ntile;  // column tiles per (sequence, head), see recurrent_step_tiles
    // Optional GroupNorm-and-gate epilogue (bf16, ntile == 1 only; z == nullptr: none):
    // z[b, h*dv + c] = ((o - mean) / sqrt(var + eps) * gn_w + gn_b) * gate over the
    // head's dv channels of the bf16 o, as groupnorm_gate_kernel computes it.
    const u16* gate;     // [B, H*dv] bf16 or nullptr (ones)
    const float* gn_w;   // [H*dv] or nullptr (ones)
    const float* gn_b;   // [H*dv] or nullptr (zeros)
    u16* z;              // [B, H*dv] bf16 out
    float eps;
};

// Row transforms of the backward (backward.hip): one job per tensor.
struct RowJob {
    const void* src;  // [B,H,N,src_ld] rows; the job reads columns src_col .. src_col + d - 1
    void* dst0;       // [B,H,N,d]; row t lands at N-1-t when flip0
    void* dst1;       // optional second copy, rows in order (nullptr: none)
    int d;            // row width in elements, a multiple of 8
    int flip0;
    int rot;          // 0: none, +1: rotate by +theta, -1: by -theta
    int src_rev;      // src rows are in reverse token order: row t holds token N-1-t (its rotation position)
    int src_ld;       // row stride of src in elements (0: d)
    int src_col;      // first column read from src
    const void* add;  // optional [B,H,N,d] rows added to src before the rotation (nullptr: none)
};

constexpr int kMaxRowJobs = 6;
constexpr int kMaxZeroRegions = 5;
struct RowJobs {
    RowJob j[kMaxRowJobs];
    int n;  // jobs in use
    int B, H, N;
    long long pos0;
    // Optional extra grid row that zero-fills nzero 16-byte units at each
    // non-null zero[i] (nzero = 0: none).
    uint4* zero[kMaxZeroRegions];
    long long nzero;
};

// State transforms of the backward: mode 0 writes x1 = s0^T, x2 = ds^T / gamma,
// x3 = ds / gamma (per head, [dk, dv] sources); mode 1 scales dsi by gamma.
// With split, x1 and x2 ([dv, dk] per head) are written as two arrays of their
// first and second dv/2 rows, [B,H,dv/2,dk] each, one after the other.
struct StateJobs {
    const float* s0;
    const float* ds;
    float* x1;
    float* x2;
    float* x3;
    float* dsi;
    int B, H, dk, dv;
    int mode;
    int split;
};

// Output stage (epilogue.hip).
struct EpilogueArgs {
    const u16* o;          // [B,H,N,dv] bf16
    const u16* gate;       // [B*N, H*dv] bf16 or nullptr
    const float* gn_weight;  // [H*dv] or nullptr (ones)
    const float* gn_bias;    // [H*dv] or nullptr (zeros)
    u16* z;                // [B*N, H*dv] bf16 out
    int B, H, N, dv;
    float eps;
};

struct GemmArgs {  // c[M, N] = a[M, K] b[N, K]^T, all bf16 row-major
    const u16* a;
    const u16* b;
    u16* c;
    float* part;  // [splits][M][N] float32 partial sums when gemm_splits(M, N, K) > 1
    int M, N, K;
    int splits;
};

int gemm_splits(int M, int N, int K);

hipError_t launch_groupnorm_gate(const EpilogueArgs& a, hipStream_t st);
hipError_t launch_gemm_bt(const GemmArgs& g, hipStream_t st);

hipError_t launch_rows(const RowJobs& jobs, const HeadParams& hp, bool bf16, hipStream_t st);
hipError_t launch_states(const StateJobs& sj, const HeadParams& hp, hipStream_t st);

// Optional timing hook: when ev is not null it holds six events, a start/stop
// pair per phase (segment pre-pass, segment scan, main chunk kernel), each pair
// recorded by the launch itself around that kernel's execution
// (hipExtLaunchKernelGGL); a phase that does not run records its pair back to
// back.
hipError_t launch_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev);
// The wide-head kernel (chunk_wide.hip): d_k 128 or 256, value tiles of 128
// columns, 128-token chunks, no rotation, gammas with gamma^128 >= 2^-64. One
// pass per chain, or with a.nseg > 1 three launches (segment end states, their
// scan in a.agg, the segments); launch_chunk_wide records the six phase events.
bool chunk_wide_supported(int dk, int dvt, int chunk, bool rotation);
int chunk_wide_rescale(const HeadParams& hp, int H);
hipError_t launch_chunk_wide(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev);
// several unrotated calls of one key width (128 or 256), chunk 128, 128-column value tiles,
// all whole (one launch) or all segmented (one launch per phase), a.rev honoured; rescale is
// filled in here
hipError_t launch_chunk_wide_multi(const ChunkCalls& cs, const HeadParams& hp, hipStream_t st);
hipError_t launch_chunk_bf16_multi(const ChunkCalls& cs, const HeadParams& hp, int dvt, hipStream_t st);
hipError_t launch_chunk_f32(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev);
hipError_t launch_parallel_bf16(const ParallelArgs& a, const HeadParams& hp, int dvt, hipStream_t st);
// The single-wave-per-SIMD parallel kernel (parallel_wide.hip): no rotation,
// d_k 64 or 128, value tiles of 128 columns (a.nvt = dv / 128).
bool parallel_wide_supported(int dk, int dv, bool rotation);
// split threshold of parallel_wide_kernel for these sizes (0: no split) and the
// workspace bytes it then needs
int parallel_wide_split(int B, int H, int N, int dv);
size_t parallel_wide_workspace(int B, int H, int N, int dv);
// point a's split schedule at a workspace of parallel_wide_workspace bytes
void parallel_wide_bind(ParallelArgs& a, void* workspace);
hipError_t launch_parallel_wide(const ParallelArgs& a, const HeadParams& hp, hipStream_t st);
hipError_t launch_parallel_f32(const ParallelArgs& a, const HeadParams& hp, int dvt, hipStream_t st);
hipError_t launch_recurrent_step(const StepArgs& a, const HeadParams& hp, hipStream_t st);
int recurrent_step_tiles(int B, int H, int dv);
hipError_t launch_segment_scan(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev);
hipError_t launch_segment_scan_multi(const ChunkCalls& cs, const HeadParams& hp, hipStream_t st);

// Launch `kernel` with the given configuration; with events, bracket its
// execution with ev[0] / ev[1].
template <typename... KArgs, typename... Args>
inline void launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                         hipEvent_t* ev, Args... args) {
    if (ev)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, ev[0], ev[1], 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
}

// Record a phase that does not run (start and stop back to back).
inline void record_empty_phase(hipStream_t st, hipEvent_t* ev) {
    if (ev) {
        (void)hipEventRecord(ev[0], st);
        (void)hipEventRecord(ev[1], st);
    }
}

}  // namespace ret
