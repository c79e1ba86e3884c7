// Host-side launch interface between the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
    float* ws;              // [B*H][nseg][dk][dv] when nseg > 1
    int B, H, N, dk, dv;
    int chunk;
    int nvt;      // value tiles per head
    int nseg;     // sequence segments per head
    int seg_len;  // tokens per segment, a multiple of chunk
    long long pos0;
};

struct ParallelArgs {
    const u16* q;
    const u16* k;
    const u16* v;
    u16* o;
    int B, H, N, dk, dv;
    int nvt;
    long long pos0;
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
};

// Optional timing hook: when ev is not null, ev[0..3] are recorded on the
// stream before the segment pre-pass, after it, after the segment scan and
// after the main chunk kernel (phases that do not run record back-to-back).
hipError_t launch_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev);
hipError_t launch_chunk_f32(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev);
hipError_t launch_parallel_bf16(const ParallelArgs& a, const HeadParams& hp, int dvt, hipStream_t st);
hipError_t launch_parallel_f32(const ParallelArgs& a, const HeadParams& hp, int dvt, hipStream_t st);
hipError_t launch_recurrent_step(const StepArgs& a, const HeadParams& hp, hipStream_t st);
hipError_t launch_segment_scan(const ChunkArgs& a, const HeadParams& hp, hipStream_t st);

}  // namespace ret
