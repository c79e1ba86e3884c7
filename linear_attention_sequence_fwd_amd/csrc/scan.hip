// Scan of per-segment end states for the segmented chunkwise forward.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "3. The
// Chunkwise Recurrent Representation": the state carried from one chunk to the
// next is decayed by gamma^L and gains the chunk's own contribution. Applied
// to runs of chunks (segments), the start state of segment s is
//     S_in(s) = gamma^seg_len S_in(s-1) + T_(s-1)
// with T_(s-1) the end state of segment s-1 built from a zero state.

#include "common.hpp"
#include "kernels.hpp"

namespace ret {

// Exclusive scan of segment end states with factor gamma^seg_len, in place.
// Slot 0 receives the initial state (state_in or zeros); slot s >= 1 holds the
// end state of segment s-1 built from zero and is replaced by the state at
// the start of segment s. One thread owns four consecutive state elements and
// walks the segments in order; a wavefront covers 256 contiguous elements.
__device__ __forceinline__ void segment_scan_body(float* ws, const float* state_in, int H, int nseg, int per_bh,
                                                  int seg_len, const HeadParams& hp, int bh, int e4) {
    if (e4 * 4 >= per_bh) return;
    const float gL = gamma_pow(log2_gamma(hp.gamma[bh % H]), seg_len);
    float4* w = reinterpret_cast<float4*>(ws + static_cast<size_t>(bh) * nseg * per_bh) + e4;
    const size_t stride = per_bh / 4;
    float4 acc = state_in ? reinterpret_cast<const float4*>(state_in + static_cast<size_t>(bh) * per_bh)[e4]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    w[0] = acc;
    // Loads are issued in batches ahead of the dependent updates so several
    // segments are in flight per thread (the slots are disjoint from the
    // ones being written, but the compiler cannot prove it).
    constexpr int kBatch = 32;
    for (int s0 = 1; s0 < nseg; s0 += kBatch) {
        float4 t[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (s0 + j < nseg) t[j] = w[(s0 + j) * stride];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (s0 + j < nseg) {
                acc.x = gL * acc.x + t[j].x;
                acc.y = gL * acc.y + t[j].y;
                acc.z = gL * acc.z + t[j].z;
                acc.w = gL * acc.w + t[j].w;
                w[(s0 + j) * stride] = acc;
            }
        }
    }
}

__global__ __launch_bounds__(256) void segment_scan_kernel(float* ws, const float* state_in, int H, int nseg,
                                                           int per_bh, int seg_len, HeadParams hp) {
    segment_scan_body(ws, state_in, H, nseg, per_bh, seg_len, hp, blockIdx.y,
                      blockIdx.x * blockDim.x + threadIdx.x);
}

// The scans of several calls in one launch (call blockIdx.z), each over its
// own workspace slots.
__global__ __launch_bounds__(256) void segment_scan_multi_kernel(ChunkCalls cs, HeadParams hp) {
    const ChunkArgs& a = cs.a[blockIdx.z];
    if (static_cast<int>(blockIdx.y) >= a.B * a.H) return;
    segment_scan_body(a.agg, a.state_in, a.H, a.nseg, a.dk * a.dv, a.seg_len, hp, blockIdx.y,
                      blockIdx.x * blockDim.x + threadIdx.x);
}

hipError_t launch_segment_scan(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev) {
    const int per_bh = a.dk * a.dv;
    dim3 grid((per_bh / 4 + 255) / 256, a.B * a.H);
    launch_timed(segment_scan_kernel, grid, dim3(256), 0, st, ev, a.agg, a.state_in, a.H, a.nseg, per_bh,
                 a.seg_len, hp);
    return hipGetLastError();
}

hipError_t launch_segment_scan_multi(const ChunkCalls& cs, const HeadParams& hp, hipStream_t st) {
    int per_max = 0, bh_max = 0;
    for (int i = 0; i < cs.n; ++i) {
        per_max = max(per_max, cs.a[i].dk * cs.a[i].dv);
        bh_max = max(bh_max, cs.a[i].B * cs.a[i].H);
    }
    const dim3 grid((per_max / 4 + 255) / 256, bh_max, cs.n);
    hipLaunchKernelGGL(segment_scan_multi_kernel, grid, dim3(256), 0, st, cs, hp);
    return hipGetLastError();
}

}  // namespace ret
