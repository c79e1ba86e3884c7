// Recurrent decode step: one token per sequence, state updated in place.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "2. The
// Recurrent Representation for Constant-Memory O(1) Decoding":
//     S <- gamma S + k^T v ;  o = q S   (the updated S)
// The step is a pure read-modify-write of the float32 d_k x d_v state, so it
// is bound by HBM: each state element is read once and written once with
// 16-byte non-temporal accesses (the state of a large batch does not fit in
// the caches, and keeping it out of them leaves room for q, k, v). One
// workgroup owns one (sequence, head) and a tile of the state's columns: the
// whole row width when there are enough (sequence, head) pairs to fill the
// chip, else d_v is split into tiles of at least 64 columns so that small
// batches still spread over the compute units (the columns of S' and o are
// independent, so tiles need no combining). A row of the tile is covered by
// tile/4 consecutive threads and each thread keeps UNROLL rows of loads in
// flight. The output o = q S' is accumulated per thread over its rows and
// reduced across row groups in LDS.

#include "common.hpp"
#include "kernels.hpp"

namespace ret {

typedef float f32v4 __attribute__((ext_vector_type(4)));

// 512 threads and 16 rows in flight per thread: a sweep of workgroup size
// (128..1024) and unroll (4..32) on 64 x 16 heads of 256 x 512 put the
// optimum here (1024 workgroups, 8 waves each).
constexpr int kStepThreads = 512;
constexpr int kStepUnroll = 16;
constexpr int kStepMaxDk = 4096;

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
    if (BF16) return bf16_to_f32(static_cast<const u16*>(p)[i]);
    return static_cast<const float*>(p)[i];
}

// Sum of v over the workgroup (every thread gets it); `scratch` holds one float
// per wave and is free again when the function returns.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();  // earlier readers of scratch are done
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kStepThreads / 64; ++w) t += scratch[w];
    return t;
}

// GroupNorm of one head's bf16 output row, held by threads 0 .. tpr-1 (four
// channels each, tpr = dv / 4), then the gain, bias and gate: the multi-scale
// output stage's first half for a workgroup that owns the whole row.
__device__ __forceinline__ void step_groupnorm_gate(const StepArgs& a, const f32v4& o, int b, int h, int tpr,
                                                    float* scratch) {
    const bool mine = static_cast<int>(threadIdx.x) < tpr;
    const float inv = 1.0f / a.dv;
    const float mean = block_sum(mine ? (o[0] + o[1]) + (o[2] + o[3]) : 0.f, scratch) * inv;
    const f32v4 d = o - mean;
    const float var = block_sum(mine ? (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]) : 0.f, scratch) * inv;
    const float rstd = rsqrtf(var + a.eps);
    if (!mine) return;
    const int c = h * a.dv + 4 * static_cast<int>(threadIdx.x);  // channel in the layer's H*dv
    const size_t zi = static_cast<size_t>(b) * a.H * a.dv + c;
    f32v4 w = {1.f, 1.f, 1.f, 1.f}, bias = {0.f, 0.f, 0.f, 0.f}, g = {1.f, 1.f, 1.f, 1.f};
    if (a.gn_w) w = *reinterpret_cast<const f32v4*>(a.gn_w + c);
    if (a.gn_b) bias = *reinterpret_cast<const f32v4*>(a.gn_b + c);
    if (a.gate) {
        const uint2 gw = *reinterpret_cast<const uint2*>(a.gate + zi);
        g = f32v4{lo_bf16(gw.x), hi_bf16(gw.x), lo_bf16(gw.y), hi_bf16(gw.y)};
    }
    const f32v4 z = (d * rstd * w + bias) * g;
    *reinterpret_cast<uint2*>(a.z + zi) = make_uint2(pack2_bf16(z[0], z[1]), pack2_bf16(z[2], z[3]));
}

template <bool BF16, int UNROLL>
__global__ __launch_bounds__(kStepThreads) void recurrent_step_kernel(StepArgs a, HeadParams hp) {
    __shared__ float qs[kStepMaxDk];
    __shared__ float ks[kStepMaxDk];
    __shared__ f32v4 red[kStepThreads];

    const int bh = blockIdx.x / a.ntile;
    const int c0 = (blockIdx.x % a.ntile) * (a.dv / a.ntile);  // first column of this tile
    const int b = bh / a.H;
    const int h = bh % a.H;
    const int tid = threadIdx.x;
    const float gam = hp.gamma[h];

    // ---- q, k of this (sequence, head) in float32, rotated when asked
    const size_t qk0 = static_cast<size_t>(bh) * a.dk;
    if (hp.has_theta) {
        const double position = static_cast<double>(a.pos[b]);
        for (int j = tid; j < a.dk / 2; j += kStepThreads) {
            float c, s;
            rot_cs(position, hp.theta[j], c, s);
            const float qr = load_elem<BF16>(a.q, qk0 + 2 * j), qi = load_elem<BF16>(a.q, qk0 + 2 * j + 1);
            const float kr = load_elem<BF16>(a.k, qk0 + 2 * j), ki = load_elem<BF16>(a.k, qk0 + 2 * j + 1);
            qs[2 * j] = qr * c - qi * s;
            qs[2 * j + 1] = qr * s + qi * c;
            ks[2 * j] = kr * c - ki * s;
            ks[2 * j + 1] = kr * s + ki * c;
        }
    } else {
        for (int j = tid; j < a.dk; j += kStepThreads) {
            qs[j] = load_elem<BF16>(a.q, qk0 + j);
            ks[j] = load_elem<BF16>(a.k, qk0 + j);
        }
    }
    __syncthreads();

    // ---- stream the tile: thread (rg, c4) owns columns c0+4*c4..+3 of rows rg, rg+RG, ...
    const int tpr = a.dv / a.ntile / 4;
    const int rgs = kStepThreads / tpr;
    const int rg = tid / tpr;
    const int c4 = tid % tpr;
    f32v4 acc = {0.f, 0.f, 0.f, 0.f};
    if (rg < rgs) {
        const size_t v0 = static_cast<size_t>(bh) * a.dv + c0 + 4 * c4;
        const f32v4 vv = {load_elem<BF16>(a.v, v0), load_elem<BF16>(a.v, v0 + 1), load_elem<BF16>(a.v, v0 + 2),
                          load_elem<BF16>(a.v, v0 + 3)};
        f32v4* S = reinterpret_cast<f32v4*>(a.state + static_cast<size_t>(bh) * a.dk * a.dv + c0) + c4;
        const size_t row_stride = static_cast<size_t>(a.dv / 4);
        int i = rg;
        for (; i + (UNROLL - 1) * rgs < a.dk; i += UNROLL * rgs) {
            f32v4 s[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) s[u] = __builtin_nontemporal_load(S + (i + u * rgs) * row_stride);
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int row = i + u * rgs;
                const float kk = ks[row], qq = qs[row];
                s[u] = gam * s[u] + kk * vv;
                acc += qq * s[u];
                __builtin_nontemporal_store(s[u], S + row * row_stride);
            }
        }
        for (; i < a.dk; i += rgs) {
            f32v4 s = __builtin_nontemporal_load(S + i * row_stride);
            s = gam * s + ks[i] * vv;
            acc += qs[i] * s;
            __builtin_nontemporal_store(s, S + i * row_stride);
        }
    }
    red[tid] = acc;
    __syncthreads();

    // ---- reduce over row groups and write o
    f32v4 o = {0.f, 0.f, 0.f, 0.f};
    if (tid < tpr) {
        o = red[tid];
        for (int g = 1; g < rgs; ++g) o += red[g * tpr + tid];
        const size_t o0 = static_cast<size_t>(bh) * a.dv + c0 + 4 * tid;
        if (BF16) {
            u16* op = static_cast<u16*>(a.o) + o0;
            const uint2 w = make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3]));
            *reinterpret_cast<uint2*>(op) = w;
            o = f32v4{lo_bf16(w.x), hi_bf16(w.x), lo_bf16(w.y), hi_bf16(w.y)};  // what a reader of o sees
        } else {
            *reinterpret_cast<f32v4*>(static_cast<float*>(a.o) + o0) = o;
        }
    }
    if constexpr (BF16) {
        if (a.z) step_groupnorm_gate(a, o, b, h, tpr, reinterpret_cast<float*>(red));
    }
}

// Column tiles per (sequence, head): halve the tile while there are fewer
// than 256 workgroups and the halves keep at least 64 columns. (A sweep of
// the target over 256..2048 and of 32-column tiles at 16 heads of 256 x 512
// put it here: 8 sequences, 23.4 us against 27.8 with a target of 512; other
// batch sizes within 2%.)
int recurrent_step_tiles(int B, int H, int dv) {
    int nt = 1;
    while (static_cast<long long>(B) * H * nt < 256 && (dv / nt) % 128 == 0) nt *= 2;
    return nt;
}

hipError_t launch_recurrent_step(const StepArgs& a, const HeadParams& hp, hipStream_t st) {
    if (a.dk > kStepMaxDk || a.dv % 4 != 0 || a.ntile < 1 || a.dv % (4 * a.ntile) != 0 ||
        a.dv / a.ntile / 4 > kStepThreads || (a.z && (a.ntile != 1 || !a.bf16)))
        return hipErrorInvalidValue;
    dim3 grid(a.B * a.H * a.ntile), block(kStepThreads);
    // narrow tiles have more row groups per workgroup and so fewer rows per thread
    const bool narrow = a.ntile > 1;
    if (a.bf16) {
        if (narrow)
            recurrent_step_kernel<true, kStepUnroll / 2><<<grid, block, 0, st>>>(a, hp);
        else
            recurrent_step_kernel<true, kStepUnroll><<<grid, block, 0, st>>>(a, hp);
    } else {
        if (narrow)
            recurrent_step_kernel<false, kStepUnroll / 2><<<grid, block, 0, st>>>(a, hp);
        else
            recurrent_step_kernel<false, kStepUnroll><<<grid, block, 0, st>>>(a, hp);
    }
    return hipGetLastError();
}

}  // namespace ret
