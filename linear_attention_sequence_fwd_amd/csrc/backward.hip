// Element-wise kernels of the chunkwise backward.
//
// Training runs retention in its parallel form over the whole sequence ("RetNet
// Guide: Retentive Networks & The Impossible Triangle", section "1. The
// Parallel Representation for High-Throughput Pretraining"), so the gradient of
// a call is that of O = ((Q' K'^T) (.) D) V + zeta (.) (Q' S0) and of the final
// state S_N = gamma^N S0 + K'^T (xi (.) V). Each gradient is itself a
// retention, which is how the backward reaches the matrix cores: with F(a, b, c;
// X) the chunkwise forward with queries a, keys b, values c and initial state X,
// and rev() the reversal of the token order,
//     dQ' = F(dO, V, K'; S0^T)
//     dK' = rev F(rev V, rev dO, rev Q'; dS^T / gamma)
//     dV  = rev F(rev K', rev Q', rev dO; dS / gamma)
// (the transposed decay matrix is the causal one of the reversed sequence, and
// the 1/gamma turns the reversed pass's initial-state weight gamma^(i+1) into
// the weight gamma^(N-1-m) with which key m enters S_N); the last pass's final
// state times gamma is dS0. The rotation is orthogonal per pair, so dQ and dK
// are dQ', dK' rotated by the opposite angle.
//
// For bf16 the matrix-core kernel runs the reversed passes in reverse token
// order itself; float32 passes run on reversed copies. When dv is wider than
// the kernel's key width (the first two passes use V and dO as keys), those
// passes run as two passes over the halves of dv, whose outputs add up: the
// scores q k^T and the carried state q S are sums over key columns. The
// kernels here are the HBM-bound glue around the passes: rows_kernel rotates,
// reverses, slices or adds rows (up to six tensors per launch, one per grid
// row; one more row can zero-fill the control words of the passes' workspace
// regions), state_kernel transposes, splits and scales the [dk, dv] states.

#include "common.hpp"
#include "kernels.hpp"

namespace ret {

namespace {

constexpr int kRowThreads = 256;
constexpr int kStateThreads = 256;

// cos/sin of position * theta for a pair that is rounded to bf16 next (hardware
// sin/cos on a float64-reduced angle) or kept in float32 (float32 sin/cos on a
// float64-reduced angle).
template <bool BF16>
__device__ __forceinline__ void pair_cs(double position, float theta, float& c, float& s) {
    if (BF16)
        rot_cs_fast(position, theta, c, s);
    else
        rot_cs(position, theta, c, s);
}

// Eight consecutive elements of a row in float32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t i, float* x) {
    if (BF16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const u16*>(base) + i);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            x[2 * p] = lo_bf16(ws[p]);
            x[2 * p + 1] = hi_bf16(ws[p]);
        }
    } else {
        const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
        const float4 a = f[0], b = f[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, size_t i, const float* x) {
    if (BF16) {
        const uint4 w = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]), pack2_bf16(x[4], x[5]),
                                   pack2_bf16(x[6], x[7]));
        *reinterpret_cast<uint4*>(static_cast<u16*>(base) + i) = w;
    } else {
        float4* f = reinterpret_cast<float4*>(static_cast<float*>(base) + i);
        f[0] = make_float4(x[0], x[1], x[2], x[3]);
        f[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
}

// One thread moves 8 elements of one row of the tensor selected by blockIdx.y.
// Row t of every (batch, head) is read from src (columns src_col .. of rows of
// src_ld elements; plus the same row of `add` when given), rotated by sign * theta at
// the position of the token it holds when the job asks (pos0 + t, or
// pos0 + N-1-t when src is in reverse order), and written to row t' of dst0
// (t' = N-1-t when flip0, else t) and to row t of dst1 when dst1 is given. A job
// whose src is dst0 without flip is an in-place update: every thread reads
// and writes only its own 8 elements.
template <bool BF16>
__global__ __launch_bounds__(kRowThreads) void rows_kernel(RowJobs jobs, HeadParams hp) {
    if (static_cast<int>(blockIdx.y) == jobs.n) {  // the zero-fill row
        const long long stride = static_cast<long long>(gridDim.x) * kRowThreads;
        for (int r = 0; r < kMaxZeroRegions; ++r) {
            if (!jobs.zero[r]) continue;
            for (long long e = static_cast<long long>(blockIdx.x) * kRowThreads + threadIdx.x; e < jobs.nzero;
                 e += stride)
                jobs.zero[r][e] = make_uint4(0u, 0u, 0u, 0u);
        }
        return;
    }
    const RowJob& jb = jobs.j[blockIdx.y];
    const int d = jb.d;
    const long long total8 = static_cast<long long>(jobs.B) * jobs.H * jobs.N * d / 8;
    const long long stride = static_cast<long long>(gridDim.x) * kRowThreads;
    for (long long e = static_cast<long long>(blockIdx.x) * kRowThreads + threadIdx.x; e < total8; e += stride) {
        const long long elem = e * 8;
        const long long row = elem / d;
        const int col = static_cast<int>(elem - row * d);
        const long long bh = row / jobs.N;
        const int t = static_cast<int>(row - bh * jobs.N);
        float x[8];
        const int ld = jb.src_ld ? jb.src_ld : d;
        load8<BF16>(jb.src, static_cast<size_t>(row * ld + jb.src_col + col), x);
        if (jb.add) {
            float y[8];
            load8<BF16>(jb.add, static_cast<size_t>(elem), y);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] += y[i];
        }
        if (jb.rot != 0) {
            const double position = static_cast<double>(jobs.pos0) + (jb.src_rev ? jobs.N - 1 - t : t);
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float c, s;
                pair_cs<BF16>(position, jb.rot * hp.theta[col / 2 + p], c, s);
                const float re = x[2 * p], im = x[2 * p + 1];
                x[2 * p] = re * c - im * s;
                x[2 * p + 1] = re * s + im * c;
            }
        }
        const long long t0 = jb.flip0 ? (jobs.N - 1 - t) : t;
        store8<BF16>(jb.dst0, static_cast<size_t>((bh * jobs.N + t0) * d + col), x);
        if (jb.dst1) store8<BF16>(jb.dst1, static_cast<size_t>(elem), x);
    }
}

// mode 0 (before the passes), per (batch, head) and element (i, j) of a
// [dk, dv] state:  x1[j][i] = s0[i][j];  x2[j][i] = ds[i][j] / gamma;
// x3[i][j] = ds[i][j] / gamma  (each only when its source is given).
// mode 1 (after them): dsi[i][j] *= gamma.
__global__ __launch_bounds__(kStateThreads) void state_kernel(StateJobs sj, HeadParams hp) {
    const long long per = static_cast<long long>(sj.dk) * sj.dv;
    const long long total = static_cast<long long>(sj.B) * sj.H * per;
    const long long stride = static_cast<long long>(gridDim.x) * kStateThreads;
    for (long long e = static_cast<long long>(blockIdx.x) * kStateThreads + threadIdx.x; e < total; e += stride) {
        const long long bh = e / per;
        const int ij = static_cast<int>(e - bh * per);
        const int i = ij / sj.dv, j = ij - (ij / sj.dv) * sj.dv;
        const float g = hp.gamma[bh % sj.H];
        // transposed position: row j of [dv, dk], in the first or second half array when split
        const int hv = sj.split ? sj.dv / 2 : sj.dv;
        const int half = j / hv, jj = j - half * hv;
        const long long tr = static_cast<long long>(half) * sj.B * sj.H * hv * sj.dk + bh * hv * sj.dk +
                             static_cast<long long>(jj) * sj.dk + i;
        if (sj.mode == 0) {
            if (sj.s0) sj.x1[tr] = sj.s0[e];
            if (sj.ds) {
                const float y = sj.ds[e] / g;
                sj.x2[tr] = y;
                sj.x3[e] = y;
            }
        } else {
            sj.dsi[e] *= g;
        }
    }
}

int grid_for(long long items, int threads) {
    long long blocks = (items + threads - 1) / threads;
    if (blocks > 4096) blocks = 4096;  // grid-stride beyond 16 workgroups per compute unit
    return static_cast<int>(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_rows(const RowJobs& jobs, const HeadParams& hp, bool bf16, hipStream_t st) {
    if (jobs.n < 0 || jobs.n > kMaxRowJobs || (jobs.n == 0 && jobs.nzero <= 0)) return hipErrorInvalidValue;
    int dmax = 0;
    for (int i = 0; i < jobs.n; ++i) dmax = jobs.j[i].d > dmax ? jobs.j[i].d : dmax;
    long long items = static_cast<long long>(jobs.B) * jobs.H * jobs.N * dmax / 8;
    if (jobs.nzero > items) items = jobs.nzero;
    const dim3 grid(grid_for(items, kRowThreads), jobs.n + (jobs.nzero > 0 ? 1 : 0));
    if (bf16)
        hipLaunchKernelGGL(rows_kernel<true>, grid, dim3(kRowThreads), 0, st, jobs, hp);
    else
        hipLaunchKernelGGL(rows_kernel<false>, grid, dim3(kRowThreads), 0, st, jobs, hp);
    return hipGetLastError();
}

hipError_t launch_states(const StateJobs& sj, const HeadParams& hp, hipStream_t st) {
    const long long items = static_cast<long long>(sj.B) * sj.H * sj.dk * sj.dv;
    hipLaunchKernelGGL(state_kernel, dim3(grid_for(items, kStateThreads)), dim3(kStateThreads), 0, st, sj, hp);
    return hipGetLastError();
}

}  // namespace ret
