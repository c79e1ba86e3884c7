// Retention forward (chunkwise and parallel forms) on float32 inputs.
//
// float32 inputs ask for float32 results throughout (a 1e-5 relative L2 bar),
// so these kernels use plain float32 FMA on the vector ALUs rather than bf16
// matrix cores. Each workgroup stages one chunk (or key block) of Q, K and a
// value tile in LDS and evaluates the definitions directly:
//   chunkwise ("RetNet Guide", section "3. The Chunkwise Recurrent
//   Representation", carry with in-chunk key decay xi_j = gamma^(L-1-j)):
//     O = ((Q K^T) (.) D) V + zeta (.) (Q S);  S <- gamma^L S + K^T (xi (.) V)
//   parallel ("RetNet Guide", section "1. The Parallel Representation"):
//     O = ((Q K^T) (.) D) V, walked over key blocks.

#include "common.hpp"
#include "kernels.hpp"

namespace ret {

constexpr int kF32Threads = 256;

__device__ __forceinline__ void rotate_row_f32(float* row, int dk, const HeadParams& hp, double position) {
    for (int j = 0; j < dk / 2; ++j) {
        float c, s;
        rot_cs(position, hp.theta[j], c, s);
        const float re = row[2 * j], im = row[2 * j + 1];
        row[2 * j] = re * c - im * s;
        row[2 * j + 1] = re * s + im * c;
    }
}

// Stage rows [t0, t0 + L) of a [*, ld] float matrix (columns c0 .. c0 + w) into
// LDS as [C][pitch], zero-filling rows >= L; optionally rotate each row. Key
// rows use pitch w + 1 so that lanes reading one column of consecutive rows
// hit different banks.
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int ld, int c0, int w, int pitch, int t0,
                                           int L, int C, bool rotate, const HeadParams& hp, long long pos0) {
    const int tid = threadIdx.x;
    for (int idx = tid; idx < C * w; idx += kF32Threads) {
        const int r = idx / w, c = idx % w;
        dst[r * pitch + c] = r < L ? src[static_cast<size_t>(t0 + r) * ld + c0 + c] : 0.0f;
    }
    if (rotate) {
        __syncthreads();
        for (int r = tid; r < L; r += kF32Threads)
            rotate_row_f32(dst + r * pitch, w, hp, static_cast<double>(pos0 + t0 + r));
    }
}

template <bool STATE_ONLY>
__global__ __launch_bounds__(kF32Threads) void chunk_f32_kernel(ChunkArgs a, HeadParams hp, int dvt) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int C = a.chunk, DK = a.dk;
    const int KP = DK + 1;            // padded key row pitch
    float* sq = smem;                 // [C][DK]
    float* sk = sq + C * DK;          // [C][KP]
    float* sv = sk + C * KP;          // [C][dvt]
    float* ss = sv + C * dvt;         // [DK][dvt]
    float* sp = ss + DK * dvt;        // [C][C]
    float* sx = sp + C * C;           // [C] key decay xi_j of the current chunk

    const int tid = threadIdx.x;
    const int nseg_grid = STATE_ONLY ? a.nseg - 1 : a.nseg;
    const int lb = blockIdx.x;
    const int vt = lb % a.nvt;
    const int seg = (lb / a.nvt) % nseg_grid;
    const int bh = lb / (a.nvt * nseg_grid);
    const int h = bh % a.H;
    const double lg2 = log2_gamma(hp.gamma[h]);
    const float lg2f = static_cast<float>(lg2);

    const int t_begin = seg * a.seg_len;
    const int t_end = min(a.N, t_begin + a.seg_len);
    const size_t tok0 = static_cast<size_t>(bh) * a.N;
    const float* Q = reinterpret_cast<const float*>(a.q) + tok0 * DK;
    const float* K = reinterpret_cast<const float*>(a.k) + tok0 * DK;
    const float* V = reinterpret_cast<const float*>(a.v) + tok0 * a.dv;
    float* O = reinterpret_cast<float*>(a.o) + tok0 * a.dv;
    const int c0 = vt * dvt;

    const float* s_src = nullptr;
    if (!STATE_ONLY) {
        if (a.nseg > 1)
            s_src = a.agg + (static_cast<size_t>(bh) * a.nseg + seg) * DK * a.dv;
        else if (a.state_in)
            s_src = a.state_in + static_cast<size_t>(bh) * DK * a.dv;
    }
    for (int idx = tid; idx < DK * dvt; idx += kF32Threads) {
        const int d = idx / dvt, c = idx % dvt;
        ss[idx] = s_src ? s_src[static_cast<size_t>(d) * a.dv + c0 + c] : 0.0f;
    }
    bool have_state = s_src != nullptr;

    for (int t0 = t_begin; t0 < t_end; t0 += C) {
        const int L = min(C, t_end - t0);
        __syncthreads();
        if (!STATE_ONLY) stage_rows(sq, Q, DK, 0, DK, DK, t0, L, C, hp.has_theta, hp, a.pos0);
        stage_rows(sk, K, DK, 0, DK, KP, t0, L, C, hp.has_theta, hp, a.pos0);
        stage_rows(sv, V, a.dv, c0, dvt, dvt, t0, L, C, false, hp, a.pos0);
        for (int j = tid; j < L; j += kF32Threads) sx[j] = exp2f(static_cast<float>(L - 1 - j) * lg2f);
        __syncthreads();
        if (!STATE_ONLY) {
            // scores with decay mask (select, so a non-finite future key never leaks)
            for (int idx = tid; idx < L * L; idx += kF32Threads) {
                const int i = idx / L, j = idx % L;
                float p = 0.0f;
                if (j <= i) {
                    float acc = 0.0f;
                    for (int d = 0; d < DK; ++d) acc = fmaf(sq[i * DK + d], sk[j * KP + d], acc);
                    p = acc * exp2f(static_cast<float>(i - j) * lg2f);
                }
                sp[i * C + j] = p;
            }
            __syncthreads();
            for (int idx = tid; idx < L * dvt; idx += kF32Threads) {
                const int i = idx / dvt, c = idx % dvt;
                float inner = 0.0f;
                for (int j = 0; j <= i; ++j) inner = fmaf(sp[i * C + j], sv[j * dvt + c], inner);
                float cross = 0.0f;
                if (have_state) {
                    for (int d = 0; d < DK; ++d) cross = fmaf(sq[i * DK + d], ss[d * dvt + c], cross);
                    cross *= gamma_pow(lg2, i + 1.0);
                }
                O[static_cast<size_t>(t0 + i) * a.dv + c0 + c] = inner + cross;
            }
            __syncthreads();
        }
        const float gL = gamma_pow(lg2, L);
        for (int idx = tid; idx < DK * dvt; idx += kF32Threads) {
            const int d = idx / dvt, c = idx % dvt;
            float acc = 0.0f;
            for (int j = 0; j < L; ++j) acc = fmaf(sk[j * KP + d] * sx[j], sv[j * dvt + c], acc);
            ss[idx] = gL * ss[idx] + acc;
        }
        have_state = true;
    }
    __syncthreads();

    float* s_dst = nullptr;
    if (STATE_ONLY)
        s_dst = a.agg + (static_cast<size_t>(bh) * a.nseg + seg + 1) * DK * a.dv;
    else if (seg == a.nseg - 1 && a.state_out)
        s_dst = a.state_out + static_cast<size_t>(bh) * DK * a.dv;
    if (s_dst) {
        for (int idx = tid; idx < DK * dvt; idx += kF32Threads) {
            const int d = idx / dvt, c = idx % dvt;
            s_dst[static_cast<size_t>(d) * a.dv + c0 + c] = ss[idx];
        }
    }
}

size_t chunk_f32_lds_bytes(int C, int dk, int dvt) {
    return sizeof(float) * (static_cast<size_t>(C) * dk + static_cast<size_t>(C) * (dk + 1) +
                            static_cast<size_t>(C) * dvt + static_cast<size_t>(dk) * dvt +
                            static_cast<size_t>(C) * C + C);
}

hipError_t launch_chunk_f32(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev) {
    const size_t lds = chunk_f32_lds_bytes(a.chunk, a.dk, dvt);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_f32_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_f32_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int bhv = a.B * a.H * a.nvt;
    if (a.nseg > 1) {
        launch_timed(chunk_f32_kernel<true>, dim3(bhv * (a.nseg - 1)), dim3(kF32Threads), lds, st, ev, a, hp, dvt);
        e = launch_segment_scan(a, hp, st, ev ? ev + 2 : nullptr);
        if (e != hipSuccess) return e;
    } else {
        record_empty_phase(st, ev);
        record_empty_phase(st, ev ? ev + 2 : nullptr);
    }
    launch_timed(chunk_f32_kernel<false>, dim3(bhv * a.nseg), dim3(kF32Threads), lds, st, ev ? ev + 4 : nullptr, a,
                 hp, dvt);
    return hipGetLastError();
}

// ---------------------------------------------------------------- parallel form

constexpr int kParF32Block = 64;

__global__ __launch_bounds__(kF32Threads) void parallel_f32_kernel(ParallelArgs a, HeadParams hp, int dvt) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int BQ = kParF32Block, DK = a.dk;
    const int KP = DK + 1;       // padded key row pitch
    float* sq = smem;            // [BQ][DK]
    float* sk = sq + BQ * DK;    // [BQ][KP]
    float* sv = sk + BQ * KP;    // [BQ][dvt]
    float* sp = sv + BQ * dvt;   // [BQ][BQ]

    const int tid = threadIdx.x;
    const int nqb = (a.N + BQ - 1) / BQ;
    const int BH = a.B * a.H;
    const int lb = blockIdx.x;
    const int vt = lb % a.nvt;
    const int bh = (lb / a.nvt) % BH;
    const int qb = nqb - 1 - lb / (a.nvt * BH);
    const int h = bh % a.H;
    const double lg2 = log2_gamma(hp.gamma[h]);
    const float lg2f = static_cast<float>(lg2);

    const size_t tok0 = static_cast<size_t>(bh) * a.N;
    const float* Q = reinterpret_cast<const float*>(a.q) + tok0 * DK;
    const float* K = reinterpret_cast<const float*>(a.k) + tok0 * DK;
    const float* V = reinterpret_cast<const float*>(a.v) + tok0 * a.dv;
    float* O = reinterpret_cast<float*>(a.o) + tok0 * a.dv;
    const int c0 = vt * dvt;
    const int q0 = qb * BQ;
    const int Lq = min(BQ, a.N - q0);

    constexpr int kMaxOut = BQ * 64 / kF32Threads;  // outputs per thread (dvt <= 64)
    float out[kMaxOut];
#pragma unroll
    for (int u = 0; u < kMaxOut; ++u) out[u] = 0.0f;

    stage_rows(sq, Q, DK, 0, DK, DK, q0, Lq, BQ, hp.has_theta, hp, a.pos0);
    for (int kb = qb; kb >= 0; --kb) {
        const int k0 = kb * BQ;
        const int Lk = min(BQ, a.N - k0);
        // every D entry of this block (and all earlier ones) below float32 underflow
        if (lg2 < 0.0 && (static_cast<double>(q0 - k0) - (BQ - 1)) * (-lg2) > 160.0) break;
        __syncthreads();
        stage_rows(sk, K, DK, 0, DK, KP, k0, Lk, BQ, hp.has_theta, hp, a.pos0);
        stage_rows(sv, V, a.dv, c0, dvt, dvt, k0, Lk, BQ, false, hp, a.pos0);
        __syncthreads();
        // one exponent per entry, (q0 + i) - (k0 + j) >= 0 for every kept entry,
        // so no factor overflows for small gamma
        for (int idx = tid; idx < BQ * BQ; idx += kF32Threads) {
            const int i = idx / BQ, j = idx % BQ;
            float p = 0.0f;
            if (i < Lq && j < Lk && (kb < qb || j <= i)) {
                float acc = 0.0f;
                for (int d = 0; d < DK; ++d) acc = fmaf(sq[i * DK + d], sk[j * KP + d], acc);
                p = acc * exp2f(static_cast<float>((q0 - k0) + i - j) * lg2f);
            }
            sp[idx] = p;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kMaxOut; ++u) {
            const int idx = tid + u * kF32Threads;
            if (idx < BQ * dvt) {
                const int i = idx / dvt, c = idx % dvt;
                float acc = out[u];
                for (int j = 0; j < Lk; ++j) acc = fmaf(sp[i * BQ + j], sv[j * dvt + c], acc);
                out[u] = acc;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxOut; ++u) {
        const int idx = tid + u * kF32Threads;
        if (idx < BQ * dvt) {
            const int i = idx / dvt, c = idx % dvt;
            if (i < Lq) O[static_cast<size_t>(q0 + i) * a.dv + c0 + c] = out[u];
        }
    }
}

size_t parallel_f32_lds_bytes(int dk, int dvt) {
    const size_t BQ = kParF32Block;
    return sizeof(float) * (BQ * dk + BQ * (dk + 1) + BQ * dvt + BQ * BQ);
}

hipError_t launch_parallel_f32(const ParallelArgs& a, const HeadParams& hp, int dvt, hipStream_t st) {
    const size_t lds = parallel_f32_lds_bytes(a.dk, dvt);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&parallel_f32_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const int nqb = (a.N + kParF32Block - 1) / kParF32Block;
    parallel_f32_kernel<<<dim3(nqb * a.B * a.H * a.nvt), dim3(kF32Threads), lds, st>>>(a, hp, dvt);
    return hipGetLastError();
}

}  // namespace ret
