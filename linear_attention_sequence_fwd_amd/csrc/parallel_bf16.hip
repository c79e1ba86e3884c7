// Parallel retention form O = ((Q K^T) (.) D) V on bf16 inputs, float32
// accumulation, for gfx950 matrix cores.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "1. The
// Parallel Representation for High-Throughput Pretraining":
// D[n][m] = gamma^(n-m) for n >= m and 0 otherwise.
//
// The N x N score matrix is never formed in memory. One workgroup owns one
// block of BQ query rows (one head, one value tile) and walks the key blocks
// from its own (diagonal) block backwards. For each key block it forms
// P^T = K Q^T on v_mfma_f32_16x16x32_bf16, multiplies by D generated in
// registers (a per-lane factor times a per-block factor), and accumulates
// O^T += V^T P^T. There is no softmax, so nothing is rescaled between blocks.
// Once a key block lies so far back that every entry of D underflows float32,
// it and all earlier blocks contribute exactly zero in float32 and the walk
// stops. Query blocks are dispatched longest-first.

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace ret {

template <int DK, int DVT, int BQ>
struct ParGeo {
    static constexpr int NW = BQ / 32;
    static constexpr int NTHR = NW * 64;
    static constexpr int NRB = BQ / 16;
    static constexpr int KSQ = DK / 32;
    static constexpr int KST = BQ / 32;
    static constexpr int NTV = DVT / 16;
    static constexpr int KB = (BQ / 8) * (DK / 8);
    static constexpr int VB = (BQ / 8) * (DVT / 8);
    static constexpr int KPT = (KB + NTHR - 1) / NTHR;
    static constexpr int VPT = (VB + NTHR - 1) / NTHR;
};

template <int DK, int DVT, int BQ>
__global__ __launch_bounds__((BQ / 32) * 64) void parallel_bf16_kernel(ParallelArgs a, HeadParams hp) {
    using G = ParGeo<DK, DVT, BQ>;
    __shared__ __attribute__((aligned(16))) u16 kbuf[BQ * DK];
    __shared__ __attribute__((aligned(16))) u16 vbuf[DVT * BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int grp = lane >> 4;

    const int nqb = (a.N + BQ - 1) / BQ;
    const int BH = a.B * a.H;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int vt = lb % a.nvt;
    const int bh = (lb / a.nvt) % BH;
    const int qb = nqb - 1 - lb / (a.nvt * BH);
    const int h = bh % a.H;

    const float gam = hp.gamma[h];
    const double lg2 = log2_gamma(gam);
    const float lg2f = static_cast<float>(lg2);

    const size_t tok0 = static_cast<size_t>(bh) * a.N;
    const u16* Kg = a.k + tok0 * DK;
    const u16* Qg = a.q + tok0 * DK;
    const u16* Vg = a.v + tok0 * a.dv + vt * DVT;
    u16* Og = a.o + tok0 * a.dv + vt * DVT;

    const int rbs[2] = {wave, G::NRB - 1 - wave};
    const int q0 = qb * BQ;
    const int Lq = min(BQ, a.N - q0);

    // D = gamma^((q0 + 16 rb + l16) - (k0 + 16 jt + 4 grp + r))
    //   = dlane[r] * gamma^(16 (rb - jt)) * gamma^(q0 - k0), the last factor in float64
    float dlane[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dlane[r] = exp2f(static_cast<float>(l16 - 4 * grp - r) * lg2f);

    // queries of this block, rotated, in MFMA operand registers
    uint4 qf[2][G::KSQ];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = rbs[i] * 16 + l16;
#pragma unroll
        for (int s = 0; s < G::KSQ; ++s) {
            uint4 x = row < Lq ? *reinterpret_cast<const uint4*>(Qg + static_cast<size_t>(q0 + row) * DK + s * 32 + grp * 8)
                               : make_uint4(0, 0, 0, 0);
            if (hp.has_theta && row < Lq)
                x = rotate8_bf16(x, hp, s * 16 + grp * 4, static_cast<double>(a.pos0 + q0 + row));
            qf[i][s] = x;
        }
    }

    f32x4 oacc[2][G::NTV];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int nt = 0; nt < G::NTV; ++nt) oacc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // number of key blocks with any entry of D above float32 underflow:
    // block qb - m has its largest decay gamma^(m BQ - BQ + 1)
    int nkb = qb + 1;
    if (lg2 < 0.0) {
        const double span = 160.0 / (-lg2);  // gamma^span < 2^-160
        const int mmax = static_cast<int>((span + BQ - 1) / BQ) + 1;
        nkb = min(nkb, mmax + 1);
    }

    uint4 kr[G::KPT][8];
    uint4 vr[G::VPT][8];
    load_blocks<DK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(q0) * DK, DK, Lq, tid);
    load_blocks<DVT, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(q0) * a.dv, a.dv, Lq, tid);

    for (int m = 0; m < nkb; ++m) {
        // Per-iteration copies the compiler cannot prove loop-invariant (see the
        // chunkwise kernel): addresses and decay factors are recomputed per block.
        int lane_it = lane;
        float lg2_it = lg2f;
        asm volatile("" : "+v"(lane_it), "+v"(lg2_it));
        const int l16 = lane_it & 15;
        const int grp = lane_it >> 4;
        const float lg2f = lg2_it;
        const int kb = qb - m;
        const int k0 = kb * BQ;
        const int Lk = min(BQ, a.N - k0);
        const bool diag = (m == 0);

        // keys row-major and V^T into LDS
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK>(idx, tb, cb);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    uint4 x = kr[u][q];
                    if (hp.has_theta && tb * 8 + q < Lk)
                        x = rotate8_bf16(x, hp, cb * 4, static_cast<double>(a.pos0 + k0 + tb * 8 + q));
                    *reinterpret_cast<uint4*>(&kbuf[kidx_rm<DK>(tb * 8 + q, cb * 8)]) = x;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G::VPT; ++u) {
            const int idx = tid + u * G::NTHR;
            if (idx < G::VB) {
                int tb, cb;
                block_coords<DVT>(idx, tb, cb);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) w[p] = elem16(vr[u][2 * p], c) | (elem16(vr[u][2 * p + 1], c) << 16);
                    *reinterpret_cast<uint4*>(&vbuf[tidx<BQ>(cb * 8 + c, tb * 8)]) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
        __syncthreads();

        if (m + 1 < nkb) {
            const int kn = (kb - 1) * BQ;
            load_blocks<DK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(kn) * DK, DK, BQ, tid);
            load_blocks<DVT, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(kn) * a.dv, a.dv, BQ, tid);
        }

        const float blkf = gamma_pow(lg2, static_cast<double>(q0 - k0));
        f32x4 pacc[2][G::NRB];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jt = 0; jt < G::NRB; ++jt) pacc[i][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jt = 0; jt < G::NRB; ++jt) {
            if ((!diag || jt <= rbs[1]) && jt * 16 < Lk) {
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s) {
                    const uint4 af = *reinterpret_cast<const uint4*>(&kbuf[kidx_rm<DK>(jt * 16 + l16, s * 32 + grp * 8)]);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (!diag || jt <= rbs[i]) pacc[i][jt] = mfma16x16x32(af, qf[i][s], pacc[i][jt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        uint4 pf[2][G::KST];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int jt = 0; jt < G::NRB; ++jt) {
                const int delta = rbs[i] - jt;
                const float blk = exp2f(static_cast<float>(16 * delta) * lg2f) * blkf;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float val = 0.0f;
                    const bool keep = !diag || delta > 0 || (delta == 0 && l16 >= 4 * grp + r);
                    if (keep) val = pacc[i][jt][r] * (dlane[r] * blk);
                    pacc[i][jt][r] = val;
                }
            }
#pragma unroll
            for (int t = 0; t < G::KST; ++t)
                pf[i][t] = make_uint4(pack2_bf16(pacc[i][2 * t][0], pacc[i][2 * t][1]),
                                      pack2_bf16(pacc[i][2 * t][2], pacc[i][2 * t][3]),
                                      pack2_bf16(pacc[i][2 * t + 1][0], pacc[i][2 * t + 1][1]),
                                      pack2_bf16(pacc[i][2 * t + 1][2], pacc[i][2 * t + 1][3]));
        }
#pragma unroll
        for (int t = 0; t < G::KST; ++t) {
            if ((!diag || 2 * t <= rbs[1]) && t * 32 < Lk) {
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
                    const int row = nt * 16 + l16;
                    const uint2 lo = *reinterpret_cast<const uint2*>(&vbuf[tidx<BQ>(row, t * 32 + grp * 4)]);
                    const uint2 hi = *reinterpret_cast<const uint2*>(&vbuf[tidx<BQ>(row, t * 32 + 16 + grp * 4)]);
                    const uint4 af = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (!diag || 2 * t <= rbs[i]) oacc[i][nt] = mfma16x16x32(af, pf[i][t], oacc[i][nt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = rbs[i] * 16 + l16;
        if (row < Lq) {
            u16* orow = Og + static_cast<size_t>(q0 + row) * a.dv;
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
                *reinterpret_cast<uint2*>(orow + nt * 16 + grp * 4) =
                    make_uint2(pack2_bf16(oacc[i][nt][0], oacc[i][nt][1]), pack2_bf16(oacc[i][nt][2], oacc[i][nt][3]));
        }
    }
}

template <int DK, int DVT, int BQ>
static hipError_t run_parallel_bf16(const ParallelArgs& a, const HeadParams& hp, hipStream_t st) {
    using G = ParGeo<DK, DVT, BQ>;
    const int nqb = (a.N + BQ - 1) / BQ;
    parallel_bf16_kernel<DK, DVT, BQ><<<dim3(nqb * a.B * a.H * a.nvt), dim3(G::NTHR), 0, st>>>(a, hp);
    return hipGetLastError();
}

hipError_t launch_parallel_bf16(const ParallelArgs& a, const HeadParams& hp, int dvt, hipStream_t st) {
    if (a.dk == 64 && dvt == 64) return run_parallel_bf16<64, 64, 64>(a, hp, st);
    if (a.dk == 64 && dvt == 128) return run_parallel_bf16<64, 128, 128>(a, hp, st);
    if (a.dk == 128 && dvt == 64) return run_parallel_bf16<128, 64, 128>(a, hp, st);
    if (a.dk == 128 && dvt == 128) return run_parallel_bf16<128, 128, 128>(a, hp, st);
    if (a.dk == 256 && dvt == 64) return run_parallel_bf16<256, 64, 128>(a, hp, st);
    if (a.dk == 256 && dvt == 128) return run_parallel_bf16<256, 128, 128>(a, hp, st);
    return hipErrorInvalidValue;
}

}  // namespace ret
