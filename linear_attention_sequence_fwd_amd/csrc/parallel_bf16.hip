// Parallel retention form O = ((Q K^T) (.) D) V on bf16 inputs, float32
// accumulation, for gfx950 matrix cores.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "1. The
// Parallel Representation for High-Throughput Pretraining":
// D[n][m] = gamma^(n-m) for n >= m and 0 otherwise.
//
// The N x N score matrix is never formed in memory. One workgroup owns one
// block of BQ query rows (one head, one value tile; one 16-row block per wave)
// and walks the key blocks from its own (diagonal) block backwards. For each
// key block it forms
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
    static constexpr int NW = BQ / 16;  // waves: one 16-row block of the query block each
    static constexpr int NTHR = NW * 64;
    static constexpr int KSQ = DK / 32;
    static constexpr int KST = BQ / 32;
    static constexpr int NTV = DVT / 16;
    static constexpr int BWK = stage_width(BQ, DK, NTHR);
    static constexpr int BWV = stage_width(BQ, DVT, NTHR);
    static constexpr int KB = (BQ / 8) * (DK / BWK);
    static constexpr int VB = (BQ / 8) * (DVT / BWV);
    static constexpr int KPT = (KB + NTHR - 1) / NTHR;
    static constexpr int VPT = (VB + NTHR - 1) / NTHR;
};

template <int DK, int DVT, int BQ>
__global__ __launch_bounds__((BQ / 16) * 64) void parallel_bf16_kernel(ParallelArgs a, HeadParams hp) {
    using G = ParGeo<DK, DVT, BQ>;
    constexpr int UK = DK / 8;
    constexpr int UC = BQ / 8;
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

    // row block of this wave; the two waves sharing a SIMD get blocks b and NW-1-b
    const int rb = wave < G::NW / 2 ? wave : (3 * G::NW / 2 - 1) - wave;
    const int q0 = qb * BQ;
    const int Lq = min(BQ, a.N - q0);

    // D = gamma^((q0 + 16 rb + l16) - (k0 + 16 jt + 4 grp + r)). Every factor is
    // kept at an exponent >= 0 so that no factor overflows for small gamma:
    //   diagonal tile (q0 = k0, jt = rb):  dlane[r] = gamma^(l16 - 4 grp - r)
    //     (negative exponents only in masked entries, which are selected away);
    //   other tiles: dlane15[r] * gamma^(16 (rb - jt) + (q0 - k0) - 15), with
    //     dlane15[r] = gamma^(l16 - 4 grp - r + 15) and the tile exponent >= 1.
    float dlane[4], dlane15[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        dlane[r] = fast_exp2(static_cast<float>(l16 - 4 * grp - r) * lg2f);
        dlane15[r] = fast_exp2(static_cast<float>(l16 - 4 * grp - r + 15) * lg2f);
    }

    // queries of this wave's rows, rotated, in MFMA operand registers
    uint4 qf[G::KSQ];
    {
        const int row = rb * 16 + l16;
        const u16* p = Qg + static_cast<size_t>(q0 + row) * DK + grp * 8;
#pragma unroll
        for (int s = 0; s < G::KSQ; ++s) {
            uint4 x = row < Lq ? *reinterpret_cast<const uint4*>(p + s * 32) : make_uint4(0, 0, 0, 0);
            if (hp.has_theta && row < Lq)
                x = rotate8_bf16(x, hp, s * 16 + grp * 4, static_cast<double>(a.pos0 + q0 + row));
            qf[s] = x;
        }
    }

    f32x4 oacc[G::NTV];
#pragma unroll
    for (int nt = 0; nt < G::NTV; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // number of key blocks with any entry of D above float32 underflow:
    // block qb - m has its largest decay gamma^(m BQ - BQ + 1)
    int nkb = qb + 1;
    if (lg2 < 0.0) {
        const double span = 160.0 / (-lg2);  // gamma^span < 2^-160
        const int mmax = static_cast<int>((span + BQ - 1) / BQ) + 1;
        nkb = min(nkb, mmax + 1);
    }

    BlockRows<G::BWK> kr[G::KPT];
    BlockRows<G::BWV> vr[G::VPT];
    load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(q0) * DK, DK, Lq, tid);
    load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(q0) * a.dv, a.dv, Lq, tid);

    for (int m = 0; m < nkb; ++m) {
        // Per-iteration copies the compiler cannot prove loop-invariant: block
        // write addresses and decay factors are recomputed per key block rather
        // than held in registers across the loop.
        int tid_it = tid;
        float lg2_it = lg2f;
        asm volatile("" : "+v"(tid_it), "+v"(lg2_it));
        const float lg2c = lg2_it;
        const int l16c = tid_it & 15;
        const int grpc = (tid_it & 63) >> 4;
        const int kb = qb - m;
        const int k0 = kb * BQ;
        const int Lk = min(BQ, a.N - k0);
        const bool diag = (m == 0);

        // keys row-major (rotated) and V^T into LDS
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid_it + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK, G::BWK>(idx, tb, cb);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int row = staged_token(tb, q);
                    if (hp.has_theta && row < Lk)
                        rotate_row<G::BWK>(kr[u].w[q], hp, cb * (G::BWK / 2), static_cast<double>(a.pos0 + k0 + row));
                    if constexpr (G::BWK == 8) {
                        *reinterpret_cast<uint4*>(&kbuf[swz<UK>(row, cb)]) =
                            make_uint4(kr[u].w[q][0], kr[u].w[q][1], kr[u].w[q][2], kr[u].w[q][3]);
                    } else {
                        *reinterpret_cast<uint2*>(&kbuf[swz<UK>(row, cb >> 1) + 4 * (cb & 1)]) =
                            make_uint2(kr[u].w[q][0], kr[u].w[q][1]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G::VPT; ++u) {
            const int idx = tid_it + u * G::NTHR;
            if (idx < G::VB) {
                int tb, cb;
                block_coords<DVT, G::BWV>(idx, tb, cb);
#pragma unroll
                for (int c = 0; c < G::BWV; ++c)
                    *reinterpret_cast<uint4*>(&vbuf[swz<UC>(cb * G::BWV + c, tb)]) = block_column(vr[u], c);
            }
        }
        __syncthreads();

        {  // next key block, issued unconditionally (past the last: a discarded re-read)
            const bool more = m + 1 < nkb;
            const int kn = more ? (kb - 1) * BQ : k0;
            load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(kn) * DK, DK, more ? BQ : 0,
                                                             tid);
            load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(kn) * a.dv, a.dv,
                                                              more ? BQ : 0, tid);
        }

        const FragAddr<UK> fa_k(l16c, grpc);
        const FragAddr<UC> fa_v(l16c, grpc);  // V^T staged unit 4 t + grp (see staged_token)
#pragma unroll
        for (int t = 0; t < G::KST; ++t) {
            // on the diagonal block, steps above this wave's rows are skipped
            if ((!diag || 2 * t <= rb) && t * 32 < Lk) {
                f32x4 pa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint4 af = *reinterpret_cast<const uint4*>(&kbuf[fa_k.at(2 * t + hh, s)]);
                        pa[hh] = mfma16x16x32(af, qf[s], pa[hh]);
                    }
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int delta = rb - (2 * t + hh);
                    const bool on_diag = diag && delta == 0;
                    const float blk = fast_exp2(static_cast<float>(16 * delta + (q0 - k0) - 15) * lg2c);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float val = 0.0f;
                        const bool keep = !diag || delta > 0 || (delta == 0 && l16 >= 4 * grp + r);
                        const float dec = on_diag ? dlane[r] : dlane15[r] * blk;
                        if (keep) val = pa[hh][r] * dec;
                        pa[hh][r] = val;
                    }
                }
                const uint4 pf = make_uint4(pack2_bf16(pa[0][0], pa[0][1]), pack2_bf16(pa[0][2], pa[0][3]),
                                            pack2_bf16(pa[1][0], pa[1][1]), pack2_bf16(pa[1][2], pa[1][3]));
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
                    const uint4 af = *reinterpret_cast<const uint4*>(&vbuf[fa_v.at(nt, t)]);
                    oacc[nt] = mfma16x16x32(af, pf, oacc[nt]);
                }
            }
        }
        __syncthreads();
    }

    {
        const int row = rb * 16 + l16;
        if (row < Lq) {
            u16* orow = Og + static_cast<size_t>(q0 + row) * a.dv + grp * 4;
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
                *reinterpret_cast<uint2*>(orow + nt * 16) =
                    make_uint2(pack2_bf16(oacc[nt][0], oacc[nt][1]), pack2_bf16(oacc[nt][2], oacc[nt][3]));
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
