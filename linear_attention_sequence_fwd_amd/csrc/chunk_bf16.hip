// Chunkwise retention forward on bf16 inputs with float32 accumulation and a
// float32 carried state, for gfx950 (MI355X) matrix cores.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "3. The
// Chunkwise Recurrent Representation": inside a chunk of L tokens
//     O = ((Q K^T) (.) D) V + zeta (.) (Q S),     zeta_i = gamma^(i+1)
//     S <- gamma^L S + K^T (xi (.) V),            xi_j   = gamma^(L-1-j)
// (the xi weights are the in-chunk key decay that the page's printed carry
// leaves out; they follow from its recurrent form).
//
// One workgroup owns one (batch, head, value tile, sequence segment) and walks
// the segment's chunks in order. Per chunk it runs four contractions on
// v_mfma_f32_16x16x32_bf16:
//   G4  S      = gamma^L S + Kx^T V   (Kx = keys scaled by xi; S in AGPR/VGPR accumulators)
//   G1  P^T    = K Q^T, masked by D (D generated in registers)
//   G3  O^T    = S^T Q^T, scaled by zeta   (reads the previous chunk's state)
//   G2  O^T   += V^T P^T
// Each wave owns two 16-row blocks of the chunk (rows w and NRB-1-w, which
// balances the causal work) and a band of rows of S. The state is kept in
// float32 accumulators; a bf16 copy of it lives in LDS for G3.
//
// LDS (bf16, 16-byte units XOR-swizzled against bank conflicts):
//   kbuf  keys of the chunk, first as K^T scaled by xi (for G4) and then as K
//         row-major (for G1)
//   vbuf  V^T of the chunk's value tile
//   sbuf  S^T of the previous chunk (bf16), for G3
// Keys and values are loaded from HBM as 8x8 blocks straight into registers
// one chunk ahead and transposed in registers on their way into LDS. Queries
// go straight from HBM into the MFMA operand registers.

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace ret {

template <int DK, int DVT, int C>
struct ChunkGeo {
    static constexpr int NW = C / 32;         // waves per workgroup
    static constexpr int NTHR = NW * 64;
    static constexpr int NRB = C / 16;        // 16-row blocks in a chunk
    static constexpr int KSQ = DK / 32;       // 32-wide contraction steps over dk
    static constexpr int KST = C / 32;        // 32-wide contraction steps over tokens
    static constexpr int MT = DK / 16 / NW;   // 16-row tiles of S per wave
    static constexpr int NTV = DVT / 16;      // 16-column tiles of the value tile
    static constexpr int KB = (C / 8) * (DK / 8);   // 8x8 key blocks per chunk
    static constexpr int VB = (C / 8) * (DVT / 8);  // 8x8 value blocks per chunk
    static constexpr int KPT = (KB + NTHR - 1) / NTHR;
    static constexpr int VPT = (VB + NTHR - 1) / NTHR;
    static_assert(C == 64 || C == 128, "chunk");
    static_assert(DK % 64 == 0 && DVT % 64 == 0, "tile sizes");
    static_assert(MT >= 1 && MT * NTV <= 32, "state accumulators per wave");
};

template <int DK, int DVT, int C, bool STATE_ONLY>
__global__ __launch_bounds__((C / 32) * 64) void chunk_bf16_kernel(ChunkArgs a, HeadParams hp) {
    using G = ChunkGeo<DK, DVT, C>;
    __shared__ __attribute__((aligned(16))) u16 kbuf[C * DK];
    __shared__ __attribute__((aligned(16))) u16 vbuf[DVT * C];
    __shared__ __attribute__((aligned(16))) u16 sbuf[STATE_ONLY ? 8 : DVT * DK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int grp = lane >> 4;

    // ---- which (batch*head, segment, value tile) this workgroup owns
    const int nseg_grid = STATE_ONLY ? a.nseg - 1 : a.nseg;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int vt = lb % a.nvt;
    const int seg = (lb / a.nvt) % nseg_grid;
    const int bh = lb / (a.nvt * nseg_grid);
    const int h = bh % a.H;

    const float gam = hp.gamma[h];
    const double lg2 = log2_gamma(gam);
    const float lg2f = static_cast<float>(lg2);

    const int t_begin = seg * a.seg_len;
    const int t_end = min(a.N, t_begin + a.seg_len);
    const int nch = (t_end - t_begin + C - 1) / C;

    const size_t tok0 = static_cast<size_t>(bh) * a.N;
    const u16* Kg = a.k + tok0 * DK;
    const u16* Qg = a.q + tok0 * DK;
    const u16* Vg = a.v + tok0 * a.dv + vt * DVT;
    u16* Og = a.o + tok0 * a.dv + vt * DVT;

    const int d_base = wave * G::MT * 16;  // first S row owned by this wave
    const int rbs[2] = {wave, G::NRB - 1 - wave};

    // ---- initial state
    f32x4 sacc[G::MT][G::NTV];
    const float* s_src = nullptr;
    if (!STATE_ONLY) {
        if (a.nseg > 1)
            s_src = a.ws + (static_cast<size_t>(bh) * a.nseg + seg) * DK * a.dv;
        else if (a.state_in)
            s_src = a.state_in + static_cast<size_t>(bh) * DK * a.dv;
    }
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = d_base + mt * 16 + grp * 4 + r;
                const int c = vt * DVT + nt * 16 + l16;
                sacc[mt][nt][r] = s_src ? s_src[static_cast<size_t>(d) * a.dv + c] : 0.0f;
            }
    bool have_state = (s_src != nullptr);
    if (!STATE_ONLY && have_state) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) {
                const int d = d_base + mt * 16 + grp * 4;
                const int c = nt * 16 + l16;
                uint2 w = make_uint2(pack2_bf16(sacc[mt][nt][0], sacc[mt][nt][1]),
                                     pack2_bf16(sacc[mt][nt][2], sacc[mt][nt][3]));
                *reinterpret_cast<uint2*>(&sbuf[sidx<DK>(c, d)]) = w;
            }
    }

    // ---- per-lane decay constants
    // D[i][j] = gamma^(i-j) with i = 16 rb + l16, j = 16 jt + 4 grp + r:
    //        = gamma^(l16 - 4 grp - r) * gamma^(16 (rb - jt)).
    float dlane[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dlane[r] = exp2f(static_cast<float>(l16 - 4 * grp - r) * lg2f);
    const float zeta0 = exp2f(static_cast<float>(16 * rbs[0] + l16 + 1) * lg2f);
    const float zeta1 = exp2f(static_cast<float>(16 * rbs[1] + l16 + 1) * lg2f);
    const float gC = gamma_pow(lg2, C);

    // ---- prefetch the first chunk
    uint4 kr[G::KPT][8];
    uint4 vr[G::VPT][8];
    uint4 qf[2][G::KSQ];
    {
        const int L0 = min(C, t_end - t_begin);
        load_blocks<DK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(t_begin) * DK, DK, L0, tid);
        load_blocks<DVT, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(t_begin) * a.dv, a.dv, L0, tid);
        if (!STATE_ONLY) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = rbs[i] * 16 + l16;
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s)
                    qf[i][s] = row < L0 ? *reinterpret_cast<const uint4*>(Qg + static_cast<size_t>(t_begin + row) * DK + s * 32 + grp * 8)
                                        : make_uint4(0, 0, 0, 0);
            }
        }
    }

    for (int ch = 0; ch < nch; ++ch) {
        // Per-iteration copies the compiler cannot prove loop-invariant: LDS
        // addresses and decay factors are recomputed each chunk (a few VALU
        // ops under the MFMAs) instead of being hoisted and held in registers.
        int lane_it = lane;
        float lg2_it = lg2f;
        asm volatile("" : "+v"(lane_it), "+v"(lg2_it));
        const int l16 = lane_it & 15;
        const int grp = lane_it >> 4;
        const float lg2f = lg2_it;
        const int t0 = t_begin + ch * C;
        const int L = min(C, t_end - t0);
        const bool has_next = (ch + 1) < nch;
        const int t1 = t0 + C;
        const int L1 = has_next ? min(C, t_end - t1) : 0;

        // ---- 1. rotate keys; K^T (scaled by xi) and V^T into LDS
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK>(idx, tb, cb);
                if (hp.has_theta) {
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (tb * 8 + q < L)
                            kr[u][q] = rotate8_bf16(kr[u][q], hp, cb * 4,
                                                    static_cast<double>(a.pos0 + t0 + tb * 8 + q));
                }
                float xi[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) xi[q] = exp2f(static_cast<float>(L - 1 - tb * 8 - q) * lg2f);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float lo = bf16_to_f32(static_cast<u16>(elem16(kr[u][2 * p], c))) * xi[2 * p];
                        const float hi = bf16_to_f32(static_cast<u16>(elem16(kr[u][2 * p + 1], c))) * xi[2 * p + 1];
                        w[p] = pack2_bf16(lo, hi);
                    }
                    *reinterpret_cast<uint4*>(&kbuf[tidx<C>(cb * 8 + c, tb * 8)]) = make_uint4(w[0], w[1], w[2], w[3]);
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
                    for (int p = 0; p < 4; ++p)
                        w[p] = elem16(vr[u][2 * p], c) | (elem16(vr[u][2 * p + 1], c) << 16);
                    *reinterpret_cast<uint4*>(&vbuf[tidx<C>(cb * 8 + c, tb * 8)]) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
        __syncthreads();  // A

        // ---- 2. G4: S = gamma^L S + Kx^T V
        {
            const float gL = (L == C) ? gC : gamma_pow(lg2, L);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[mt][nt][r] *= gL;
#pragma unroll
            for (int t = 0; t < G::KST; ++t) {
                if (t * 32 < L) {
                    uint4 af[G::MT];
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt)
                        af[mt] = *reinterpret_cast<const uint4*>(&kbuf[tidx<C>(d_base + mt * 16 + l16, t * 32 + grp * 8)]);
#pragma unroll
                    for (int nt = 0; nt < G::NTV; ++nt) {
                        const uint4 bfr = *reinterpret_cast<const uint4*>(&vbuf[tidx<C>(nt * 16 + l16, t * 32 + grp * 8)]);
#pragma unroll
                        for (int mt = 0; mt < G::MT; ++mt) sacc[mt][nt] = mfma16x16x32(af[mt], bfr, sacc[mt][nt]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (STATE_ONLY) {
            __syncthreads();  // everyone done reading kbuf / vbuf
            if (has_next) {
                load_blocks<DK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(t1) * DK, DK, L1, tid);
                load_blocks<DVT, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(t1) * a.dv, a.dv, L1, tid);
            }
            continue;
        }

        __syncthreads();  // B: K^T reads done

        // ---- 3. K row-major into LDS; prefetch next chunk's keys and values
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK>(idx, tb, cb);
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    *reinterpret_cast<uint4*>(&kbuf[kidx_rm<DK>(tb * 8 + q, cb * 8)]) = kr[u][q];
            }
        }
        if (has_next) {
            load_blocks<DK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(t1) * DK, DK, L1, tid);
            load_blocks<DVT, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(t1) * a.dv, a.dv, L1, tid);
        }
        // rotate this chunk's queries while the writes settle
        if (hp.has_theta) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = rbs[i] * 16 + l16;
                if (row < L) {
#pragma unroll
                    for (int s = 0; s < G::KSQ; ++s)
                        qf[i][s] = rotate8_bf16(qf[i][s], hp, s * 16 + grp * 4,
                                                static_cast<double>(a.pos0 + t0 + row));
                }
            }
        }
        __syncthreads();  // C

        // ---- 4. G1: P^T = K Q^T, decay mask in registers, one 32-token step at
        //         a time, packed straight into bf16 B operands for G2
        const int rb_max = rbs[1];  // rbs[1] >= rbs[0]
        uint4 pf[2][G::KST];
#pragma unroll
        for (int t = 0; t < G::KST; ++t) {
            f32x4 pa[2][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) pa[i][0] = pa[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int jt = 2 * t + hh;
                if (jt <= rb_max && jt * 16 < L) {
#pragma unroll
                    for (int s = 0; s < G::KSQ; ++s) {
                        const uint4 af = *reinterpret_cast<const uint4*>(&kbuf[kidx_rm<DK>(jt * 16 + l16, s * 32 + grp * 8)]);
#pragma unroll
                        for (int i = 0; i < 2; ++i)
                            if (jt <= rbs[i]) pa[i][hh] = mfma16x16x32(af, qf[i][s], pa[i][hh]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int delta = rbs[i] - (2 * t + hh);
                    const float blk = exp2f(static_cast<float>(16 * delta) * lg2f);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float val = 0.0f;
                        if (delta > 0 || (delta == 0 && l16 >= 4 * grp + r)) val = pa[i][hh][r] * (dlane[r] * blk);
                        pa[i][hh][r] = val;
                    }
                }
                pf[i][t] = make_uint4(pack2_bf16(pa[i][0][0], pa[i][0][1]), pack2_bf16(pa[i][0][2], pa[i][0][3]),
                                      pack2_bf16(pa[i][1][0], pa[i][1][1]), pack2_bf16(pa[i][1][2], pa[i][1][3]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- 5. G3: O^T = S^T Q^T (previous state), times zeta
        f32x4 oacc[2][G::NTV];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) oacc[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (have_state) {
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) {
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s) {
                    const uint4 af = *reinterpret_cast<const uint4*>(&sbuf[sidx<DK>(nt * 16 + l16, s * 32 + grp * 8)]);
#pragma unroll
                    for (int i = 0; i < 2; ++i) oacc[i][nt] = mfma16x16x32(af, qf[i][s], oacc[i][nt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    oacc[0][nt][r] *= zeta0;
                    oacc[1][nt][r] *= zeta1;
                }
        }

        // ---- prefetch next chunk's queries (qf is dead for this chunk now)
        if (has_next) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = rbs[i] * 16 + l16;
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s)
                    qf[i][s] = row < L1 ? *reinterpret_cast<const uint4*>(Qg + static_cast<size_t>(t1 + row) * DK + s * 32 + grp * 8)
                                        : make_uint4(0, 0, 0, 0);
            }
        }

        // ---- 6. G2: O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < G::KST; ++t) {
            if (2 * t <= rb_max && t * 32 < L) {
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
                    const int row = nt * 16 + l16;
                    const uint2 lo = *reinterpret_cast<const uint2*>(&vbuf[tidx<C>(row, t * 32 + grp * 4)]);
                    const uint2 hi = *reinterpret_cast<const uint2*>(&vbuf[tidx<C>(row, t * 32 + 16 + grp * 4)]);
                    const uint4 af = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (2 * t <= rbs[i]) oacc[i][nt] = mfma16x16x32(af, pf[i][t], oacc[i][nt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- 7. store O (bf16)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = rbs[i] * 16 + l16;
            if (row < L) {
                u16* orow = Og + static_cast<size_t>(t0 + row) * a.dv;
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
                    const uint2 w = make_uint2(pack2_bf16(oacc[i][nt][0], oacc[i][nt][1]),
                                               pack2_bf16(oacc[i][nt][2], oacc[i][nt][3]));
                    *reinterpret_cast<uint2*>(orow + nt * 16 + grp * 4) = w;
                }
            }
        }
        __syncthreads();  // D: reads of kbuf, vbuf, sbuf done

        // ---- 8. bf16 copy of the new state for the next chunk's G3
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) {
                const int d = d_base + mt * 16 + grp * 4;
                const int c = nt * 16 + l16;
                const uint2 w = make_uint2(pack2_bf16(sacc[mt][nt][0], sacc[mt][nt][1]),
                                           pack2_bf16(sacc[mt][nt][2], sacc[mt][nt][3]));
                *reinterpret_cast<uint2*>(&sbuf[sidx<DK>(c, d)]) = w;
            }
        have_state = true;
    }

    // ---- final state
    float* s_dst = nullptr;
    if (STATE_ONLY)
        s_dst = a.ws + (static_cast<size_t>(bh) * a.nseg + seg + 1) * DK * a.dv;
    else if (seg == a.nseg - 1 && a.state_out)
        s_dst = a.state_out + static_cast<size_t>(bh) * DK * a.dv;
    if (s_dst) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = d_base + mt * 16 + grp * 4 + r;
                    const int c = vt * DVT + nt * 16 + l16;
                    s_dst[static_cast<size_t>(d) * a.dv + c] = sacc[mt][nt][r];
                }
    }
}

template <int DK, int DVT, int C>
static hipError_t run_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev) {
    using G = ChunkGeo<DK, DVT, C>;
    const int bhv = a.B * a.H * a.nvt;
    if (ev) (void)hipEventRecord(ev[0], st);
    if (a.nseg > 1) chunk_bf16_kernel<DK, DVT, C, true><<<dim3(bhv * (a.nseg - 1)), dim3(G::NTHR), 0, st>>>(a, hp);
    if (ev) (void)hipEventRecord(ev[1], st);
    if (a.nseg > 1) {
        const hipError_t e = launch_segment_scan(a, hp, st);
        if (e != hipSuccess) return e;
    }
    if (ev) (void)hipEventRecord(ev[2], st);
    chunk_bf16_kernel<DK, DVT, C, false><<<dim3(bhv * a.nseg), dim3(G::NTHR), 0, st>>>(a, hp);
    if (ev) (void)hipEventRecord(ev[3], st);
    return hipGetLastError();
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev) {
#define RET_CASE(DK_, DVT_, C_) \
    if (a.dk == DK_ && dvt == DVT_ && a.chunk == C_) return run_chunk_bf16<DK_, DVT_, C_>(a, hp, st, ev);
    RET_CASE(64, 64, 64)
    RET_CASE(64, 128, 64)
    RET_CASE(128, 64, 64)
    RET_CASE(128, 128, 64)
    RET_CASE(256, 64, 64)
    RET_CASE(64, 64, 128)
    RET_CASE(64, 128, 128)
    RET_CASE(128, 64, 128)
    RET_CASE(128, 128, 128)
    RET_CASE(256, 64, 128)
    RET_CASE(256, 128, 128)
#undef RET_CASE
    return hipErrorInvalidValue;
}

}  // namespace ret
