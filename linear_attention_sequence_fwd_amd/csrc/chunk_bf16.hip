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
// v_mfma_f32_16x16x32_bf16, in this order:
//   G3  O^T    = S^T Q^T, scaled by zeta   (the previous chunk's state, bf16 copy in LDS)
//   G4  S      = gamma^L S + Kx^T V   (Kx = keys scaled by xi; S in float32 accumulators)
//   G1  P^T    = K Q^T, masked by D (D generated in registers)
//   G2  O^T   += V^T P^T
// G3 runs before G4 so that the bf16 copy of the new state can be written
// straight after G4, without keeping a converted copy of S alive across G1/G2.
// Each wave owns one 16-row block of the chunk (paired so that the two waves
// sharing a SIMD carry equal causal work) and a grid cell of S tiles. The state
// is kept in float32 accumulators; a bf16 copy of it lives in LDS for G3.
// With C/16 waves per workgroup (8 for 128-token chunks) two waves share each
// SIMD, so one wave's LDS and HBM waits overlap the other's MFMAs.
//
// Keys and values are staged token-permuted inside each 32-token group (see
// staged_token), so a 16-byte unit of K^T / V^T holds the 8 tokens a lane
// group contracts over in both G4 and G2.
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

// Split of the (DK/16) x (DVT/16) state tiles over the waves: NG column
// groups times NW/NG row groups, chosen to minimise the LDS fragment reads of
// G4 per wave (proportional to row tiles + column tiles).
constexpr int pick_state_col_groups(int tm, int tn, int nw) {
    int best = 1, best_cost = 1 << 30;
    for (int ng = 1; ng <= nw; ng *= 2) {
        const int mg = nw / ng;
        if (nw % ng != 0 || tn % ng != 0 || tm % mg != 0) continue;
        const int cost = tm / mg + tn / ng;
        if (cost < best_cost) {
            best_cost = cost;
            best = ng;
        }
    }
    return best;
}

template <int DK, int DVT, int C>
struct ChunkGeo {
    static constexpr int NW = C / 16;         // waves per workgroup: one 16-row block of the chunk each
    static constexpr int NTHR = NW * 64;
    static constexpr int KSQ = DK / 32;       // 32-wide contraction steps over dk
    static constexpr int KST = C / 32;        // 32-wide contraction steps over tokens
    static constexpr int TM = DK / 16;        // 16-row tiles of S
    static constexpr int NTV = DVT / 16;      // 16-column tiles of S and O
    static constexpr int NG = pick_state_col_groups(TM, NTV, NW);
    static constexpr int MG = NW / NG;
    static constexpr int MT = TM / MG;        // S row tiles per wave
    static constexpr int NT = NTV / NG;       // S column tiles per wave
    static constexpr int BWK = stage_width(C, DK, NTHR);   // staging block widths
    static constexpr int BWV = stage_width(C, DVT, NTHR);
    static constexpr int KB = (C / 8) * (DK / BWK);   // key staging blocks per chunk
    static constexpr int VB = (C / 8) * (DVT / BWV);  // value staging blocks per chunk
    static constexpr int KPT = (KB + NTHR - 1) / NTHR;
    static constexpr int VPT = (VB + NTHR - 1) / NTHR;
    static_assert(C == 64 || C == 128, "chunk");
    static_assert(DK % 64 == 0 && DVT % 64 == 0, "tile sizes");
    static_assert(MG * MT == TM && NG * NT == NTV, "state split");
};

// Row block owned by wave w: waves w and w + NW/2 (which the dispatcher puts
// on the same SIMD) get blocks b and NW-1-b, so the causal work per SIMD is
// the same for every SIMD.
template <int NW>
__device__ __forceinline__ int wave_row_block(int w) {
    return w < NW / 2 ? w : (3 * NW / 2 - 1) - w;
}

template <int DK, int DVT, int C, bool STATE_ONLY>
__global__ __launch_bounds__((C / 16) * 64) void chunk_bf16_kernel(ChunkArgs a, HeadParams hp) {
    using G = ChunkGeo<DK, DVT, C>;
    constexpr int UK = DK / 8;  // 16-byte units in a row of K (row-major) and of S^T
    constexpr int UC = C / 8;   // 16-byte units in a row of K^T and V^T
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

    const int rb = wave_row_block<G::NW>(wave);      // this wave's 16 chunk rows
    const int d_base = (wave % G::MG) * G::MT * 16;  // this wave's S rows ...
    const int c_base = (wave / G::MG) * G::NT * 16;  // ... and S columns (within the value tile)

    // ---- prefetch the first chunk (issued before the initial-state loads so the
    //      two HBM round trips overlap)
    BlockRows<G::BWK> kr[G::KPT];
    BlockRows<G::BWV> vr[G::VPT];
    uint4 qf[G::KSQ];
    auto load_q = [&](int t, int Lq) {
        const int row = rb * 16 + l16;
        const u16* p = Qg + static_cast<size_t>(t + row) * DK + grp * 8;
#pragma unroll
        for (int s = 0; s < G::KSQ; ++s)
            qf[s] = row < Lq ? *reinterpret_cast<const uint4*>(p + s * 32) : make_uint4(0, 0, 0, 0);
    };
    {
        const int L0 = min(C, t_end - t_begin);
        load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(t_begin) * DK, DK, L0, tid);
        load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(t_begin) * a.dv, a.dv, L0, tid);
        if (!STATE_ONLY) load_q(t_begin, L0);
    }

    // ---- initial state
    f32x4 sacc[G::MT][G::NT];
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
        for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = d_base + mt * 16 + grp * 4 + r;
                const int c = vt * DVT + c_base + nt * 16 + l16;
                sacc[mt][nt][r] = s_src ? s_src[static_cast<size_t>(d) * a.dv + c] : 0.0f;
            }
    bool have_state = (s_src != nullptr);

    // bf16 copy of this wave's state tiles into S^T (row = value column, 4 consecutive dk)
    auto write_state_copy = [&](int l16_, int grp_) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt) {
                const int d = d_base + mt * 16 + grp_ * 4;
                const int c = c_base + nt * 16 + l16_;
                const uint2 w = make_uint2(pack2_bf16(sacc[mt][nt][0], sacc[mt][nt][1]),
                                           pack2_bf16(sacc[mt][nt][2], sacc[mt][nt][3]));
                *reinterpret_cast<uint2*>(&sbuf[swz<UK>(c, d >> 3) + (d & 7)]) = w;
            }
    };
    if (!STATE_ONLY && have_state) write_state_copy(l16, grp);

    // ---- per-lane decay constants
    // D[i][j] = gamma^(i-j) with i = 16 rb + l16, j = 16 jt + 4 grp + r:
    //        = gamma^(l16 - 4 grp - r) * gamma^(16 (rb - jt)).
    float dlane[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dlane[r] = fast_exp2(static_cast<float>(l16 - 4 * grp - r) * lg2f);
    const float zeta = fast_exp2(static_cast<float>(16 * rb + l16 + 1) * lg2f);
    const float gC = gamma_pow(lg2, C);

    for (int ch = 0; ch < nch; ++ch) {
        // Per-iteration copies the compiler cannot prove loop-invariant: the
        // block-write addresses and the decay factors are recomputed each
        // chunk (a few VALU ops under the MFMAs) instead of being hoisted out
        // of the loop and held in registers for its whole length.
        int tid_it = tid;
        float lg2_it = lg2f;
        asm volatile("" : "+v"(tid_it), "+v"(lg2_it));
        const float lg2c = lg2_it;
        const int l16c = tid_it & 15;
        const int grpc = (tid_it & 63) >> 4;
        const int t0 = t_begin + ch * C;
        const int L = min(C, t_end - t0);
        const bool has_next = (ch + 1) < nch;
        const int t1 = t0 + C;
        const int L1 = has_next ? min(C, t_end - t1) : 0;

        // ---- 1. rotate keys; K^T (scaled by xi) and V^T into LDS; rotate queries
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid_it + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK, G::BWK>(idx, tb, cb);
                if (hp.has_theta) {
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        if (staged_token(tb, q) < L)
                            rotate_row<G::BWK>(kr[u].w[q], hp, cb * (G::BWK / 2),
                                               static_cast<double>(a.pos0 + t0 + staged_token(tb, q)));
                }
                float xi[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) xi[q] = fast_exp2(static_cast<float>(L - 1 - staged_token(tb, q)) * lg2c);
#pragma unroll
                for (int c = 0; c < G::BWK; ++c) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float lo = bf16_to_f32(static_cast<u16>(elem16(kr[u].w[2 * p], c))) * xi[2 * p];
                        const float hi = bf16_to_f32(static_cast<u16>(elem16(kr[u].w[2 * p + 1], c))) * xi[2 * p + 1];
                        w[p] = pack2_bf16(lo, hi);
                    }
                    *reinterpret_cast<uint4*>(&kbuf[swz<UC>(cb * G::BWK + c, tb)]) = make_uint4(w[0], w[1], w[2], w[3]);
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
        if (!STATE_ONLY && hp.has_theta) {
            const int row = rb * 16 + l16;
            if (row < L) {
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s)
                    qf[s] = rotate8_bf16(qf[s], hp, s * 16 + grp * 4, static_cast<double>(a.pos0 + t0 + row));
            }
        }
        __syncthreads();  // A: K^T, V^T written

        // ---- 2. G3: O^T = S^T Q^T with the previous chunk's state, times zeta
        f32x4 oacc[G::NTV];
        if (!STATE_ONLY) {
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (have_state) {
                const FragAddr<UK> fa_s(l16c, grpc);  // S^T rows 16 nt + l16, dk 32 s + 8 grp
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
#pragma unroll
                    for (int s = 0; s < G::KSQ; ++s) {
                        const uint4 af = *reinterpret_cast<const uint4*>(&sbuf[fa_s.at(nt, s)]);
                        oacc[nt] = mfma16x16x32(af, qf[s], oacc[nt]);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[nt][r] *= zeta;
            }
        }

        // ---- 3. G4: S = gamma^L S + Kx^T V on this wave's tiles
        {
            const float gL = (L == C) ? gC : gamma_pow(lg2, L);
            const FragAddr<UC> fa_kt(d_base + l16c, grpc);  // K^T rows d_base + 16 mt + l16, tokens 32 t + 8 grp
            const FragAddr<UC> fa_vt(c_base + l16c, grpc);  // V^T rows c_base + 16 nt + l16, tokens 32 t + 8 grp
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[mt][nt][r] *= gL;
#pragma unroll
            for (int t = 0; t < G::KST; ++t) {
                if (t * 32 < L) {
                    uint4 af[G::MT];
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt) af[mt] = *reinterpret_cast<const uint4*>(&kbuf[fa_kt.at(mt, t)]);
#pragma unroll
                    for (int nt = 0; nt < G::NT; ++nt) {
                        const uint4 bfr = *reinterpret_cast<const uint4*>(&vbuf[fa_vt.at(nt, t)]);
#pragma unroll
                        for (int mt = 0; mt < G::MT; ++mt) sacc[mt][nt] = mfma16x16x32(af[mt], bfr, sacc[mt][nt]);
                    }
                }
            }
        }

        if (STATE_ONLY) {
            __syncthreads();  // everyone done reading kbuf / vbuf
            if (has_next) {
                load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(t1) * DK, DK, L1, tid);
                load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(t1) * a.dv, a.dv, L1, tid);
            }
            continue;
        }

        __syncthreads();  // B: S^T and K^T reads done

        // ---- 4. new bf16 state copy, K row-major into LDS, prefetch next keys/values
        write_state_copy(l16c, grpc);
        have_state = true;
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid_it + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK, G::BWK>(idx, tb, cb);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int row = staged_token(tb, q);
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
        if (has_next) {
            load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(t1) * DK, DK, L1, tid);
            load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(t1) * a.dv, a.dv, L1, tid);
        }
        __syncthreads();  // C: K row-major written

        // ---- 5. G1: P^T = K Q^T for this wave's rows, decay mask in registers,
        //         one 32-token step at a time, packed into bf16 B operands for G2.
        //         Steps entirely above the diagonal are skipped (one uniform
        //         branch per step); inside a step both 16-key halves run and
        //         the mask zeroes what lies above the diagonal.
        uint4 pf[G::KST];
        {
            const FragAddr<UK> fa_k(l16c, grpc);  // K rows 16 jt + l16, dk 32 s + 8 grp
#pragma unroll
            for (int t = 0; t < G::KST; ++t) {
                pf[t] = make_uint4(0, 0, 0, 0);
                if (2 * t <= rb) {
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
                        const float blk = fast_exp2(static_cast<float>(16 * delta) * lg2c);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float val = 0.0f;
                            if (delta > 0 || (delta == 0 && l16 >= 4 * grp + r)) val = pa[hh][r] * (dlane[r] * blk);
                            pa[hh][r] = val;
                        }
                    }
                    pf[t] = make_uint4(pack2_bf16(pa[0][0], pa[0][1]), pack2_bf16(pa[0][2], pa[0][3]),
                                       pack2_bf16(pa[1][0], pa[1][1]), pack2_bf16(pa[1][2], pa[1][3]));
                }
            }
        }

        // ---- prefetch next chunk's queries (qf is dead for this chunk now)
        if (has_next) load_q(t1, L1);

        // ---- 6. G2: O^T += V^T P^T
        {
            // V^T rows 16 nt + l16, staged unit 4 t + grp: tokens 32 t + 4 grp + {0..3, 16..19},
            // the order in which pf holds this lane group's scores
            const FragAddr<UC> fa_v(l16c, grpc);
#pragma unroll
            for (int t = 0; t < G::KST; ++t) {
                if (2 * t <= rb) {
#pragma unroll
                    for (int nt = 0; nt < G::NTV; ++nt) {
                        const uint4 af = *reinterpret_cast<const uint4*>(&vbuf[fa_v.at(nt, t)]);
                        oacc[nt] = mfma16x16x32(af, pf[t], oacc[nt]);
                    }
                }
            }
        }

        // ---- 7. store O (bf16)
        {
            const int row = rb * 16 + l16;
            if (row < L) {
                u16* orow = Og + static_cast<size_t>(t0 + row) * a.dv + grp * 4;
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
                    const uint2 w = make_uint2(pack2_bf16(oacc[nt][0], oacc[nt][1]),
                                               pack2_bf16(oacc[nt][2], oacc[nt][3]));
                    *reinterpret_cast<uint2*>(orow + nt * 16) = w;
                }
            }
        }
        __syncthreads();  // D: reads of kbuf and vbuf done before the next chunk's writes
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
            for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = d_base + mt * 16 + grp * 4 + r;
                    const int c = vt * DVT + c_base + nt * 16 + l16;
                    s_dst[static_cast<size_t>(d) * a.dv + c] = sacc[mt][nt][r];
                }
    }
}

template <int DK, int DVT, int C>
static hipError_t run_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev) {
    using G = ChunkGeo<DK, DVT, C>;
    const int bhv = a.B * a.H * a.nvt;
    if (a.nseg > 1) {
        launch_timed(chunk_bf16_kernel<DK, DVT, C, true>, dim3(bhv * (a.nseg - 1)), dim3(G::NTHR), 0, st, ev, a,
                     hp);
        const hipError_t e = launch_segment_scan(a, hp, st, ev ? ev + 2 : nullptr);
        if (e != hipSuccess) return e;
    } else {
        record_empty_phase(st, ev);
        record_empty_phase(st, ev ? ev + 2 : nullptr);
    }
    launch_timed(chunk_bf16_kernel<DK, DVT, C, false>, dim3(bhv * a.nseg), dim3(G::NTHR), 0, st,
                 ev ? ev + 4 : nullptr, a, hp);
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
