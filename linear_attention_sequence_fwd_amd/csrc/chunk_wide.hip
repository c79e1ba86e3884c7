// Chunkwise retention forward for wide heads (d_k of 128 or 256, value tiles of
// 128 columns, 128-token chunks) on gfx950 (MI355X) matrix cores: bf16 inputs,
// float32 accumulation and state, no rotation.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "3. The
// Chunkwise Recurrent Representation": inside a chunk of L tokens
//     O = ((Q K^T) (.) D) V + zeta (.) (Q S),     zeta_i = gamma^(i+1)
//     S <- gamma^L S + K^T (xi (.) V),            xi_j   = gamma^(L-1-j)
// (xi is the in-chunk key decay that the page's printed carry leaves out).
//
// Rescaled form over decay groups. Chunks are taken in groups of R (R C
// tokens); tau counts tokens from the start of the group. With
//     V3 = gamma^-(tau+1) V    (each value row scaled once, at staging)
// and A = gamma^-e S, where e is the number of group tokens already folded in,
// every decay factor moves out of the contractions:
//     O   = gamma^(tau_i + 1) (Q A + mask(Q K^T) V3)     (row i at group offset tau_i)
//     A  <- A + K^T V3
// and only at the end of a group is A scaled back to S (A <- gamma^e A), so the
// float32 state is touched by the vector ALU once per R chunks. The host picks
// the largest R in {8, 4, 2, 1} with gamma^(R C) >= 2^-64 for every head,
// which keeps every factor far inside the float32 range.
//
// One workgroup of eight waves (two per SIMD, each in half the SIMD's register
// file) owns one (batch, head, value tile) and walks its chunks in order. Wave
// w owns one query block of 16 tokens (w, or 11 - w for w >= 4, so that the two
// waves of a SIMD carry blocks b and 7 - b and every SIMD the same causal work);
// while one wave of a SIMD waits for its LDS operands the other issues matrix
// instructions (four waves owning two blocks each, every fragment feeding two
// instructions, measured 6% slower). The float32 state is split over the waves
// by d_k rows: wave w holds rows [w d_k/8, (w+1) d_k/8) of all 128 columns in
// MFMA accumulators. Per chunk, on v_mfma_f32_16x16x32_bf16:
//   G3  O^T  = A^T Q^T                    (bf16 copy of A^T in LDS)
//   G1  P^T  = K Q^T, causal select on the diagonal tiles
//   G2  O^T += V3^T P^T                   (V3^T by transposing LDS reads)
//   G4  A   += K^T V3                     (K^T by transposing LDS reads)
//
// LDS (bf16, 16-byte units XOR-swizzled by row against bank conflicts): two
// key-sized buffers that trade roles every chunk (this chunk's keys; the state
// copy, which G3 reads first, after which the next chunk's keys are loaded
// into it straight from HBM), and V3 of the chunk. Values come through
// registers one chunk ahead (they are scaled on the way in); queries go from
// HBM straight into MFMA operand registers. Buffer loads make rows past the
// end of the sequence read as zero, and output stores past it are dropped.

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"
#include "wide.hpp"

#include <cmath>

namespace ret {

namespace {

using namespace wide;

constexpr int kWideC = 128;            // tokens per chunk
constexpr int kWideDvt = 128;          // value columns per workgroup
constexpr int kWideThreads = 512;      // eight waves, two per SIMD
constexpr int kPipeDepth = 4;          // steps between an LDS read and its use

// What one workgroup computes for its chain (batch x head x value tile):
constexpr int kWideWhole = 0;      // outputs and end state of the whole sequence
constexpr int kWideStatePass = 1;  // the end state of segment `seg` from a zero state (no outputs)
constexpr int kWideSegPass = 2;    // outputs of segment `seg` from its start state (after the scan)

template <int DK>
struct WideGeo {
    static constexpr int UK = DK / 8;                      // 16-byte units per key row
    static constexpr int UV = kWideDvt / 8;                // 16-byte units per value row (of the tile)
    static constexpr int KSQ = DK / 32;                    // 32-wide contraction steps over d_k
    static constexpr int NTV = kWideDvt / 16;              // 16-column tiles of the value tile
    static constexpr int MT = DK / 128;                    // 16-row state tiles per wave
    static constexpr int VU = kWideC * UV / kWideThreads;  // value units per thread
    static constexpr int VROWS = kWideThreads / UV;        // value rows per load step
    static constexpr int KBLK = kWideC * DK * 2 / 1024 / 8;  // 1 KiB key blocks per wave
    static_assert(DK == 128 || DK == 256, "key width");
};

}  // namespace

namespace {

// One call's chain `chain` (batch x head x value tile), over the whole
// sequence or one segment of it (MODE). MULTI only tells the kernels' copies
// apart (each kernel its own specialization, as each holds its own LDS).
// Segmented calls keep their states in the workspace as float32
// [B*H][nseg][d_k][d_v]: slot s + 1 receives segment s's end state from zero
// (state pass), the scan turns slot s into segment s's start state, and the
// segment pass starts from it.
template <int DK, bool MULTI, int MODE = kWideWhole>
__device__ __forceinline__ void chunk_wide_body(const ChunkArgs& a, const HeadParams& hp, const int chain,
                                                const int seg) {
    using G = WideGeo<DK>;
    constexpr int C = kWideC;
    constexpr int UK = G::UK;
    // separate objects, so the compiler can tell reads of one from the loads into the other
    __shared__ __attribute__((aligned(16))) u16 pb0[C * DK];
    __shared__ __attribute__((aligned(16))) u16 pb1[C * DK];
    __shared__ __attribute__((aligned(16))) u16 vbuf[C * kWideDvt];

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    // Per-lane indices. Inside the chunk loop they are refreshed from an opaque
    // copy of the thread index every chunk, so per-lane addresses and factors
    // are recomputed there (a few ALU operations under the matrix work) rather
    // than hoisted out of the loop and held in registers for its whole length.
    int tid = threadIdx.x;
    int lane = tid & 63;
    int l16 = lane & 15;
    int grp = lane >> 4;
    auto refresh_lane = [&]() __attribute__((always_inline)) {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        tid = t;
        lane = t & 63;
        l16 = t & 15;
        grp = (t & 63) >> 4;
    };

    const int vt = chain % a.nvt;
    const int bh = chain / a.nvt;
    const int h = bh % a.H;
    const float gam = hp.gamma[h];
    const double lg2 = log2_gamma(gam);
    const float lg2f = static_cast<float>(lg2);
    const int N = a.N;
    const int t_begin = MODE == kWideWhole ? 0 : seg * a.seg_len;  // tokens [t_begin, t_end) of this pass
    const int t_end = MODE == kWideWhole ? N : min(N, t_begin + a.seg_len);
    const int nch = (t_end - t_begin + C - 1) / C;
    const int R = a.rescale;
    const float g_group = gamma_pow(lg2, static_cast<double>(R) * C);  // gamma^(R C)

    const size_t tok0 = static_cast<size_t>(bh) * N;
    const int ldqk = a.ldqk > 0 ? a.ldqk : DK;  // query / key row stride, elements
    const char* Kg = reinterpret_cast<const char*>(a.k + tok0 * ldqk);
    const char* Qg = reinterpret_cast<const char*>(a.q + tok0 * ldqk);
    const char* Vg = reinterpret_cast<const char*>(a.v + tok0 * a.dv + vt * kWideDvt);
    char* Og = reinterpret_cast<char*>(a.o + tok0 * a.dv + vt * kWideDvt);
    const int ldv = a.dv * 2;    // value / output row stride, bytes
    const int ldk = ldqk * 2;  // key / query row stride, bytes
    constexpr int tile_bytes = kWideDvt * 2;
    const int d0 = wave * (DK / 8);  // this wave's state rows
    // this wave's query block: waves w and w + 4 share a SIMD (a workgroup's waves
    // are dealt to the SIMDs in turn), so they take blocks w and 7 - w and every
    // SIMD carries the same causal work
    const int qblk = wave < 4 ? wave : 11 - wave;

    uint4 vst[G::VU];           // the next chunk's values (scaled to V3 in registers before staging)
    uint4 qf[G::KSQ];           // queries of block wave: row 16 wave + l16, d_k 32 s + 8 grp
    f32x4 sacc[G::MT][G::NTV];  // A: rows d0 + 16 mt + 4 grp + r, columns 16 nt + l16
    f32x4 oacc[G::NTV];         // O^T: [column tile]
    uint4 pf[4];                // P^T as bf16 B operands: [32-key step]

    // Rows of one chunk in memory (t: first token of the pass, L valid rows): a
    // buffer resource over the L rows. In reverse token order (a.rev) pass row r
    // of the chunk is row L - 1 - r of the resource. Rows past L fall outside it
    // either way (a negative offset reads as out of range), so they load as zero
    // and their stores are dropped.
    const bool rev = a.rev != 0;
    auto first_row = [&](int t, int L) __attribute__((always_inline)) { return rev ? N - t - L : t; };
    auto mrow = [&](int L, int row) __attribute__((always_inline)) { return rev ? L - 1 - row : row; };
    auto key_rsrc = [&](int t, int L) __attribute__((always_inline)) {
        return make_rsrc(Kg + static_cast<size_t>(first_row(t, L)) * ldk, (L - 1) * ldk + DK * 2);
    };
    auto q_rsrc = [&](int t, int L) __attribute__((always_inline)) {
        return make_rsrc(Qg + static_cast<size_t>(first_row(t, L)) * ldk, (L - 1) * ldk + DK * 2);
    };
    auto value_rsrc = [&](int t, int L) __attribute__((always_inline)) {
        return make_rsrc(Vg + static_cast<size_t>(first_row(t, L)) * ldv, (L - 1) * ldv + tile_bytes);
    };
    auto out_rsrc = [&](int t, int L) __attribute__((always_inline)) {
        return make_rsrc(Og + static_cast<size_t>(first_row(t, L)) * ldv, (L - 1) * ldv + tile_bytes);
    };
    // Key block i (1 KiB) of this wave's share, straight into LDS: each wave
    // instruction fills 1 KiB of consecutive LDS (lane l the 16-byte unit at
    // 16 l), so each lane fetches the unit the swizzled layout puts there.
    auto load_key_block = [&](__amdgpu_buffer_rsrc_t rk, int L, u16* dst, int i) __attribute__((always_inline)) {
        const int blk = wave * G::KBLK + i;
        const int e = blk * 512 + lane * 8;  // element offset of this lane's unit
        const int row = e / DK;              // LDS row = pass row of the chunk
        const int unit = ((e % DK) >> 3) ^ (row & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_ptr)(dst + blk * 512), 16,
                                                 mrow(L, row) * ldk + unit * 16, 0, 0, 0);
    };
    auto load_value_unit = [&](__amdgpu_buffer_rsrc_t rv, int L, int j) __attribute__((always_inline)) {
        vst[j] = buf_load16(rv, mrow(L, tid / G::UV + j * G::VROWS) * ldv + (tid % G::UV) * 16);
    };
    // query unit s
    auto load_q_unit = [&](__amdgpu_buffer_rsrc_t rq, int L, int s) __attribute__((always_inline)) {
        qf[s] = buf_load16(rq, mrow(L, 16 * qblk + l16) * ldk + grp * 16 + s * 64);
    };
    // value unit j to V3 (tau0: group offset of the chunk's first token)
    auto scale_value_unit = [&](int j, int tau0) __attribute__((always_inline)) {
        const int row = tid / G::UV + j * G::VROWS;
        vst[j] = scale8_bf16(vst[j], fast_exp2(-static_cast<float>(tau0 + row + 1) * lg2f));
    };
    auto write_values = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < G::VU; ++j)
            *reinterpret_cast<uint4*>(&vbuf[swz<G::UV>(tid / G::UV + j * G::VROWS, tid % G::UV)]) = vst[j];
    };
    // bf16 copy of the state (A^T, row = value column) for G3
    auto write_state_copy = [&](u16* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) {
                const int d = d0 + mt * 16 + grp * 4;
                const int c = nt * 16 + l16;
                const uint2 w = make_uint2(pack2_bf16(sacc[mt][nt][0], sacc[mt][nt][1]),
                                           pack2_bf16(sacc[mt][nt][2], sacc[mt][nt][3]));
                *reinterpret_cast<uint2*>(&dst[swz<UK>(c, d >> 3) + (d & 7)]) = w;
            }
    };
    // Transposing-read fragment (8 tokens of 32-token step t, rows 4 grp + {0..3, 16..19})
    // of 16 consecutive columns from a row-major tile: lane (l16, grp) points at
    // token 4 grp + l16/4 (+16), columns col0 + 4 (l16 % 4) .. +3.
    auto tr_frag = [&](const u16* buf, auto width_tag, int col0, int t) __attribute__((always_inline)) {
        constexpr int W = decltype(width_tag)::value;  // row width in elements
        const int tok = 4 * grp + (l16 >> 2);
        const int c = col0 + 4 * (l16 & 3);
        const int base = swz<W / 8>(tok, c >> 3) + (c & 7);
        const uint2 lo = lds_read_tr16x4(&buf[base + (32 * t) * W]);
        const uint2 hi = lds_read_tr16x4(&buf[base + (32 * t + 16) * W]);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };

    // G1 and G2 for the wave owning block W. The next chunk's keys go into LDS during G1.
    auto g12 = [&](const u16* __restrict__ kb, u16* __restrict__ next_kb, __amdgpu_buffer_rsrc_t rk, int Lk, auto wtag)
                   __attribute__((always_inline)) {
        constexpr int B0 = decltype(wtag)::value;
        constexpr int T0 = B0 / 2 + 1;
        const FragAddr<UK> fk(l16, grp);  // K rows 16 kt + l16, d_k 32 s + 8 grp
        // G1, step j: 32-key step t = j / KSQ (key tiles 2t, 2t+1), d_k step s = j % KSQ
        struct KF {
            uint4 a, b;
        };
        f32x4 p[2];  // tiles 2t and 2t+1
        constexpr int NS1 = T0 * G::KSQ;
        pipelined<NS1, kPipeDepth>(
            [&](auto j) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::KSQ, s = decltype(j)::value % G::KSQ;
                KF f;
                f.a = *reinterpret_cast<const uint4*>(&kb[fk.at(2 * t, s)]);
                if constexpr (2 * t + 1 <= B0) f.b = *reinterpret_cast<const uint4*>(&kb[fk.at(2 * t + 1, s)]);
                return f;
            },
            [&](auto j, const KF& f) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::KSQ, s = decltype(j)::value % G::KSQ;
                constexpr bool two = 2 * t + 1 <= B0;
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                p[0] = mfma16x16x32(f.a, qf[s], s == 0 ? zero : p[0]);
                if constexpr (two) p[1] = mfma16x16x32(f.b, qf[s], s == 0 ? zero : p[1]);
                if constexpr (s == G::KSQ - 1) {
                    f32x4 r[2] = {p[0], two ? p[1] : zero};
                    // causal select on diagonal tiles: key 16 kt + 4 grp + q vs token 16 blk + l16
                    auto mask = [&](f32x4& x, bool diag) __attribute__((always_inline)) {
                        if (diag) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) x[q] = (4 * grp + q <= l16) ? x[q] : 0.0f;
                        }
                    };
                    mask(r[0], 2 * t == B0);
                    mask(r[1], 2 * t + 1 == B0);
                    pf[t] = make_uint4(pack2_bf16(r[0][0], r[0][1]), pack2_bf16(r[0][2], r[0][3]),
                                       pack2_bf16(r[1][0], r[1][1]), pack2_bf16(r[1][2], r[1][3]));
                }
            },
            [&](auto j) __attribute__((always_inline)) {
                spread<G::KBLK, NS1, decltype(j)::value>([&](auto i) { load_key_block(rk, Lk, next_kb, i); });
            });
        // G2, step j: 32-key step t = j / NTV, column tile nt = j % NTV
        constexpr int NS2 = T0 * G::NTV;
        pipelined<NS2, kPipeDepth>(
            [&](auto j) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                return tr_frag(vbuf, Ic<kWideDvt>{}, 16 * nt, t);
            },
            [&](auto j, const uint4& vf) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                oacc[nt] = mfma16x16x32(vf, pf[t], oacc[nt]);
            },
            [](auto) {});
    };
    // G4: A += K^T V3 on this wave's state tiles. Step j: 32-key step t =
    // j / NTV, column tile nt = j % NTV; the first step of each t also brings
    // that step's key fragments. Riding along: the chunk's outputs (scaled by
    // z, rounded and stored), the next chunk's query loads and the scaling of
    // its values (tau_next: their group offset).
    auto g4 = [&](const u16* kb, __amdgpu_buffer_rsrc_t ro, int Lo, __amdgpu_buffer_rsrc_t rq, int Lq, float z,
                  int tau_next) __attribute__((always_inline)) {
        struct F4 {
            uint4 v;
            uint4 k[G::MT];
        };
        uint4 kt[G::MT];
        constexpr int NS4 = 4 * G::NTV;
        pipelined<NS4, kPipeDepth>(
            [&](auto j) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                F4 f;
                f.v = tr_frag(vbuf, Ic<kWideDvt>{}, 16 * nt, t);
                if constexpr (nt == 0) {
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt) f.k[mt] = tr_frag(kb, Ic<DK>{}, d0 + 16 * mt, t);
                }
                return f;
            },
            [&](auto j, const F4& f) __attribute__((always_inline)) {
                constexpr int nt = decltype(j)::value % G::NTV;
                if constexpr (nt == 0) {
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt) kt[mt] = f.k[mt];
                }
#pragma unroll
                for (int mt = 0; mt < G::MT; ++mt) sacc[mt][nt] = mfma16x16x32(kt[mt], f.v, sacc[mt][nt]);
            },
            [&](auto j) __attribute__((always_inline)) {
                constexpr int J = decltype(j)::value;
                spread<G::NTV, NS4, J>([&](auto i) {
                    constexpr int nt = decltype(i)::value;
                    const f32x4 o = oacc[nt];
                    const uint2 w = make_uint2(pack2_bf16(o[0] * z, o[1] * z), pack2_bf16(o[2] * z, o[3] * z));
                    buf_store8(w, ro, mrow(Lo, 16 * qblk + l16) * ldv + grp * 8 + nt * 32);
                });
                spread<G::KSQ, NS4, J>([&](auto i) { load_q_unit(rq, Lq, i); });
                spread<G::VU, NS4, J>([&](auto i) { scale_value_unit(decltype(i)::value, tau_next); });
            });
    };

    // ---- start: the first chunk's values, keys and queries; the initial state
    {
        const int L0 = min(C, t_end - t_begin);
        const __amdgpu_buffer_rsrc_t rv = value_rsrc(t_begin, L0), rk = key_rsrc(t_begin, L0);
#pragma unroll
        for (int j = 0; j < G::VU; ++j) load_value_unit(rv, L0, j);
#pragma unroll
        for (int i = 0; i < G::KBLK; ++i) load_key_block(rk, L0, pb0, i);
        if constexpr (MODE != kWideStatePass) {
            const __amdgpu_buffer_rsrc_t rq = q_rsrc(t_begin, L0);
#pragma unroll
            for (int i = 0; i < G::KSQ; ++i) load_q_unit(rq, L0, i);
            // the per-chunk wait before barrier A counts the operations issued after
            // a chunk's key loads in the loop; the first chunk's are waited for here
            wait_vm_lgkm0<0>();
#pragma unroll
            for (int j = 0; j < G::VU; ++j) scale_value_unit(j, 0);
        }
    }
    const float* s_in = nullptr;
    if constexpr (MODE == kWideSegPass)
        s_in = a.agg + (static_cast<size_t>(bh) * a.nseg + seg) * DK * a.dv;
    else if constexpr (MODE == kWideWhole)
        s_in = a.state_in ? a.state_in + static_cast<size_t>(bh) * DK * a.dv : nullptr;
    bool have_state = s_in != nullptr;
    if (have_state) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = d0 + mt * 16 + grp * 4 + r;
                    const int c = vt * kWideDvt + nt * 16 + l16;
                    sacc[mt][nt][r] = s_in[static_cast<size_t>(d) * a.dv + c];
                }
        write_state_copy(pb1);  // read after barrier A
    } else {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) sacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int tau0 = 0;  // group offset of the current chunk's first token
    // One chunk: its keys in kb (loaded during the previous chunk), the state
    // copy in sb, its values scaled in vst.
    auto chunk = [&](int ch, u16* __restrict__ kb, u16* __restrict__ sb) __attribute__((always_inline)) {
        const int t0 = t_begin + ch * C;
        const int L = min(C, t_end - t0);
        const bool has_next = ch + 1 < nch;
        const int t1 = has_next ? t0 + C : t0;  // past the end: a discarded re-read
        const int L1 = has_next ? min(C, t_end - t1) : L;
        refresh_lane();

        write_values();
        // A: this chunk's keys have landed (issued after them, in program order:
        // the previous chunk's output stores and the queries, both during its G4;
        // every chunk issues the same operations, past the end as re-reads);
        // V3 and the state copy are written
        wait_vm_lgkm0<G::KSQ + G::NTV>();
        __builtin_amdgcn_s_barrier();

        // ---- G3: O^T = A^T Q^T (the state before this chunk); the next chunk's values load meanwhile
#pragma unroll
        for (int nt = 0; nt < G::NTV; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const __amdgpu_buffer_rsrc_t rv = value_rsrc(t1, L1);
        if (have_state) {
            const FragAddr<UK> fs(l16, grp);  // A^T rows 16 nt + l16, d_k 32 s + 8 grp
            // step j: d_k step s = j / NTV, column tile nt = j % NTV
            constexpr int NS3 = G::KSQ * G::NTV;
            pipelined<NS3, kPipeDepth>(
                [&](auto j) __attribute__((always_inline)) {
                    constexpr int s = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                    return *reinterpret_cast<const uint4*>(&sb[fs.at(nt, s)]);
                },
                [&](auto j, const uint4& af) __attribute__((always_inline)) {
                    constexpr int s = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                    oacc[nt] = mfma16x16x32(af, qf[s], oacc[nt]);
                },
                [&](auto j) __attribute__((always_inline)) {
                    spread<G::VU, NS3, decltype(j)::value>([&](auto i) { load_value_unit(rv, L1, i); });
                });
        } else {
#pragma unroll
            for (int j = 0; j < G::VU; ++j) load_value_unit(rv, L1, j);
        }
        // every wave has read the state copy: the next chunk's keys go there
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();

        // ---- G1, G2 (the wave's blocks decide the causal extent)
        const __amdgpu_buffer_rsrc_t rk = key_rsrc(t1, L1);
        switch (qblk) {
            case 0: g12(kb, sb, rk, L1, Ic<0>{}); break;
            case 1: g12(kb, sb, rk, L1, Ic<1>{}); break;
            case 2: g12(kb, sb, rk, L1, Ic<2>{}); break;
            case 3: g12(kb, sb, rk, L1, Ic<3>{}); break;
            case 4: g12(kb, sb, rk, L1, Ic<4>{}); break;
            case 5: g12(kb, sb, rk, L1, Ic<5>{}); break;
            case 6: g12(kb, sb, rk, L1, Ic<6>{}); break;
            default: g12(kb, sb, rk, L1, Ic<7>{}); break;
        }

        // ---- G4, with the outputs O = gamma^(tau + 1) O^T stored as bf16 meanwhile
        const float z = fast_exp2(static_cast<float>(tau0 + 16 * qblk + l16 + 1) * lg2f);
        tau0 += L;
        const bool group_end = tau0 >= R * C || !has_next;
        g4(kb, out_rsrc(t0, L), L, q_rsrc(t1, L1), L1, z, group_end ? 0 : tau0);

        // ---- end of a decay group (or of the sequence): A back to S
        if (group_end) {
            // (no float64 in the loop: its exp2 constants would be held in registers)
            const float ge = tau0 == R * C ? g_group : fast_exp2(static_cast<float>(tau0) * lg2f);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[mt][nt][r] *= ge;
            tau0 = 0;
        }
        // B: every read of the keys and V3 done
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        write_state_copy(kb);
        have_state = true;
    };
    // State pass: per chunk only G4 (A += K^T V3) and the group-end scaling;
    // the next chunk's keys go into the other key buffer and its values into
    // registers during G4, and are scaled at the start of that chunk.
    auto state_chunk = [&](int ch, u16* __restrict__ kb, u16* __restrict__ nkb) __attribute__((always_inline)) {
        const int t0 = t_begin + ch * C;
        const int L = min(C, t_end - t0);
        const bool has_next = ch + 1 < nch;
        const int t1 = has_next ? t0 + C : t0;  // past the end: a discarded re-read
        const int L1 = has_next ? min(C, t_end - t1) : L;
        refresh_lane();
#pragma unroll
        for (int j = 0; j < G::VU; ++j) scale_value_unit(j, tau0);
        write_values();
        // A: this chunk's keys have landed (nothing else is in flight), V3 is written
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        const __amdgpu_buffer_rsrc_t rk = key_rsrc(t1, L1), rv = value_rsrc(t1, L1);
        struct F4 {
            uint4 v;
            uint4 k[G::MT];
        };
        uint4 kt[G::MT];
        constexpr int NS4 = 4 * G::NTV;
        pipelined<NS4, kPipeDepth>(
            [&](auto j) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                F4 f;
                f.v = tr_frag(vbuf, Ic<kWideDvt>{}, 16 * nt, t);
                if constexpr (nt == 0) {
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt) f.k[mt] = tr_frag(kb, Ic<DK>{}, d0 + 16 * mt, t);
                }
                return f;
            },
            [&](auto j, const F4& f) __attribute__((always_inline)) {
                constexpr int nt = decltype(j)::value % G::NTV;
                if constexpr (nt == 0) {
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt) kt[mt] = f.k[mt];
                }
#pragma unroll
                for (int mt = 0; mt < G::MT; ++mt) sacc[mt][nt] = mfma16x16x32(kt[mt], f.v, sacc[mt][nt]);
            },
            [&](auto j) __attribute__((always_inline)) {
                constexpr int J = decltype(j)::value;
                spread<G::KBLK, NS4, J>([&](auto i) { load_key_block(rk, L1, nkb, i); });
                spread<G::VU, NS4, J>([&](auto i) { load_value_unit(rv, L1, decltype(i)::value); });
            });
        tau0 += L;
        if (tau0 >= R * C || !has_next) {
            const float ge = tau0 == R * C ? g_group : fast_exp2(static_cast<float>(tau0) * lg2f);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[mt][nt][r] *= ge;
            tau0 = 0;
        }
        // B: every read of the keys and V3 done
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
    };
    if constexpr (MODE == kWideStatePass) {
        for (int ch = 0; ch < nch; ch += 2) {
            state_chunk(ch, pb0, pb1);
            if (ch + 1 < nch) state_chunk(ch + 1, pb1, pb0);
        }
    } else {
        for (int ch = 0; ch < nch; ch += 2) {
            chunk(ch, pb0, pb1);
            if (ch + 1 < nch) chunk(ch + 1, pb1, pb0);
        }
    }
    // the last chunk's discarded re-reads (into LDS among them) end before the workgroup does
    wait_vm_lgkm0<0>();

    float* s_dst = nullptr;
    if constexpr (MODE == kWideStatePass)
        s_dst = a.agg + (static_cast<size_t>(bh) * a.nseg + seg + 1) * DK * a.dv;
    else if (a.state_out && (MODE == kWideWhole || seg == a.nseg - 1))
        s_dst = a.state_out + static_cast<size_t>(bh) * DK * a.dv;
    if (s_dst) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = d0 + mt * 16 + grp * 4 + r;
                    const int c = vt * kWideDvt + nt * 16 + l16;
                    s_dst[static_cast<size_t>(d) * a.dv + c] = sacc[mt][nt][r];
                }
    }
}

}  // namespace

template <int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void chunk_wide_kernel(ChunkArgs a, HeadParams hp) {
    // (batch, head, value tile); the value tiles of one head run on one XCD
    const int chain = xcd_logical_block(blockIdx.x, gridDim.x);
    chunk_wide_body<DK, false>(a, hp, chain, 0);
}

// Segmented calls (few chains: the sequence is cut into a.nseg segments so the
// grid fills the chip): workgroup b serves chain b % chains, segment b / chains.
template <int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void chunk_wide_state_kernel(ChunkArgs a, HeadParams hp) {
    const int chains = a.B * a.H * a.nvt;
    const int b = blockIdx.x;
    chunk_wide_body<DK, false, kWideStatePass>(a, hp, b % chains, b / chains);
}

template <int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void chunk_wide_seg_kernel(ChunkArgs a, HeadParams hp) {
    const int chains = a.B * a.H * a.nvt;
    const int b = blockIdx.x;
    chunk_wide_body<DK, false, kWideSegPass>(a, hp, b % chains, b / chains);
}

// Several calls of one key width in one launch (the backward's passes):
// workgroups [first[c], first[c+1]) of the XCD-ordered block index serve call c.
template <int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void chunk_wide_multi_kernel(ChunkCalls cs, HeadParams hp) {
    const int b = xcd_logical_block(blockIdx.x, gridDim.x);
    int c = 0;
    while (c + 1 < cs.n && b >= cs.first[c + 1]) ++c;
    chunk_wide_body<DK, true>(cs.a[c], hp, b - cs.first[c], 0);
}

// Segmented calls of several passes (the backward's) in one launch per phase:
// workgroups [first[c], first[c+1]) serve call c, chain local % chains,
// segment local / chains.
template <int DK, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(kWideThreads, kWideThreads), amdgpu_waves_per_eu(2, 2)))
void chunk_wide_multi_seg_kernel(ChunkCalls cs, HeadParams hp) {
    const int b = blockIdx.x;
    int c = 0;
    while (c + 1 < cs.n && b >= cs.first[c + 1]) ++c;
    const int chains = cs.a[c].B * cs.a[c].H * cs.a[c].nvt;
    const int local = b - cs.first[c];
    chunk_wide_body<DK, true, MODE>(cs.a[c], hp, local % chains, local / chains);
}

// Chunks per decay group: the largest R in {8, 4, 2, 1} with gamma^(R C) >=
// 2^-64 for every head (0: the rescaled form does not fit these gammas).
int chunk_wide_rescale(const HeadParams& hp, int H) {
    double worst = 0.0;
    for (int h = 0; h < H; ++h) worst = std::fmin(worst, std::log2(static_cast<double>(hp.gamma[h])));
    for (int R = 8; R >= 1; R /= 2)
        if (worst * R * kWideC >= -64.0) return R;
    return 0;
}

bool chunk_wide_supported(int dk, int dvt, int chunk, bool rotation) {
    return !rotation && dvt == kWideDvt && chunk == kWideC && (dk == 128 || dk == 256);
}

hipError_t launch_chunk_wide_multi(const ChunkCalls& in, const HeadParams& hp, hipStream_t st) {
    if (in.n < 1 || in.n > kMaxChunkCalls) return hipErrorInvalidValue;
    ChunkCalls cs = in;
    const int R = chunk_wide_rescale(hp, cs.a[0].H);
    if (R == 0) return hipErrorInvalidValue;
    // every call whole (one pass per chain) or every call segmented (state pass,
    // scan, segment pass per call, each phase one launch for all calls)
    const bool seg = cs.a[0].nseg > 1;
    for (int i = 0; i < cs.n; ++i) {
        ChunkArgs& b = cs.a[i];
        if (b.dk != cs.a[0].dk || b.H != cs.a[0].H || !chunk_wide_supported(b.dk, b.dv / b.nvt, b.chunk, false) ||
            b.orot || (b.nseg > 1) != seg || (seg && (!b.agg || b.seg_len % kWideC != 0)))
            return hipErrorInvalidValue;
        b.rescale = R;
    }
    cs.interleave = 0;
    const dim3 block(kWideThreads);
    auto ranges = [&](int extra) {  // workgroups per call: chains x (nseg + extra)
        cs.first[0] = 0;
        for (int i = 0; i < cs.n; ++i)
            cs.first[i + 1] = cs.first[i] + cs.a[i].B * cs.a[i].H * cs.a[i].nvt * (seg ? cs.a[i].nseg + extra : 1);
        return dim3(cs.first[cs.n]);
    };
    if (!seg) {
        const dim3 grid = ranges(0);
        if (cs.a[0].dk == 256)
            hipLaunchKernelGGL(chunk_wide_multi_kernel<256>, grid, block, 0, st, cs, hp);
        else
            hipLaunchKernelGGL(chunk_wide_multi_kernel<128>, grid, block, 0, st, cs, hp);
        return hipGetLastError();
    }
    dim3 grid = ranges(-1);
    if (cs.a[0].dk == 256)
        hipLaunchKernelGGL((chunk_wide_multi_seg_kernel<256, kWideStatePass>), grid, block, 0, st, cs, hp);
    else
        hipLaunchKernelGGL((chunk_wide_multi_seg_kernel<128, kWideStatePass>), grid, block, 0, st, cs, hp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_segment_scan_multi(cs, hp, st);
    if (e != hipSuccess) return e;
    grid = ranges(0);
    if (cs.a[0].dk == 256)
        hipLaunchKernelGGL((chunk_wide_multi_seg_kernel<256, kWideSegPass>), grid, block, 0, st, cs, hp);
    else
        hipLaunchKernelGGL((chunk_wide_multi_seg_kernel<128, kWideSegPass>), grid, block, 0, st, cs, hp);
    return hipGetLastError();
}

// ev: six events (start / stop of the state pass, the scan and the segment or
// whole pass), or null.
hipError_t launch_chunk_wide(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev) {
    const int chains = a.B * a.H * a.nvt;
    const dim3 block(kWideThreads);
    if (a.nseg <= 1) {
        record_empty_phase(st, ev);
        record_empty_phase(st, ev ? ev + 2 : nullptr);
        const dim3 grid(chains);
        if (a.dk == 256)
            launch_timed(chunk_wide_kernel<256>, grid, block, 0, st, ev ? ev + 4 : nullptr, a, hp);
        else
            launch_timed(chunk_wide_kernel<128>, grid, block, 0, st, ev ? ev + 4 : nullptr, a, hp);
        return hipGetLastError();
    }
    // segments: end states from zero, their scan (float32 [B*H][nseg][d_k][d_v] in the
    // workspace's state region), then every segment's outputs from its start state
    if (!a.agg || a.rev || a.seg_len % kWideC != 0) return hipErrorInvalidValue;
    const dim3 gs(chains * (a.nseg - 1)), gm(chains * a.nseg);
    if (a.dk == 256)
        launch_timed(chunk_wide_state_kernel<256>, gs, block, 0, st, ev, a, hp);
    else
        launch_timed(chunk_wide_state_kernel<128>, gs, block, 0, st, ev, a, hp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_segment_scan(a, hp, st, ev ? ev + 2 : nullptr);
    if (e != hipSuccess) return e;
    if (a.dk == 256)
        launch_timed(chunk_wide_seg_kernel<256>, gm, block, 0, st, ev ? ev + 4 : nullptr, a, hp);
    else
        launch_timed(chunk_wide_seg_kernel<128>, gm, block, 0, st, ev ? ev + 4 : nullptr, a, hp);
    return hipGetLastError();
}

}  // namespace ret
