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
#include "wide.hpp"

#include <cmath>
#include <type_traits>

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
    // When the key and value blocks together need no more than one block per
    // thread, the value blocks go to the threads the key blocks leave free
    // (threads VOFF..), so staging work is spread over every wave.
    static constexpr int VOFF = (KB + VB <= NTHR) ? KB : 0;
    static_assert(C == 32 || C == 64 || C == 128, "chunk");
    static_assert(DK % 64 == 0 && DVT % 64 == 0, "tile sizes");
    static_assert(MG * MT == TM && NG * NT == NTV, "state split");
};

// Index of thread t among the value-staging threads (see ChunkGeo::VOFF);
// threads without a value block get an index >= VB.
template <typename G>
__device__ __forceinline__ int value_thread(int t) {
    return t >= G::VOFF ? t - G::VOFF : t + G::NTHR - G::VOFF;
}

// Row block owned by wave w: waves w and w + NW/2 (which the dispatcher puts
// on the same SIMD) get blocks b and NW-1-b, so the causal work per SIMD is
// the same for every SIMD.
template <int NW>
__device__ __forceinline__ int wave_row_block(int w) {
    return w < NW / 2 ? w : (3 * NW / 2 - 1) - w;
}

// Segmented form: the workgroups of one (batch, head, value tile) chain split
// its sequence into segments and pass states along the chain with a look-back,
// all inside one launch:
//   1. Workgroups take tickets from their chain's counter in the workspace;
//      ticket order is segment order, so every segment a workgroup waits for
//      belongs to a workgroup that took its ticket earlier and is running.
//   2. Segment 0 publishes its end state P_0 (from the initial state); every
//      other segment but the last publishes T_s, its end state from a zero
//      start. Publishing never waits on anything.
//   3. Segment s >= 1 forms S_in(s) = sum_{0<j<s} g^(s-1-j) T_j + g^(s-1) P_0,
//      g = gamma^seg_len, from its group predecessors' states and one published
//      aggregate per earlier group of segments (see look_back), always in the
//      same order, so results are bitwise reproducible.
//   4. It runs its chunks from S_in(s) (or runs them from zero first and
//      corrects the held outputs by gamma^(n+1) q_n S_in(s), see kLocalPass).
// Every wait targets a workgroup that is running and publishes without
// waiting, so every wait ends; a spin bound backs this up (a look-back that
// exceeds it poisons the start state with NaN instead of hanging). A flag
// carries the chain's launch generation (the high half of its counter,
// advanced by the workgroup that draws the chain's last ticket) and the chain
// index, so no flag left by an earlier call, of any size, reads as published,
// and the workspace needs zero-filling only once, before its first use.
//
// Published states and flags move through device-coherent (agent-scope)
// loads and stores, which bypass the per-XCD L2 caches; a publisher waits
// for its state stores to complete before a barrier and the flag store. This
// avoids device-scope fences, which on this chip write back or invalidate
// a whole L2 and cost tens of microseconds under load.
constexpr unsigned kMaxLookbackSpins = 1u << 20;

constexpr int imax(int x, int y) { return x > y ? x : y; }

// Wait until this thread's global stores have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Kernel forms: one pass per (batch, head, value tile) chain; segmented with a
// state-only first pass; segmented with outputs held back (segments of at
// most kKeepChunks chunks).
enum ChunkMode { kSinglePass = 0, kTwoPass = 1, kLocalPass = 2 };
constexpr int kKeepChunks = 2;

// The body of one workgroup: `bid` is its index among the `nblk` workgroups of
// its call (the launch may carry several calls of the same shape). With REVM,
// a call whose `rev` is set reads and writes its rows in reverse token order:
// kernel token t is memory row N-1-t (rotation is not supported then).
template <int DK, int DVT, int C, int MODE, bool FAST, int REVM>
__device__ __forceinline__ void chunk_body(const ChunkArgs& a, const HeadParams& hp, unsigned bid, unsigned nblk) {
    constexpr bool SEGMENTED = MODE != kSinglePass;
    using G = ChunkGeo<DK, DVT, C>;
    constexpr int UK = DK / 8;  // 16-byte units in a row of K (row-major) and of S^T
    constexpr int UC = C / 8;   // 16-byte units in a row of K^T and V^T
    // the multi-call kernel's output rotation (a.orot, see store_o) keeps this
    // value tile's DVT/2 frequencies in float32 after the keys
    constexpr bool kORot = REVM != 0 && chunk_orot_fits(DK, DVT, C);
    __shared__ __attribute__((aligned(16))) u16 kbuf[C * DK + (kORot ? DVT : 0)];
    __shared__ __attribute__((aligned(16))) u16 vbuf[DVT * C];
    __shared__ __attribute__((aligned(16))) u16 sbuf[DVT * DK];
    float* s_oth = reinterpret_cast<float*>(kbuf + C * DK);
    // Broadcast slots of the segmented form (ticket, look-back status), overlaid
    // on sbuf: both are read before the first write of the state copy (a
    // barrier lies in between).
    unsigned long long* s_ticket = reinterpret_cast<unsigned long long*>(sbuf);
    int* s_lookback = reinterpret_cast<int*>(sbuf + 4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int grp = lane >> 4;

    // Rotation frequencies this thread applies (kernels with 64-token chunks,
    // see rotate_key_row): read before anything else, so the round trip to the
    // kernel arguments hides under the ticket and the first chunk's loads.
    constexpr bool kThetaRegs = C == 64;
    float thk[G::KPT][G::BWK / 2], thq[G::KSQ][4];
    if (kThetaRegs && hp.has_theta) {
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid + u * G::NTHR;
            int tb, cb;
            block_coords<DK, G::BWK, C / 8>(idx < G::KB ? idx : 0, tb, cb);
#pragma unroll
            for (int p = 0; p < G::BWK / 2; ++p) thk[u][p] = hp.theta[cb * (G::BWK / 2) + p];
        }
#pragma unroll
        for (int s = 0; s < G::KSQ; ++s)
#pragma unroll
            for (int p = 0; p < 4; ++p) thq[s][p] = hp.theta[s * 16 + grp * 4 + p];
    }

    // ---- which (batch*head, value tile) chain and segment this workgroup owns
    int chain, seg = 0;
    unsigned gen = 0;
    if constexpr (SEGMENTED) {
        const int nchains = a.B * a.H * a.nvt;
        chain = bid % static_cast<unsigned>(nchains);
        unsigned long long* ctl = a.ctl + static_cast<size_t>(chain) * kCtlStride;
        if (tid == 0) *s_ticket = __hip_atomic_fetch_add(ctl, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const unsigned long long tk = *s_ticket;
        const unsigned nseg = static_cast<unsigned>(a.nseg);
        seg = static_cast<int>(static_cast<unsigned>(tk) % nseg);
        gen = static_cast<unsigned>(tk >> 32);
        if (tid == 0 && static_cast<unsigned>(tk) == nseg - 1)  // chain's last ticket: reset count, next generation
            __hip_atomic_fetch_add(ctl, (1ull << 32) - nseg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        chain = xcd_logical_block(bid, nblk);
    }
    const int vt = chain % a.nvt;
    const int bh = chain / a.nvt;
    const int h = bh % a.H;
    if constexpr (kORot) {  // the column pairs of this value tile; read after later barriers
        if (a.orot && tid < DVT / 2) s_oth[tid] = hp.theta[vt * (DVT / 2) + tid];
    }

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
    const bool rev = REVM != 0 && a.rev != 0;
    // first memory row of the chunk at kernel token t with L valid rows (at
    // least one, so a discarded re-read past the end stays inside the sequence)
    auto mrow0 = [&](int t, int L) __attribute__((always_inline)) { return rev ? a.N - t - max(L, 1) : t; };

    const int rb = wave_row_block<G::NW>(wave);      // this wave's 16 chunk rows
    const int d_base = (wave % G::MG) * G::MT * 16;  // this wave's S rows ...
    const int c_base = (wave / G::MG) * G::NT * 16;  // ... and S columns (within the value tile)

    BlockRows<G::BWK> kr[G::KPT];
    BlockRows<G::BWV> vr[G::VPT];
    uint4 qf[G::KSQ];
    f32x4 sacc[G::MT][G::NT];

    // queries of this wave's rows: unconditional loads (a wave-uniform base plus
    // a 32-bit per-lane byte offset, like every global access of the chunk
    // loop: no 64-bit per-lane pointers to keep). Rows past the end of the
    // segment read the last valid row instead; they only feed output rows
    // that are never stored, so they need no zeroing (a select here would be
    // turned into branches around the loads).
    auto load_q = [&](uint4 (&qd)[G::KSQ], int t, int Lq) __attribute__((always_inline)) {
        const int lastq = Lq > 0 ? Lq - 1 : 0;
        const int rc = rev ? lastq - min(rb * 16 + l16, lastq) : min(rb * 16 + l16, lastq);
        const char* base = reinterpret_cast<const char*>(Qg + static_cast<size_t>(mrow0(t, Lq)) * DK);
        const uint32_t off = static_cast<uint32_t>((rc * DK + grp * 8) * 2);
#pragma unroll
        for (int s = 0; s < G::KSQ; ++s) qd[s] = *reinterpret_cast<const uint4*>(base + off + s * 64);
    };
    // first chunk of the segment (issued before state loads so the HBM round trips overlap)
    auto prefetch_first = [&](bool with_q) __attribute__((always_inline)) {
        const int L0 = min(C, t_end - t_begin);
        load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(kr, Kg + static_cast<size_t>(mrow0(t_begin, L0)) * DK, DK,
                                                        L0, tid, rev);
        load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vr, Vg + static_cast<size_t>(mrow0(t_begin, L0)) * a.dv,
                                                          a.dv, L0, value_thread<G>(tid), rev);
        if (with_q) load_q(qf, t_begin, L0);
    };
    // this head's state from a caller's [B*H][dk][dv] float32 array, or zeros
    auto load_state_to = [&](f32x4 (&dst)[G::MT][G::NT], const float* states) __attribute__((always_inline)) {
        const float* src = states ? states + static_cast<size_t>(bh) * DK * a.dv : nullptr;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = d_base + mt * 16 + grp * 4 + r;
                    const int c = vt * DVT + c_base + nt * 16 + l16;
                    dst[mt][nt][r] = src ? src[static_cast<size_t>(d) * a.dv + c] : 0.0f;
                }
    };
    auto load_state = [&](const float* states) __attribute__((always_inline)) { load_state_to(sacc, states); };
    // bf16 copy of this wave's state tiles into S^T (row = value column, 4 consecutive dk)
    auto write_state_copy_of = [&](const f32x4 (&st)[G::MT][G::NT], int l16_, int grp_) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt) {
                const int d = d_base + mt * 16 + grp_ * 4;
                const int c = c_base + nt * 16 + l16_;
                const uint2 w = make_uint2(pack2_bf16(st[mt][nt][0], st[mt][nt][1]),
                                           pack2_bf16(st[mt][nt][2], st[mt][nt][3]));
                *reinterpret_cast<uint2*>(&sbuf[swz<UK>(c, d >> 3) + (d & 7)]) = w;
            }
    };
    auto write_state_copy = [&](int l16_, int grp_) __attribute__((always_inline)) {
        write_state_copy_of(sacc, l16_, grp_);
    };

    // ---- per-lane decay constants
    // D[i][j] = gamma^(i-j) with i = 16 rb + l16, j = 16 jt + 4 grp + r, with no
    // factor at a negative exponent (small gammas would overflow it):
    //   diagonal tile (jt = rb): dlane[r] = gamma^(l16 - 4 grp - r), negative
    //     exponents only in masked entries, which are selected away;
    //   jt < rb: dlane15[r] * gamma^(16 (rb - jt) - 15), dlane15[r] =
    //     gamma^(l16 - 4 grp - r + 15).
    float dlane[4], dlane15[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        dlane[r] = fast_exp2(static_cast<float>(l16 - 4 * grp - r) * lg2f);
        dlane15[r] = FAST ? 0.0f : fast_exp2(static_cast<float>(l16 - 4 * grp - r + 15) * lg2f);
    }
    const float zeta = fast_exp2(static_cast<float>(16 * rb + l16 + 1) * lg2f);
    const float gC = gamma_pow(lg2, C);
    bool have_state = false;

    // Rotation of this thread's key staging columns and query units. Kernels
    // with 64-token chunks hold the frequencies in registers (thk, thq, loaded
    // at the start) and rotate by angle addition: once per chunk, the angle of
    // the chunk's first position is reduced in float64 (b = frac(t0 w), in
    // revolutions, w = theta / 2 pi); each row at offset k then turns by
    // b + k w, formed and reduced in float32 (|k w| < 11 revolutions, error
    // ~1e-6 rad), so the per-row work has no float64. The other kernels reduce
    // each row's angle in float64 (their registers are short).
    float bk[G::KPT][G::BWK / 2], bq[G::KSQ][4];
    constexpr float kInvTwoPiF = 0.15915494309189533577f;
    // the chunk's base angles (position pos0 + t0), once per chunk
    auto theta_bases = [&](int t0) __attribute__((always_inline)) {
        if constexpr (kThetaRegs) {
            constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
            const double p0 = static_cast<double>(a.pos0 + t0);
            auto frac = [&](float th) __attribute__((always_inline)) {
                const double x = p0 * (static_cast<double>(th) * kInvTwoPi);
                return static_cast<float>(x - rint(x));
            };
#pragma unroll
            for (int u = 0; u < G::KPT; ++u)
#pragma unroll
                for (int p = 0; p < G::BWK / 2; ++p) bk[u][p] = frac(thk[u][p]);
#pragma unroll
            for (int s = 0; s < G::KSQ; ++s)
#pragma unroll
                for (int p = 0; p < 4; ++p) bq[s][p] = frac(thq[s][p]);
        }
    };
    // rotate the pairs of x by revolutions base[p] + k step[p]
    auto rotate_pairs_rev = [&](uint32_t* w, int n, const float* base, const float* th, float k)
                                __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < n; ++p) {
            float r = fmaf(k, th[p] * kInvTwoPiF, base[p]);
            r -= rintf(r);
            const float sn = __builtin_amdgcn_sinf(r), cs = __builtin_amdgcn_cosf(r);
            const float re = lo_bf16(w[p]), im = hi_bf16(w[p]);
            w[p] = pack2_bf16(re * cs - im * sn, re * sn + im * cs);
        }
    };
    // key row at token t0 + k of staging block u (columns of block column cb)
    auto rotate_key_row = [&](uint32_t (&w)[G::BWK / 2], int u, int cb, int t0, int k) __attribute__((always_inline)) {
        if constexpr (kThetaRegs)
            rotate_pairs_rev(w, G::BWK / 2, bk[u], thk[u], static_cast<float>(k));
        else
            rotate_row<G::BWK>(w, hp, cb * (G::BWK / 2), static_cast<double>(a.pos0 + t0 + k));
    };
    // query unit s (8 bf16 = 4 pairs) of the row at token t0 + k
    auto rotate_query_unit = [&](uint4 x, int s, int t0, int k) __attribute__((always_inline)) {
        if constexpr (kThetaRegs) {
            uint32_t w[4] = {x.x, x.y, x.z, x.w};
            rotate_pairs_rev(w, 4, bq[s], thq[s], static_cast<float>(k));
            return make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            return rotate8_bf16(x, hp, s * 16 + grp * 4, static_cast<double>(a.pos0 + t0 + k));
        }
    };

    // ---- pieces of the chunk loop
    // Step 7: this wave's 16 output rows of the chunk at token t0 (L valid), as bf16.
    // With a.orot, each row is first rotated by minus theta at its token's
    // position: the lane's columns 16 nt + 4 grp .. +3 are pairs 8 nt + 2 grp
    // and 8 nt + 2 grp + 1 of the tile (frequencies from LDS, so no global load
    // sits behind the branch).
    auto store_o = [&](const f32x4 (&o)[G::NTV], int t0, int L) __attribute__((always_inline)) {
        const int row = rev ? L - 1 - (rb * 16 + l16) : rb * 16 + l16;
        if (rb * 16 + l16 < L) {
            char* base = reinterpret_cast<char*>(Og + static_cast<size_t>(mrow0(t0, L)) * a.dv);
            const uint32_t off = static_cast<uint32_t>((row * a.dv + grp * 4) * 2);
            f32x4 x[G::NTV];
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) x[nt] = o[nt];
            if constexpr (kORot) {
                if (a.orot) {
                    const double position = static_cast<double>(a.pos0 + mrow0(t0, L) + row);
#pragma unroll
                    for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                        for (int p = 0; p < 2; ++p) {
                            float c, sn;
                            rot_cs_fast(position, -s_oth[nt * 8 + grp * 2 + p], c, sn);
                            const float re = x[nt][2 * p], im = x[nt][2 * p + 1];
                            x[nt][2 * p] = re * c - im * sn;
                            x[nt][2 * p + 1] = re * sn + im * c;
                        }
                }
            }
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) {
                const uint2 w = make_uint2(pack2_bf16(x[nt][0], x[nt][1]), pack2_bf16(x[nt][2], x[nt][3]));
                *reinterpret_cast<uint2*>(base + off + nt * 32) = w;
            }
        }
    };
    // Step 1: rotate the chunk's keys; K^T (scaled by xi) and V^T into LDS.
    auto stage_kv = [&](auto& krb, auto& vrb, int t0, int L, int tid_it, float lg2c) __attribute__((always_inline)) {
        if (hp.has_theta) theta_bases(t0);  // also used by the queries of this chunk
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid_it + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK, G::BWK, C / 8>(idx, tb, cb);
                if (hp.has_theta) {  // rows past the end are zero: rotating them is harmless
#pragma unroll
                    for (int q = 0; q < 8; ++q) rotate_key_row(krb[u].w[q], u, cb, t0, staged_token(tb, q));
                }
                float xi[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) xi[q] = fast_exp2(static_cast<float>(L - 1 - staged_token(tb, q)) * lg2c);
#pragma unroll
                for (int c = 0; c < G::BWK; ++c) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float lo = bf16_to_f32(static_cast<u16>(elem16(krb[u].w[2 * p], c))) * xi[2 * p];
                        const float hi = bf16_to_f32(static_cast<u16>(elem16(krb[u].w[2 * p + 1], c))) * xi[2 * p + 1];
                        w[p] = pack2_bf16(lo, hi);
                    }
                    *reinterpret_cast<uint4*>(&kbuf[swz<UC>(cb * G::BWK + c, tb)]) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G::VPT; ++u) {
            const int idx = value_thread<G>(tid_it) + u * G::NTHR;
            if (idx < G::VB) {
                int tb, cb;
                block_coords<DVT, G::BWV, C / 8>(idx, tb, cb);
#pragma unroll
                for (int c = 0; c < G::BWV; ++c)
                    *reinterpret_cast<uint4*>(&vbuf[swz<UC>(cb * G::BWV + c, tb)]) = block_column(vrb[u], c);
            }
        }
    };
    // K and V of the chunk starting at token t (L valid tokens) into staging
    // registers (tid_it: the thread index, an opaque per-chunk copy inside the
    // chunk loops, so the per-row offsets are recomputed instead of being held
    // in registers across the loop).
    auto load_kv = [&](auto& krb, auto& vrb, int t, int L, int tid_it) __attribute__((always_inline)) {
        load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR>(krb, Kg + static_cast<size_t>(mrow0(t, L)) * DK, DK, L,
                                                        tid_it, rev);
        load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR>(vrb, Vg + static_cast<size_t>(mrow0(t, L)) * a.dv, a.dv, L,
                                                          value_thread<G>(tid_it), rev);
    };
    // Rows R0 .. R1-1 of every staging block of those loads (one chunk's loads
    // can be spread over several points of the loop).
    auto load_kv_rows = [&](auto& krb, auto& vrb, int t, int L, int tid_it, auto r0_tag, auto r1_tag)
                            __attribute__((always_inline)) {
        constexpr int R0 = decltype(r0_tag)::value, R1 = decltype(r1_tag)::value;
        load_blocks<DK, G::BWK, G::KB, G::KPT, G::NTHR, R0, R1>(krb, Kg + static_cast<size_t>(mrow0(t, L)) * DK, DK,
                                                                L, tid_it, rev);
        load_blocks<DVT, G::BWV, G::VB, G::VPT, G::NTHR, R0, R1>(vrb, Vg + static_cast<size_t>(mrow0(t, L)) * a.dv,
                                                                a.dv, L, value_thread<G>(tid_it), rev);
    };
    // Step 3 (G4): S = gamma^L S + Kx^T V on this wave's tiles.
    auto g4 = [&](int L, int l16c, int grpc) __attribute__((always_inline)) {
        const float gL = (L == C) ? gC : fast_exp2(static_cast<float>(L) * lg2f);  // no float64 in the loop
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
    };

    // ---- the FAST form's pieces (see the kernel comment): keys row-major only,
    //      values scaled by gamma^-(j+1) on their way into V''^T.
    auto stage_fast = [&](auto& krb, auto& vrb, int t0, int L, int tid_it, float lg2c) __attribute__((always_inline)) {
        if (hp.has_theta) theta_bases(t0);  // also used by the queries of this chunk
#pragma unroll
        for (int u = 0; u < G::KPT; ++u) {
            const int idx = tid_it + u * G::NTHR;
            if (idx < G::KB) {
                int tb, cb;
                block_coords<DK, G::BWK, C / 8>(idx, tb, cb);
                if (hp.has_theta) {  // rows past the end are zero: rotating them is harmless
#pragma unroll
                    for (int q = 0; q < 8; ++q) rotate_key_row(krb[u].w[q], u, cb, t0, staged_token(tb, q));
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int row = staged_token(tb, q);
                    if constexpr (G::BWK == 8) {
                        *reinterpret_cast<uint4*>(&kbuf[swz<UK>(row, cb)]) =
                            make_uint4(krb[u].w[q][0], krb[u].w[q][1], krb[u].w[q][2], krb[u].w[q][3]);
                    } else {
                        *reinterpret_cast<uint2*>(&kbuf[swz<UK>(row, cb >> 1) + 4 * (cb & 1)]) =
                            make_uint2(krb[u].w[q][0], krb[u].w[q][1]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G::VPT; ++u) {
            const int idx = value_thread<G>(tid_it) + u * G::NTHR;
            if (idx < G::VB) {
                int tb, cb;
                block_coords<DVT, G::BWV, C / 8>(idx, tb, cb);
                float f[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) f[q] = fast_exp2(-static_cast<float>(staged_token(tb, q) + 1) * lg2c);
#pragma unroll
                for (int c = 0; c < G::BWV; ++c) {
                    uint32_t w[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const float lo = bf16_to_f32(static_cast<u16>(elem16(vrb[u].w[2 * p], c))) * f[2 * p];
                        const float hi = bf16_to_f32(static_cast<u16>(elem16(vrb[u].w[2 * p + 1], c))) * f[2 * p + 1];
                        w[p] = pack2_bf16(lo, hi);
                    }
                    *reinterpret_cast<uint4*>(&vbuf[swz<UC>(cb * G::BWV + c, tb)]) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    };
    // G4 of the FAST form: S = gamma^L (S + K^T V''). The K^T operand comes from
    // the row-major keys by transposing reads: lane (grp, r) points at token
    // 32 t + 4 grp + r/4 (+16), dk columns 4 (r%4) .. +3 of its tile, and
    // receives dk row l16 at tokens 32 t + 4 grp + {0..3} (+16): the token
    // order of the V''^T units.
    auto g4_fast = [&](int L, int l16c, int grpc) __attribute__((always_inline)) {
        const float gL = (L == C) ? gC : fast_exp2(static_cast<float>(L) * lg2f);  // no float64 in the loop
        const int tok = 4 * grpc + (l16c >> 2);
        int kb[G::MT];
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt) {
            const int d = d_base + 16 * mt + 4 * (l16c & 3);
            kb[mt] = swz<UK>(tok, d >> 3) + (d & 7);
        }
        const FragAddr<UC> fa_vt(c_base + l16c, grpc);  // V''^T rows c_base + 16 nt + l16, unit 4 t + grp
#pragma unroll
        for (int t = 0; t < G::KST; ++t) {
            if (t * 32 < L) {
                uint4 af[G::MT];
#pragma unroll
                for (int mt = 0; mt < G::MT; ++mt) {
                    const uint2 lo = lds_read_tr16x4(&kbuf[kb[mt] + (32 * t) * (UK * 8)]);
                    const uint2 hi = lds_read_tr16x4(&kbuf[kb[mt] + (32 * t + 16) * (UK * 8)]);
                    af[mt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt) {
                    const uint4 bfr = *reinterpret_cast<const uint4*>(&vbuf[fa_vt.at(nt, t)]);
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt) sacc[mt][nt] = mfma16x16x32(af[mt], bfr, sacc[mt][nt]);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[mt][nt][r] *= gL;
    };

    // The state recurrence alone over this segment (keys and values only), with
    // two chunks of loads in flight: chunk ch + 2 is fetched into the registers
    // chunk ch has just been staged from, under G4 of chunk ch.
    BlockRows<G::BWK> kr2[G::KPT];
    BlockRows<G::BWV> vr2[G::VPT];
    auto run_state_only = [&]() __attribute__((always_inline)) {
        load_kv(kr2, vr2, nch > 1 ? t_begin + C : t_begin, nch > 1 ? min(C, t_end - t_begin - C) : 0, tid);
        auto step = [&](auto& krb, auto& vrb, int ch) __attribute__((always_inline)) {
            // per-iteration opaque copies: see run_chunks
            int tid_it = tid;
            float lg2_it = lg2f;
            asm volatile("" : "+v"(tid_it), "+v"(lg2_it));
            const int t0 = t_begin + ch * C;
            const int L = min(C, t_end - t0);
            if constexpr (FAST)
                stage_fast(krb, vrb, t0, L, tid_it, lg2_it);
            else
                stage_kv(krb, vrb, t0, L, tid_it, lg2_it);
            const bool far = ch + 2 < nch;
            load_kv(krb, vrb, far ? t0 + 2 * C : t0, far ? min(C, t_end - t0 - 2 * C) : 0, tid_it);
            __syncthreads();  // keys and values written
            if constexpr (FAST)
                g4_fast(L, tid_it & 15, (tid_it & 63) >> 4);
            else
                g4(L, tid_it & 15, (tid_it & 63) >> 4);
            __syncthreads();  // keys and values read
        };
        for (int ch = 0; ch < nch; ch += 2) {
            step(kr, vr, ch);
            if (ch + 1 < nch) step(kr2, vr2, ch + 1);
        }
    };

    // The full chunk loop over this segment: outputs and state. With KEEP the
    // outputs stay in registers (with the rotated queries) instead of going to
    // HBM: the segment was started from a zero state and is corrected once its
    // start state is known.
    f32x4 oacc_keep[kKeepChunks][G::NTV];
    uint4 qf_keep[kKeepChunks][G::KSQ];
    auto run_chunks = [&](auto keep_tag) __attribute__((always_inline)) {
        constexpr bool KEEP = decltype(keep_tag)::value;
        auto body = [&](int ch, uint4 (&qfb)[G::KSQ], uint4 (&qnext)[G::KSQ]) __attribute__((always_inline)) {
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

            // ---- 1. K^T (scaled by xi) and V^T into LDS
            stage_kv(kr, vr, t0, L, tid_it, lg2c);
            __syncthreads();  // A: K^T, V^T written
            // rotate the queries (after the barrier: their loads land under the staging)
            if (hp.has_theta) {  // every row: those past the end are never stored
                const int row = rb * 16 + l16;
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s) qfb[s] = rotate_query_unit(qfb[s], s, t0, row);
            }

            // ---- 2. G3: O^T = S^T Q^T with the previous chunk's state, times zeta
            f32x4 oacc[G::NTV];
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (have_state) {
                const FragAddr<UK> fa_s(l16c, grpc);  // S^T rows 16 nt + l16, dk 32 s + 8 grp
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) {
#pragma unroll
                    for (int s = 0; s < G::KSQ; ++s) {
                        const uint4 af = *reinterpret_cast<const uint4*>(&sbuf[fa_s.at(nt, s)]);
                        oacc[nt] = mfma16x16x32(af, qfb[s], oacc[nt]);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) oacc[nt][r] *= zeta;
            }

            // ---- 3. G4: S = gamma^L S + Kx^T V on this wave's tiles
            g4(L, l16c, grpc);
            __syncthreads();  // B: S^T and K^T reads done

            // ---- 4. new bf16 state copy, K row-major into LDS, prefetch next keys/values
            write_state_copy(l16c, grpc);
            have_state = true;
#pragma unroll
            for (int u = 0; u < G::KPT; ++u) {
                const int idx = tid_it + u * G::NTHR;
                if (idx < G::KB) {
                    int tb, cb;
                    block_coords<DK, G::BWK, C / 8>(idx, tb, cb);
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
            load_kv(kr, vr, has_next ? t1 : t0, L1, tid_it);  // past the end: a discarded re-read
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
                                pa[hh] = mfma16x16x32(af, qfb[s], pa[hh]);
                            }
                        }
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int delta = rb - (2 * t + hh);
                            const float blk = fast_exp2(static_cast<float>(16 * delta - 15) * lg2c);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                float val = 0.0f;
                                const float dec = delta == 0 ? dlane[r] : dlane15[r] * blk;
                                if (delta > 0 || (delta == 0 && l16 >= 4 * grp + r)) val = pa[hh][r] * dec;
                                pa[hh][r] = val;
                            }
                        }
                        pf[t] = make_uint4(pack2_bf16(pa[0][0], pa[0][1]), pack2_bf16(pa[0][2], pa[0][3]),
                                           pack2_bf16(pa[1][0], pa[1][1]), pack2_bf16(pa[1][2], pa[1][3]));
                    }
                }
            }

            // ---- prefetch next chunk's queries (qf is dead for this chunk now)
            load_q(qnext, has_next ? t1 : t0, L1);

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
            if constexpr (KEEP) {
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) oacc_keep[ch][nt] = oacc[nt];
            } else {
                store_o(oacc, t0, L);
            }
            __syncthreads();  // D: reads of kbuf and vbuf done before the next chunk's writes
        };
        // The FAST form of a chunk: two barriers. Staging writes row-major keys
        // and V''^T and issues the next chunk's loads (its registers are free);
        // one matrix-core phase reads LDS only: G3, G1, G2 into one accumulator,
        // the outputs (times gamma^(i+1)) are stored, then G4; after the second
        // barrier the new state copy is written.
        auto body_fast = [&](int ch, uint4 (&qfb)[G::KSQ], uint4 (&qnext)[G::KSQ]) __attribute__((always_inline)) {
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

            // ---- 1. keys row-major, V''^T into LDS; fetch the next chunk
            stage_fast(kr, vr, t0, L, tid_it, lg2c);
            // The next chunk's keys and values are fetched in three parts (half
            // now, a quarter before G1, a quarter with the queries after G1):
            // every workgroup reaches this point at about the same time, and
            // spreading the requests over the chunk keeps them from queueing
            // behind one another (past the end: discarded re-reads).
            using I0 = std::integral_constant<int, 0>;
            using I4 = std::integral_constant<int, 4>;
            using I6 = std::integral_constant<int, 6>;
            using I8 = std::integral_constant<int, 8>;
            load_kv_rows(kr, vr, has_next ? t1 : t0, L1, tid_it, I0{}, I4{});
            __syncthreads();  // A: keys and V''^T written
            // rotate the queries (after the barrier: their loads land under the staging)
            if (hp.has_theta) {  // every row: those past the end are never stored
                const int row = rb * 16 + l16;
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s) qfb[s] = rotate_query_unit(qfb[s], s, t0, row);
            }

            // ---- 2. G3: O^T = S^T Q^T (the previous chunk's state)
            f32x4 oacc[G::NTV];
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (have_state) {
                const FragAddr<UK> fa_s(l16c, grpc);  // S^T rows 16 nt + l16, dk 32 s + 8 grp
                // (s outer: consecutive MFMAs go to different accumulators)
#pragma unroll
                for (int s = 0; s < G::KSQ; ++s) {
#pragma unroll
                    for (int nt = 0; nt < G::NTV; ++nt) {
                        const uint4 af = *reinterpret_cast<const uint4*>(&sbuf[fa_s.at(nt, s)]);
                        oacc[nt] = mfma16x16x32(af, qfb[s], oacc[nt]);
                    }
                }
            }

            load_kv_rows(kr, vr, has_next ? t1 : t0, L1, tid_it, I4{}, I6{});
            // ---- 3. G1: P^T = K Q^T, causal mask on the diagonal tile only (the
            //         decay is carried by V'' and the final gamma^(i+1))
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
                                pa[hh] = mfma16x16x32(af, qfb[s], pa[hh]);
                            }
                        }
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int delta = rb - (2 * t + hh);
                            if (delta <= 0) {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    pa[hh][r] = (delta == 0 && l16 >= 4 * grp + r) ? pa[hh][r] : 0.0f;
                            }
                        }
                        pf[t] = make_uint4(pack2_bf16(pa[0][0], pa[0][1]), pack2_bf16(pa[0][2], pa[0][3]),
                                           pack2_bf16(pa[1][0], pa[1][1]), pack2_bf16(pa[1][2], pa[1][3]));
                    }
                }
            }
            load_q(qnext, has_next ? t1 : t0, L1);  // queries are dead for this chunk now
            load_kv_rows(kr, vr, has_next ? t1 : t0, L1, tid_it, I6{}, I8{});

            // ---- 4. G2: O^T += V''^T P^T
            {
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

            // ---- 5. outputs times gamma^(i+1), stored now (G4 does not touch them): the
            //         stores of waves with little causal work overlap the others' MFMAs
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[nt][r] *= zeta;
            if constexpr (KEEP) {
#pragma unroll
                for (int nt = 0; nt < G::NTV; ++nt) oacc_keep[ch][nt] = oacc[nt];
            } else {
                store_o(oacc, t0, L);
            }

            // ---- 6. G4: S = gamma^L (S + K^T V'')
            g4_fast(L, l16c, grpc);
            __syncthreads();  // B: every read of keys, V''^T and the state copy done

            // ---- 7. new state copy
            write_state_copy(l16c, grpc);
            have_state = true;
        };
        if constexpr (KEEP) {  // each chunk's queries stay in their own registers
            static_assert(kKeepChunks == 2, "held chunks");
            uint4 q_unused[G::KSQ];  // target of the last chunk's discarded query re-read
            if constexpr (FAST) {
                body_fast(0, qf_keep[0], qf_keep[1]);
                if (nch > 1) body_fast(1, qf_keep[1], q_unused);
            } else {
                body(0, qf_keep[0], qf_keep[1]);
                if (nch > 1) body(1, qf_keep[1], q_unused);
            }
        } else {
            if constexpr (FAST) {
                for (int ch = 0; ch < nch; ++ch) body_fast(ch, qf, qf);
            } else {
                for (int ch = 0; ch < nch; ++ch) body(ch, qf, qf);
            }
        }
    };

    // ---- final state of the last segment
    auto write_final_state = [&](const f32x4 (&st)[G::MT][G::NT]) __attribute__((always_inline)) {
        if (seg != a.nseg - 1 || !a.state_out) return;
        float* s_dst = a.state_out + static_cast<size_t>(bh) * DK * a.dv;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = d_base + mt * 16 + grp * 4 + r;
                    const int c = vt * DVT + c_base + nt * 16 + l16;
                    s_dst[static_cast<size_t>(d) * a.dv + c] = st[mt][nt][r];
                }
    };

    if constexpr (!SEGMENTED) {
        prefetch_first(true);
        load_state(a.state_in);
        have_state = a.state_in != nullptr;
        if (have_state) write_state_copy(l16, grp);
        run_chunks(std::false_type{});
        write_final_state(sacc);
        return;
    }

    // Published states are stored in accumulator order: thread (wave, lane)
    // keeps its (mt, nt) tile as one float4 at ((wave, mt, nt) * 64 + lane) * 16
    // bytes of the slot, so each wave instruction moves 1 KiB of consecutive
    // bytes through 16-byte device-coherent accesses by the thread that uses
    // the value.
    constexpr int kSlot = DK * DVT;
    const int eoff = (wave * G::MT * G::NT * 64 + lane) * 16;
    auto at = [&](int mt, int nt) __attribute__((always_inline)) { return eoff + (mt * G::NT + nt) * 1024; };
    auto slot = [&](int j) __attribute__((always_inline)) {
        return wide::make_rsrc(a.agg + (static_cast<size_t>(chain) * a.nseg + j) * kSlot, kSlot * 4);
    };
    unsigned long long* flags = a.flags + static_cast<size_t>(chain) * a.nseg * kFlagStride;
    const unsigned long long f_agg =
        (static_cast<unsigned long long>(gen + 1) << 32) | (static_cast<unsigned long long>(chain) << 1);
    const unsigned long long f_inc = f_agg | 1ull;
    auto publish = [&](const f32x4 (&st)[G::MT][G::NT], unsigned long long flag) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t dst = slot(seg);
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt) wide::store_coherent16(st[mt][nt], dst, at(mt, nt));
        wait_stores();
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(flags + static_cast<size_t>(seg) * kFlagStride, flag, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    const float gseg = static_cast<float>(gamma_pow(lg2, a.seg_len));
    // Segment groups of a.grp segments: the last member of each group (when it
    // is not the chain's last segment) publishes the group aggregate
    //     A_q = sum_{j in group q} g^(last_q - j) T_j     (T_0 read as P_0),
    // so a segment reads its group predecessors and one aggregate per earlier
    // group: S_in(s) = sum_{first<=j<s} g^(s-1-j) T_j + sum_{q<group(s)} g^(s-1-last_q) A_q.
    const int ngroups = (a.nseg + a.grp - 1) / a.grp;
    unsigned long long* gflags = a.gflags + static_cast<size_t>(chain) * ngroups * kFlagStride;
    auto gslot = [&](int q) __attribute__((always_inline)) {
        return wide::make_rsrc(a.gagg + (static_cast<size_t>(chain) * ngroups + q) * kSlot, kSlot * 4);
    };
    // Wait (wave 0, then the whole workgroup) until flags fl[lo .. hi] all read as
    // published (want_lo for index 0 of the chain's segments, else want).
    // Returns nonzero when the spin bound ran out.
    auto wait_published = [&](const unsigned long long* fl, int lo, int hi, unsigned long long want,
                              unsigned long long want0) __attribute__((always_inline)) {
        if (wave == 0) {
            // lane i watches index j0 - i, a window of 64 at a time
            int failed = 0;
            unsigned spins = 0;
            for (int j0 = hi; j0 >= lo;) {
                const int j = j0 - lane;
                const unsigned long long w = j == 0 ? want0 : want;
                const unsigned long long f =
                    j >= lo ? __hip_atomic_load(fl + static_cast<size_t>(j) * kFlagStride, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : w;
                if (__ballot(f != w) == 0) {
                    j0 -= 64;
                    continue;
                }
                if (++spins > kMaxLookbackSpins) {
                    failed = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            if (lane == 0) s_lookback[0] = failed;
        }
        __syncthreads();
        const int failed = s_lookback[0];
        __syncthreads();  // slot read before it is written again (or before sbuf receives a state copy)
        return failed;
    };
    // sin += sum_{i < n} fac_i * state(src(i)), fac_0 = fac, fac_(i+1) = fac_i * step, in order of i;
    // returns the factor after the last entry. Loads go out in predicated batches.
    auto accumulate = [&](f32x4 (&sin)[G::MT][G::NT], int n, auto src, float fac, float step)
                          __attribute__((always_inline)) {
        constexpr int kBatch = imax(1, (C == 64 ? 32 : 16) / (G::MT * G::NT));
        for (int i0 = 0; i0 < n; i0 += kBatch) {
            f32x4 t[kBatch][G::MT][G::NT];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (i0 + u < n) {
                    const __amdgpu_buffer_rsrc_t sp = src(i0 + u);
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < G::NT; ++nt) t[u][mt][nt] = wide::load_coherent16(sp, at(mt, nt));
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (i0 + u < n) {
#pragma unroll
                    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < G::NT; ++nt) sin[mt][nt] += fac * t[u][mt][nt];
                    fac *= step;
                }
            }
        }
        return fac;
    };
    // S_in of this segment (seg >= 1) into sin, always in the same order (so the
    // result does not depend on which segments finished first). When sin is
    // not sacc, sacc holds T_s (needed if this segment closes a group).
    auto look_back = [&](f32x4 (&sin)[G::MT][G::NT]) __attribute__((always_inline)) {
        const int grp_sz = a.grp;
        const int q = seg / grp_sz, first = q * grp_sz, pos = seg - first;
        int failed = pos > 0 ? wait_published(flags, first, seg - 1, f_agg, f_inc) : 0;
#pragma unroll
        for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < G::NT; ++nt) sin[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // group predecessors: entry i is segment seg-1-i with weight g^i
        const float fq = accumulate(sin, pos, [&](int i) { return slot(seg - 1 - i); }, 1.0f, gseg);
        if (pos == grp_sz - 1 && seg < a.nseg - 1) {  // close the group: A_q = T_s + g * (its predecessors)
            // a failed wait publishes NaN, so every later segment and the final state see it
            const float poison = failed ? NAN : 0.0f;
            const __amdgpu_buffer_rsrc_t dst = gslot(q);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt)
                    wide::store_coherent16(sacc[mt][nt] + gseg * sin[mt][nt] + poison, dst, at(mt, nt));
            wait_stores();
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(gflags + static_cast<size_t>(q) * kFlagStride, f_agg, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        // earlier groups: entry k is group q-1-k with weight g^(pos + k grp)
        if (q > 0) {
            failed |= wait_published(gflags, 0, q - 1, f_agg, f_agg);
            const float gstep = static_cast<float>(gamma_pow(lg2, static_cast<double>(grp_sz) * a.seg_len));
            accumulate(sin, q, [&](int k) { return gslot(q - 1 - k); }, fq, gstep);
        }
        if (failed) {
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt) sin[mt][nt] = f32x4{NAN, NAN, NAN, NAN};
        }
    };

    if constexpr (MODE == kTwoPass) {
        // ---- pass 1: this segment's own state (all segments but the last)
        if (seg < a.nseg - 1) {
            prefetch_first(false);
            load_state(seg == 0 ? a.state_in : nullptr);
            run_state_only();
            publish(sacc, seg == 0 ? f_inc : f_agg);
        }
        // ---- the start state
        prefetch_first(true);
        if (seg == 0) {
            load_state(a.state_in);
            if (a.state_in && a.state_out) {
                // state_out may alias state_in: the last segment stores the final state only
                // after this second read of it is done (its flag slot is otherwise unused)
                wait_stores();
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_store(flags + static_cast<size_t>(a.nseg - 1) * kFlagStride, f_agg, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        } else if (seg < a.nseg - 1) {  // T_s stays in sacc while the look-back may close a group
            f32x4 sin[G::MT][G::NT];
            look_back(sin);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt) sacc[mt][nt] = sin[mt][nt];
        } else {
            look_back(sacc);
        }
        // ---- pass 2: outputs and state from the start state
        have_state = seg > 0 || a.state_in != nullptr;
        if (have_state) write_state_copy(l16, grp);
        run_chunks(std::false_type{});
        if (seg == a.nseg - 1 && a.state_in && a.state_out) {
            __syncthreads();  // the look-back status slot overlays the state copy, written by every wave above
            if (wait_published(flags, a.nseg - 1, a.nseg - 1, f_agg, f_agg)) {
#pragma unroll
                for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                    for (int nt = 0; nt < G::NT; ++nt) sacc[mt][nt] = f32x4{NAN, NAN, NAN, NAN};
            }
        }
        write_final_state(sacc);
    } else if constexpr (MODE == kLocalPass) {
        // ---- every segment runs from a zero state, outputs held back
        {
            const int L0 = min(C, t_end - t_begin);
            load_kv(kr, vr, t_begin, L0, tid);
            load_q(qf_keep[0], t_begin, L0);
        }
        load_state(nullptr);
        run_chunks(std::true_type{});  // sacc = T_s
        f32x4 sin[G::MT][G::NT];
        if (seg == 0) {
            // the start state is known (the initial state or zero): publish the
            // end state P_0 = T_0 + g S_0 at once; segment 0 is never the last
            load_state_to(sin, a.state_in);
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt) sacc[mt][nt] += gseg * sin[mt][nt];
            publish(sacc, f_inc);
        } else {
            if (seg < a.nseg - 1) publish(sacc, f_agg);
            look_back(sin);
        }
        // ---- correction: o_n += gamma^(n+1) q_n S_in (n counted from the segment start)
        const bool correct = seg > 0 || a.state_in != nullptr;
        if (correct) {
            write_state_copy_of(sin, l16, grp);
            __syncthreads();  // S_in^T copy written
        }
        {
            const FragAddr<UK> fa_s(l16, grp);  // S^T rows 16 nt + l16, dk 32 s + 8 grp
#pragma unroll
            for (int c = 0; c < kKeepChunks; ++c) {
                if (c < nch) {
                    const int t0 = t_begin + c * C;
                    const float zc = zeta * fast_exp2(static_cast<float>(c * C) * lg2f);
                    if (correct) {
#pragma unroll
                        for (int nt = 0; nt < G::NTV; ++nt) {
                            f32x4 corr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int s = 0; s < G::KSQ; ++s) {
                                const uint4 af = *reinterpret_cast<const uint4*>(&sbuf[fa_s.at(nt, s)]);
                                corr = mfma16x16x32(af, qf_keep[c][s], corr);
                            }
#pragma unroll
                            for (int r = 0; r < 4; ++r) oacc_keep[c][nt][r] += zc * corr[r];
                        }
                    }
                    store_o(oacc_keep[c], t0, min(C, t_end - t0));
                }
            }
        }
        if (seg == a.nseg - 1) {  // end state = gamma^len S_in + T_s
            const float glen = static_cast<float>(gamma_pow(lg2, t_end - t_begin));
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
                for (int nt = 0; nt < G::NT; ++nt) sacc[mt][nt] += glen * sin[mt][nt];
            write_final_state(sacc);
        }
    }
}

// With 64-token chunks of 64 x 64 tiles the body fits the registers of two
// waves per SIMD (224 VGPRs, no spills), so two workgroups share a compute
// unit: the multi-scale workload's 256 workgroups then start together with
// room to spare, 3% faster than at one wave per SIMD (248 + 24 registers).
template <int DK, int DVT, int C>
constexpr int kWavesPerSimd = (C == 64 && DK == 64 && DVT == 64) ? 2 : 1;

template <int DK, int DVT, int C, int MODE, bool FAST>
__global__ __launch_bounds__((C / 16) * 64, (kWavesPerSimd<DK, DVT, C>)) void chunk_bf16_kernel(ChunkArgs a,
                                                                                               HeadParams hp) {
    chunk_body<DK, DVT, C, MODE, FAST, 0>(a, hp, blockIdx.x, gridDim.x);
}

// Several calls in one launch. Calls of one shape interleave their workgroups
// so that all of them progress together (workgroup b serves call b % n);
// calls of different sizes (same tile and form) take consecutive ranges.

template <int DK, int DVT, int C, int MODE, bool FAST>
__global__ __launch_bounds__((C / 16) * 64, (kWavesPerSimd<DK, DVT, C>)) void chunk_bf16_multi_kernel(ChunkCalls cs,
                                                                                                  HeadParams hp) {
    const int n = cs.n;
    const int b = blockIdx.x;
    if (cs.interleave) {
        chunk_body<DK, DVT, C, MODE, FAST, 1>(cs.a[b % n], hp, b / n, gridDim.x / n);
    } else {  // calls of different sizes: call c owns workgroups first[c] .. first[c+1]-1
        int c = 0;
        while (c + 1 < n && b >= cs.first[c + 1]) ++c;
        chunk_body<DK, DVT, C, MODE, FAST, 1>(cs.a[c], hp, b - cs.first[c], cs.first[c + 1] - cs.first[c]);
    }
}

// Holding two chunks of outputs and queries in registers fits with 64-token
// chunks (one wave per SIMD) and with small 128-token tiles.
template <int DK, int DVT, int C>
constexpr bool kLocalFits = C == 64 || DK + DVT <= 192;

template <int DK, int DVT, int C>
int chunk_mode(const ChunkArgs& a) {
    if (a.nseg == 1) return kSinglePass;
    if (kLocalFits<DK, DVT, C> && a.seg_len <= kKeepChunks * C) return kLocalPass;
    return kTwoPass;
}

template <int DK, int DVT, int C, bool FAST>
static void launch_chunk_form(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* e) {
    using G = ChunkGeo<DK, DVT, C>;
    constexpr int kLocal = kLocalFits<DK, DVT, C> ? kLocalPass : kTwoPass;
    const int blocks = a.B * a.H * a.nvt * a.nseg;
    switch (chunk_mode<DK, DVT, C>(a)) {
        case kSinglePass:
            launch_timed(chunk_bf16_kernel<DK, DVT, C, kSinglePass, FAST>, dim3(blocks), dim3(G::NTHR), 0, st, e,
                         a, hp);
            break;
        case kLocalPass:
            launch_timed(chunk_bf16_kernel<DK, DVT, C, kLocal, FAST>, dim3(blocks), dim3(G::NTHR), 0, st, e, a, hp);
            break;
        default:
            launch_timed(chunk_bf16_kernel<DK, DVT, C, kTwoPass, FAST>, dim3(blocks), dim3(G::NTHR), 0, st, e, a,
                         hp);
    }
}

template <int DK, int DVT, int C, bool FAST>
static void launch_chunk_multi_form(const ChunkCalls& cs, const HeadParams& hp, hipStream_t st) {
    using G = ChunkGeo<DK, DVT, C>;
    constexpr int kLocal = kLocalFits<DK, DVT, C> ? kLocalPass : kTwoPass;
    const ChunkArgs& a = cs.a[0];
    const dim3 grid(cs.first[cs.n]);
    switch (chunk_mode<DK, DVT, C>(a)) {
        case kSinglePass:
            hipLaunchKernelGGL((chunk_bf16_multi_kernel<DK, DVT, C, kSinglePass, FAST>), grid, dim3(G::NTHR), 0, st,
                               cs, hp);
            break;
        case kLocalPass:
            hipLaunchKernelGGL((chunk_bf16_multi_kernel<DK, DVT, C, kLocal, FAST>), grid, dim3(G::NTHR), 0, st, cs,
                               hp);
            break;
        default:
            hipLaunchKernelGGL((chunk_bf16_multi_kernel<DK, DVT, C, kTwoPass, FAST>), grid, dim3(G::NTHR), 0, st,
                               cs, hp);
    }
}

// The FAST form scales values by gamma^-(j+1) for j < C and outputs by
// gamma^(i+1): every head's gamma^C must stay far from the float32 range
// limits, which holds for gamma^C >= 2^-64 (any gamma >= 0.71 at C = 128,
// >= 0.5 at C = 64, and every default gamma 1 - 2^(-5-h)).
bool fast_form_ok(const HeadParams& hp, int H, int chunk) {
    for (int h = 0; h < H; ++h)
        if (std::log2(static_cast<double>(hp.gamma[h])) * chunk < -64.0) return false;
    return true;
}

template <int DK, int DVT, int C>
static hipError_t run_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, hipStream_t st, hipEvent_t* ev) {
    // Unrotated heads of width 128 or 256 in 128-token chunks run on the wide
    // kernel, segmented (state pass, scan, segment pass) when the plan cuts the
    // sequence; it takes its six phase events itself.
    if (chunk_wide_supported(DK, DVT, C, hp.has_theta != 0) && (a.nseg == 1 || a.agg != nullptr)) {
        const int R = chunk_wide_rescale(hp, a.H);
        if (R > 0) {
            ChunkArgs aw = a;
            aw.rescale = R;
            return launch_chunk_wide(aw, hp, st, ev);
        }
    }
    // the segmented form of this kernel is a single launch: the pre-pass and scan phases are empty
    record_empty_phase(st, ev);
    record_empty_phase(st, ev ? ev + 2 : nullptr);
    hipEvent_t* e = ev ? ev + 4 : nullptr;
    if (fast_form_ok(hp, a.H, C))
        launch_chunk_form<DK, DVT, C, true>(a, hp, st, e);
    else
        launch_chunk_form<DK, DVT, C, false>(a, hp, st, e);
    return hipGetLastError();
}

template <int DK, int DVT, int C>
static hipError_t run_chunk_bf16_multi(const ChunkCalls& cs, const HeadParams& hp, hipStream_t st) {
    if (fast_form_ok(hp, cs.a[0].H, C))
        launch_chunk_multi_form<DK, DVT, C, true>(cs, hp, st);
    else
        launch_chunk_multi_form<DK, DVT, C, false>(cs, hp, st);
    return hipGetLastError();
}

#define RET_CHUNK_SHAPES \
    RET_CASE(64, 64, 32)   \
    RET_CASE(128, 64, 32)  \
    RET_CASE(256, 64, 32)  \
    RET_CASE(64, 64, 64)   \
    RET_CASE(64, 128, 64)  \
    RET_CASE(128, 64, 64)  \
    RET_CASE(128, 128, 64) \
    RET_CASE(256, 64, 64)  \
    RET_CASE(64, 64, 128)  \
    RET_CASE(64, 128, 128) \
    RET_CASE(128, 64, 128) \
    RET_CASE(128, 128, 128) \
    RET_CASE(256, 64, 128) \
    RET_CASE(256, 128, 128)

// The kernel form (single pass, local pass, two-pass) a call takes.
static int call_form(const ChunkArgs& a) {
    if (a.nseg == 1) return kSinglePass;
    const bool local_fits = a.chunk == 64 || a.dk + a.dv / a.nvt <= 192;
    return (local_fits && a.seg_len <= kKeepChunks * a.chunk) ? kLocalPass : kTwoPass;
}

hipError_t launch_chunk_bf16_multi(const ChunkCalls& in, const HeadParams& hp, int dvt, hipStream_t st) {
    if (in.n < 1 || in.n > kMaxChunkCalls) return hipErrorInvalidValue;
    ChunkCalls cs = in;
    const ChunkArgs& a = cs.a[0];
    bool same = true;
    cs.first[0] = 0;
    for (int i = 0; i < cs.n; ++i) {  // one tile and one kernel form for every call
        const ChunkArgs& b = cs.a[i];
        if (b.dk != a.dk || b.chunk != a.chunk || b.dv % dvt != 0 || b.dv / dvt != b.nvt ||
            call_form(b) != call_form(a) || (b.orot && !chunk_orot_fits(b.dk, dvt, b.chunk)))
            return hipErrorInvalidValue;
        same = same && b.B == a.B && b.H == a.H && b.N == a.N && b.dv == a.dv && b.nseg == a.nseg &&
               b.seg_len == a.seg_len && b.grp == a.grp;
        cs.first[i + 1] = cs.first[i] + b.B * b.H * b.nvt * b.nseg;
    }
    cs.interleave = same ? 1 : 0;
#define RET_CASE(DK_, DVT_, C_) \
    if (a.dk == DK_ && dvt == DVT_ && a.chunk == C_) return run_chunk_bf16_multi<DK_, DVT_, C_>(cs, hp, st);
    RET_CHUNK_SHAPES
#undef RET_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, const HeadParams& hp, int dvt, hipStream_t st, hipEvent_t* ev) {
#define RET_CASE(DK_, DVT_, C_) \
    if (a.dk == DK_ && dvt == DVT_ && a.chunk == C_) return run_chunk_bf16<DK_, DVT_, C_>(a, hp, st, ev);
    RET_CHUNK_SHAPES
#undef RET_CASE
    return hipErrorInvalidValue;
}

#undef RET_CHUNK_SHAPES

}  // namespace ret
