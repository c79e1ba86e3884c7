// Parallel retention form O = ((Q K^T) (.) D) V for heads without rotation, on
// gfx950 (MI355X) matrix cores: bf16 inputs, float32 accumulation.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "1. The
// Parallel Representation for High-Throughput Pretraining": D[n][m] =
// gamma^(n-m) for n >= m and 0 otherwise.
//
// One workgroup of eight waves (two per SIMD) owns 128 query rows of one
// (batch, head, 128-column value tile) and walks the key blocks of 128 tokens
// from its diagonal block backwards; wave w owns query rows 16 w .. 16 w + 15.
// Each wave fits in half a SIMD's register file, so while one wave waits for
// its LDS operands the other issues matrix instructions (one wave per SIMD
// owning two row blocks, every fragment feeding two instructions, measured
// 15% slower: it cannot hide the LDS latency alone). On the diagonal block
// wave w has w + 1 causal tiles; every other block is the same work for all.
// Per key block, on v_mfma_f32_16x16x32_bf16:
//   G1  P^T = K Q^T, times D in registers, rounded to bf16 B operands
//   G2  O^T += V^T P^T       (V^T by transposing LDS reads)
// Keys and values of the next key block go from HBM straight into LDS (two
// buffers each) while the current block is multiplied. D is a per-lane factor
// times a per-tile factor, every exponent kept >= 0; the walk stops at the
// first key block whose entries of D all underflow float32, since it and every
// earlier block then add exactly zero. Query blocks are dispatched
// longest-first. The causal work of a query block grows with its position, so
// when the blocks alone would leave compute units idle the walk of every block
// longer than T key blocks is split: one workgroup takes the T blocks from the
// diagonal, another the rest. The first of the two to finish (by a ticket)
// writes its float32 partial of O to the workspace and marks it written; the
// second adds it to its own and stores O. Retention has no softmax
// normaliser, so the two partials simply add; a sum of two float32 values does
// not depend on their order, so the result repeats bit for bit whichever
// finishes first.

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"
#include "wide.hpp"

namespace ret {

namespace {

using namespace wide;

constexpr int kParBQ = 128;       // query rows per workgroup, keys per key block
constexpr int kParDvt = 128;      // value columns per workgroup
constexpr int kParThreads = 512;  // eight waves, two per SIMD
constexpr int kParPipe = 4;       // steps between an LDS read and its use
// Bound of the second half's wait for the first half's partial (the first is
// running: it took its ticket before writing). Past it O is stored as NaN and
// the pair's counter is left undefined (the workspace then needs zero-filling
// again); a wait can only run out if the first half stops making progress.
constexpr unsigned kMaxHandoverSpins = 1u << 20;

template <int DK>
struct ParWGeo {
    static constexpr int UK = DK / 8;                         // 16-byte units per key row
    static constexpr int UV = kParDvt / 8;                    // 16-byte units per value row (of the tile)
    static constexpr int KSQ = DK / 32;                       // 32-wide contraction steps over d_k
    static constexpr int NTV = kParDvt / 16;                  // 16-column tiles of the value tile
    static constexpr int KBLK = kParBQ * DK * 2 / 1024 / 8;   // 1 KiB key blocks per wave
    static constexpr int VBLK = kParBQ * kParDvt * 2 / 1024 / 8;  // 1 KiB value blocks per wave
    static_assert(DK == 64 || DK == 128, "key width");
};

}  // namespace

template <int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(kParThreads, kParThreads), amdgpu_waves_per_eu(2, 2)))
void parallel_wide_kernel(ParallelArgs a, HeadParams hp) {
    using G = ParWGeo<DK>;
    constexpr int BQ = kParBQ;
    constexpr int UK = G::UK;
    __shared__ __attribute__((aligned(16))) u16 kb0[BQ * DK];
    __shared__ __attribute__((aligned(16))) u16 kb1[BQ * DK];
    __shared__ __attribute__((aligned(16))) u16 vb0[BQ * kParDvt];
    __shared__ __attribute__((aligned(16))) u16 vb1[BQ * kParDvt];
    __shared__ unsigned s_ticket;

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15;
    const int grp = lane >> 4;

    const int nqb = (a.N + BQ - 1) / BQ;
    const int BH = a.B * a.H;
    // Block order as dispatched: the hardware deals consecutive blocks to the eight XCDs
    // in turn, so each XCD receives every eighth entry of the longest-first order (an even
    // share of long and short walks), and with (batch, head, value tile) the fastest index
    // a multiple of eight of them keeps each head's keys and values in one XCD's L2.
    const int lb = static_cast<int>(blockIdx.x);
    const int vt = lb % a.nvt;
    const int bh = (lb / a.nvt) % BH;
    // Position li of this workgroup in its (batch, head, value tile)'s longest-first
    // order. Unsplit (T = 0): query block nqb - 1 - li, whole walk. Split: first the
    // diagonal parts of blocks nqb-1 .. T (T key blocks each), then blocks T-1 .. nqb-T
    // alone (walks T .. nqb-T+1), then per length w = nqb-T .. 1 the block w-1 alone
    // and the rest of block w+T-1 (key blocks T .. w+T-1 back from its diagonal).
    const int T = a.split_t;
    const int S = T > 0 ? nqb - T : 0;  // split query blocks
    const int li = lb / (a.nvt * BH);
    int qb, m_lo, m_hi, part;  // walk m_lo <= m < m_hi blocks back from the diagonal; part 0: whole
    if (S == 0 || li < S) {
        qb = nqb - 1 - li;
        m_lo = 0;
        m_hi = S == 0 ? qb + 1 : T;
        part = S == 0 ? 0 : 1;
    } else {
        const int r = li - S, c1 = 2 * T - nqb;
        if (r < c1) {
            qb = T - 1 - r;
            part = 0;
        } else {
            const int w = nqb - T - (r - c1) / 2;
            part = ((r - c1) & 1) ? 2 : 0;
            qb = part ? w + T - 1 : w - 1;
        }
        m_lo = part ? T : 0;
        m_hi = qb + 1;
    }
    const int h = bh % a.H;
    const float gam = hp.gamma[h];
    const double lg2 = log2_gamma(gam);
    const float lg2f = static_cast<float>(lg2);

    const size_t tok0 = static_cast<size_t>(bh) * a.N;
    const char* Kg = reinterpret_cast<const char*>(a.k + tok0 * DK);
    const char* Qg = reinterpret_cast<const char*>(a.q + tok0 * DK);
    const char* Vg = reinterpret_cast<const char*>(a.v + tok0 * a.dv + vt * kParDvt);
    char* Og = reinterpret_cast<char*>(a.o + tok0 * a.dv + vt * kParDvt);
    const int ldv = a.dv * 2;    // value / output row stride, bytes
    constexpr int ldk = DK * 2;  // key / query row stride, bytes
    constexpr int tile_bytes = kParDvt * 2;
    const int q0 = qb * BQ;
    const int Lq = min(BQ, a.N - q0);

    // Key block i (1 KiB) of this wave's share of key block `kb`, straight into
    // LDS: each wave instruction fills 1 KiB of consecutive LDS (lane l the
    // 16-byte unit at 16 l), so each lane fetches the unit the swizzled layout
    // puts there. Rows past the sequence end read as zero.
    auto load_keys = [&](int kbk, u16* dst, int i) __attribute__((always_inline)) {
        const int k0 = kbk * BQ;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(Kg + static_cast<size_t>(k0) * ldk, min(BQ, a.N - k0) * ldk);
        const int blk = wave * G::KBLK + i;
        const int e = blk * 512 + lane * 8;
        const int row = e / DK;
        const int unit = ((e % DK) >> 3) ^ (row & ((UK < 16 ? UK : 16) - 1));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(dst + blk * 512), 16, row * ldk + unit * 16, 0,
                                                 0, 0);
    };
    auto load_values = [&](int kbk, u16* dst, int i) __attribute__((always_inline)) {
        const int k0 = kbk * BQ;
        const int L = min(BQ, a.N - k0);
        const __amdgpu_buffer_rsrc_t r = make_rsrc(Vg + static_cast<size_t>(k0) * ldv, (L - 1) * ldv + tile_bytes);
        const int blk = wave * G::VBLK + i;
        const int e = blk * 512 + lane * 8;
        const int row = e / kParDvt;
        const int unit = ((e % kParDvt) >> 3) ^ (row & 15);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(dst + blk * 512), 16, row * ldv + unit * 16, 0,
                                                 0, 0);
    };
    // Transposing-read fragment of V (8 keys of 32-key step t, rows 4 grp + {0..3, 16..19})
    // of value columns 16 nt .. +15: lane (l16, grp) points at key 4 grp + l16/4 (+16),
    // columns 16 nt + 4 (l16 % 4) .. +3.
    auto v_frag = [&](const u16* buf, int nt, int t) __attribute__((always_inline)) {
        const int tok = 4 * grp + (l16 >> 2);
        const int c = 16 * nt + 4 * (l16 & 3);
        const int base = swz<G::UV>(tok, c >> 3) + (c & 7);
        const uint2 lo = lds_read_tr16x4(&buf[base + (32 * t) * kParDvt]);
        const uint2 hi = lds_read_tr16x4(&buf[base + (32 * t + 16) * kParDvt]);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    };

    // queries of blocks wave and 7-wave: row 16 blk + l16, d_k 32 s + 8 grp
    uint4 qf[G::KSQ];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg + static_cast<size_t>(q0) * ldk, Lq * ldk);
#pragma unroll
        for (int s = 0; s < G::KSQ; ++s) qf[s] = buf_load16(rq, (16 * wave + l16) * ldk + grp * 16 + s * 64);
    }
    f32x4 oacc[G::NTV];  // O^T: [column tile]
#pragma unroll
    for (int nt = 0; nt < G::NTV; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 pf[4];  // P^T (times D) as bf16 B operands: [32-key step]

    // D = gamma^((q0 + 16 blk + l16) - (k0 + 16 kt + 4 grp + r)):
    //   diagonal tile (q0 = k0, kt = blk): dlane[r] = gamma^(l16 - 4 grp - r)
    //     (negative exponents only in masked entries, which are selected away);
    //   other tiles: dlane15[r] gamma^(16 (blk - kt) + (q0 - k0) - 15), the tile exponent >= 1.
    float dlane[4], dlane15[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        dlane[r] = fast_exp2(static_cast<float>(l16 - 4 * grp - r) * lg2f);
        dlane15[r] = fast_exp2(static_cast<float>(l16 - 4 * grp - r + 15) * lg2f);
    }

    // key blocks with any entry of D above float32 underflow: block qb - m has
    // its largest decay gamma^(128 m - 127)
    int nkb = m_hi;
    if (lg2 < 0.0) {
        const double span = 160.0 / (-lg2);  // gamma^span < 2^-160
        const int mmax = static_cast<int>((span + BQ - 1) / BQ) + 1;
        nkb = min(nkb, mmax + 1);
    }

    // G1 for the wave owning block W against the key block in kb (delta = q0 - k0);
    // DIAG: the diagonal block (causal tiles only). Riding along: the next key
    // block's keys and values into the other buffers (next < 0: none).
    auto g1 = [&](const u16* __restrict__ kb, u16* __restrict__ nkbuf, u16* __restrict__ nvbuf, int next, int delta,
                  auto wtag, auto diag_tag) __attribute__((always_inline)) {
        constexpr int B0 = decltype(wtag)::value;
        constexpr bool DIAG = decltype(diag_tag)::value;
        constexpr int T0 = DIAG ? B0 / 2 + 1 : 4;
        const FragAddr<UK> fk(l16, grp);
        struct KF {
            uint4 a, b;
        };
        f32x4 p[2];
        constexpr int NS1 = T0 * G::KSQ;
        pipelined<NS1, kParPipe>(
            [&](auto j) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::KSQ, s = decltype(j)::value % G::KSQ;
                KF f;
                f.a = *reinterpret_cast<const uint4*>(&kb[fk.at(2 * t, s)]);
                if constexpr (!DIAG || 2 * t + 1 <= B0)
                    f.b = *reinterpret_cast<const uint4*>(&kb[fk.at(2 * t + 1, s)]);
                return f;
            },
            [&](auto j, const KF& f) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::KSQ, s = decltype(j)::value % G::KSQ;
                constexpr bool two = !DIAG || 2 * t + 1 <= B0;
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                p[0] = mfma16x16x32(f.a, qf[s], s == 0 ? zero : p[0]);
                if constexpr (two) p[1] = mfma16x16x32(f.b, qf[s], s == 0 ? zero : p[1]);
                if constexpr (s == G::KSQ - 1) {
                    f32x4 r[2] = {p[0], two ? p[1] : zero};
                    auto decay = [&](f32x4& x, int blk, int kt, bool present) __attribute__((always_inline)) {
                        if (!present) return;
                        if (DIAG && kt == blk) {
#pragma unroll
                            for (int q = 0; q < 4; ++q) x[q] = (4 * grp + q <= l16) ? x[q] * dlane[q] : 0.0f;
                        } else {
                            const float tf = fast_exp2(static_cast<float>(16 * (blk - kt) + delta - 15) * lg2f);
#pragma unroll
                            for (int q = 0; q < 4; ++q) x[q] *= dlane15[q] * tf;
                        }
                    };
                    const int blk0 = DIAG ? B0 : wave;
                    decay(r[0], blk0, 2 * t, true);
                    decay(r[1], blk0, 2 * t + 1, two);
                    pf[t] = make_uint4(pack2_bf16(r[0][0], r[0][1]), pack2_bf16(r[0][2], r[0][3]),
                                       pack2_bf16(r[1][0], r[1][1]), pack2_bf16(r[1][2], r[1][3]));
                }
            },
            [&](auto j) __attribute__((always_inline)) {
                constexpr int J = decltype(j)::value;
                if (next >= 0) {
                    spread<G::KBLK, NS1, J>([&](auto i) { load_keys(next, nkbuf, i); });
                    spread<G::VBLK, NS1, J>([&](auto i) { load_values(next, nvbuf, i); });
                }
            });
    };
    auto g2 = [&](const u16* __restrict__ vb, auto wtag, auto diag_tag) __attribute__((always_inline)) {
        constexpr int B0 = decltype(wtag)::value;
        constexpr bool DIAG = decltype(diag_tag)::value;
        constexpr int T0 = DIAG ? B0 / 2 + 1 : 4;
        constexpr int NS2 = T0 * G::NTV;
        pipelined<NS2, kParPipe>(
            [&](auto j) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                return v_frag(vb, nt, t);
            },
            [&](auto j, const uint4& vf) __attribute__((always_inline)) {
                constexpr int t = decltype(j)::value / G::NTV, nt = decltype(j)::value % G::NTV;
                oacc[nt] = mfma16x16x32(vf, pf[t], oacc[nt]);
            },
            [](auto) {});
    };
    auto step = [&](int m, u16* __restrict__ kb, u16* __restrict__ vb, u16* __restrict__ nk, u16* __restrict__ nv)
                    __attribute__((always_inline)) {
        // this key block has landed (nothing else is in flight) and every wave
        // has finished with the other buffers
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
        const int next = m + 1 < nkb ? qb - m - 1 : -1;
        const int delta = m * BQ;
        if (m == 0) {
            switch (wave) {
                case 0: g1(kb, nk, nv, next, delta, Ic<0>{}, Ic<1>{}); g2(vb, Ic<0>{}, Ic<1>{}); break;
                case 1: g1(kb, nk, nv, next, delta, Ic<1>{}, Ic<1>{}); g2(vb, Ic<1>{}, Ic<1>{}); break;
                case 2: g1(kb, nk, nv, next, delta, Ic<2>{}, Ic<1>{}); g2(vb, Ic<2>{}, Ic<1>{}); break;
                case 3: g1(kb, nk, nv, next, delta, Ic<3>{}, Ic<1>{}); g2(vb, Ic<3>{}, Ic<1>{}); break;
                case 4: g1(kb, nk, nv, next, delta, Ic<4>{}, Ic<1>{}); g2(vb, Ic<4>{}, Ic<1>{}); break;
                case 5: g1(kb, nk, nv, next, delta, Ic<5>{}, Ic<1>{}); g2(vb, Ic<5>{}, Ic<1>{}); break;
                case 6: g1(kb, nk, nv, next, delta, Ic<6>{}, Ic<1>{}); g2(vb, Ic<6>{}, Ic<1>{}); break;
                default: g1(kb, nk, nv, next, delta, Ic<7>{}, Ic<1>{}); g2(vb, Ic<7>{}, Ic<1>{}); break;
            }
        } else {
            // off the diagonal every wave does the same work
            g1(kb, nk, nv, next, delta, Ic<0>{}, Ic<0>{});
            g2(vb, Ic<0>{}, Ic<0>{});
        }
    };

    // the first key block of the walk (the diagonal one unless this is the rest of a split walk)
    if (m_lo < nkb) {
#pragma unroll
        for (int i = 0; i < G::KBLK; ++i) load_keys(qb - m_lo, kb0, i);
#pragma unroll
        for (int i = 0; i < G::VBLK; ++i) load_values(qb - m_lo, vb0, i);
    }
    for (int m = m_lo; m < nkb; m += 2) {
        step(m, kb0, vb0, kb1, vb1);
        if (m + 1 < nkb) step(m + 1, kb1, vb1, kb0, vb0);
    }

    if (part != 0) {  // half of a split walk: the first to finish hands its partial over, the second stores O
        // a partial in register order: (wave, block, column tile) a 1 KiB run, lane l its
        // 16 bytes at 16 l (the two halves share the order, so they add element by element).
        // The pair's ticket counts arrivals (+1 each) and the partial's completion (+2).
        const size_t si = (static_cast<size_t>(bh) * a.nvt + vt) * S + (qb - T);
        constexpr int kPartBytes = BQ * kParDvt * 4;
        const __amdgpu_buffer_rsrc_t mine = make_rsrc(a.part + (si * 2 + (part - 1)) * (BQ * kParDvt), kPartBytes);
        const __amdgpu_buffer_rsrc_t other = make_rsrc(a.part + (si * 2 + (2 - part)) * (BQ * kParDvt), kPartBytes);
        auto at = [&](int nt) { return ((wave * G::NTV + nt) * 64 + lane) * 16; };
        if (threadIdx.x == 0)
            s_ticket = __hip_atomic_fetch_add(a.ctr + si, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const unsigned t0 = s_ticket;
        __syncthreads();  // every thread has read the ticket before s_ticket is reused
        if (t0 == 0) {  // first: write the partial, then mark it complete
#pragma unroll
            for (int nt = 0; nt < G::NTV; ++nt) store_coherent16(oacc[nt], mine, at(nt));
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial is out
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_fetch_add(a.ctr + si, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        // second: the other's partial is complete once the counter reads 4 (1 + 1 + 2)
        if (threadIdx.x == 0) {
            unsigned v = t0 + 1, spins = 0;
            while (v < 4 && spins++ < kMaxHandoverSpins) {
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load(a.ctr + si, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            s_ticket = v;
            // ready for the next call (the first is done with the counter)
            __hip_atomic_store(a.ctr + si, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const bool ok = s_ticket >= 4;
#pragma unroll
        for (int nt = 0; nt < G::NTV; ++nt) {
            const f32x4 x = load_coherent16(other, at(nt));
            oacc[nt] += ok ? x : f32x4{NAN, NAN, NAN, NAN};
        }
    }

    // O = O^T transposed back: lane (l16, grp) holds rows 16 blk + l16, columns 16 nt + 4 grp .. +3
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(Og + static_cast<size_t>(q0) * ldv, (Lq - 1) * ldv + tile_bytes);
#pragma unroll
    for (int nt = 0; nt < G::NTV; ++nt) {
        const f32x4 o = oacc[nt];
        buf_store8(make_uint2(pack2_bf16(o[0], o[1]), pack2_bf16(o[2], o[3])), ro,
                   (16 * wave + l16) * ldv + grp * 8 + nt * 32);
    }
}

bool parallel_wide_supported(int dk, int dv, bool rotation) {
    return !rotation && (dk == 64 || dk == 128) && dv % kParDvt == 0;
}

// Split the long walks when the query blocks (over heads and value tiles) are at
// most two per compute unit: beyond that the longest-first dispatch keeps the
// units busy by itself. T = ceil(nqb / 2): no workgroup walks more than T blocks.
int parallel_wide_split(int B, int H, int N, int dv) {
    const long long nqb = (static_cast<long long>(N) + kParBQ - 1) / kParBQ;
    const long long blocks = nqb * B * H * (dv / kParDvt);
    if (nqb < 2 || blocks > 512) return 0;
    return static_cast<int>((nqb + 1) / 2);
}

// Workspace: the tickets first, in a region of fixed size (at most 512 query blocks,
// of which at most half split: 256 tickets), so that calls of any sizes sharing a
// workspace find theirs where earlier calls left tickets at zero, never partials;
// then two float32 128 x 128 partials per split block.
constexpr size_t kParTicketBytes = 256 * sizeof(unsigned);

size_t parallel_wide_workspace(int B, int H, int N, int dv) {
    const int T = parallel_wide_split(B, H, N, dv);
    if (T == 0) return 0;
    const size_t nqb = (static_cast<size_t>(N) + kParBQ - 1) / kParBQ;
    const size_t nsplit = (nqb - T) * B * H * (dv / kParDvt);
    return kParTicketBytes + nsplit * 2 * kParBQ * kParDvt * sizeof(float);
}

void parallel_wide_bind(ParallelArgs& a, void* workspace) {
    a.split_t = parallel_wide_split(a.B, a.H, a.N, a.dv);
    a.ctr = static_cast<unsigned*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kParTicketBytes);
}

hipError_t launch_parallel_wide(const ParallelArgs& a, const HeadParams& hp, hipStream_t st) {
    const int nqb = (a.N + kParBQ - 1) / kParBQ;
    if (a.split_t != 0 && (a.split_t != parallel_wide_split(a.B, a.H, a.N, a.dv) || !a.part || !a.ctr ||
                           static_cast<size_t>(nqb - a.split_t) * a.B * a.H * a.nvt > kParTicketBytes / sizeof(unsigned)))
        return hipErrorInvalidValue;
    const int per = nqb + (a.split_t ? nqb - a.split_t : 0);  // workgroups per (batch, head, value tile)
    const dim3 grid(per * a.B * a.H * a.nvt), block(kParThreads);
    if (a.dk == 128)
        hipLaunchKernelGGL(parallel_wide_kernel<128>, grid, block, 0, st, a, hp);
    else
        hipLaunchKernelGGL(parallel_wide_kernel<64>, grid, block, 0, st, a, hp);
    return hipGetLastError();
}

}  // namespace ret
