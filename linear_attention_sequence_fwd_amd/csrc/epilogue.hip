// Output stage of multi-scale retention: GroupNorm over each head of each
// token, an optional element-wise gate, and the output projection W_O.
//
// "RetNet Guide: Retentive Networks & The Impossible Triangle", section "1. The
// Parallel Representation for High-Throughput Pretraining": MSR(X) =
// GroupNorm(Concat(R_1, ..., R_H)) W_O, with one normalisation group per head
// (its listing: eps 1e-6, per-channel weight and bias, a bias-free projection
// whose weight is [d_out, H*dv]). "How RetNet Combines Parallel Training and
// Constant Inference" applies a gate together with the GroupNorm; the gate is
// a tensor the caller supplies.
//
// Two kernels:
//   groupnorm_gate_kernel: reads O [B,H,N,dv] once, writes Z [B*N, H*dv] (the
//     heads of a token side by side) normalised, scaled, shifted and gated, in
//     bf16. HBM-bound: 2 bytes read and 2 written per element (+2 for a gate).
//   gemm_bt_kernel: Y [M, d_out] = Z [M, K] W^T with W [d_out, K], both
//     K-contiguous; bf16 operands on v_mfma_f32_16x16x32_bf16, float32
//     accumulation. Tiles of 256 x 256 (256 x 128) per workgroup of eight
//     waves that each hold a 64 x 128 (64 x 64) output block, so a 16-byte
//     operand read from LDS feeds 4 to 8 matrix instructions; 64-deep K steps
//     double-buffered in LDS and filled by direct global-to-LDS loads (the
//     next step's loads are in flight while the current one is multiplied);
//     output staged through LDS for 16-byte stores.
//   gemm_split_kernel + reduce_splits_kernel: the same product for at most 64
//     rows, its K range split over workgroups (about one per compute unit)
//     with three LDS stages, then the float32 partials summed in split order.
// A decode step whose workgroups own whole rows normalises and gates in the
// step kernel itself (decode.hip), and only the projection runs here.

#include "common.hpp"
#include "kernels.hpp"

namespace ret {

namespace {

constexpr int kNormThreads = 256;

// Sum over the G consecutive lanes that share a row (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ void unpack8(const uint4& w, float* x) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        x[2 * p] = lo_bf16(ws[p]);
        x[2 * p + 1] = hi_bf16(ws[p]);
    }
}

// One (token, head) row of DV channels per group of G lanes, U 16-byte chunks
// (8 channels each) per lane; every load of a row is issued before the
// reductions that need it.
template <int DV>
__global__ __launch_bounds__(kNormThreads) void groupnorm_gate_kernel(EpilogueArgs a) {
    constexpr int U = DV >= 256 ? DV / 128 : 1;  // chunks per lane
    constexpr int G = DV / (8 * U);               // lanes per row (8 or 16)
    constexpr int RPB = kNormThreads / G;         // rows per workgroup
    const int tid = threadIdx.x;
    const long long row = static_cast<long long>(blockIdx.x) * RPB + tid / G;  // (b, h, n) of O
    const long long rows = static_cast<long long>(a.B) * a.H * a.N;
    if (row >= rows) return;  // whole groups leave together: no shuffle partner is lost
    const int lg = tid % G;
    const long long bh = row / a.N;
    const int n = static_cast<int>(row - bh * a.N);
    const int b = static_cast<int>(bh / a.H), h = static_cast<int>(bh % a.H);
    const int K = a.H * DV;
    const size_t zrow = (static_cast<size_t>(b) * a.N + n) * K + static_cast<size_t>(h) * DV;

    // chunk u of this lane covers channels (u * G + lg) * 8 .. + 7 of the head
    uint4 ow[U], gw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ow[u] = *reinterpret_cast<const uint4*>(a.o + row * DV + (u * G + lg) * 8);
    if (a.gate) {
#pragma unroll
        for (int u = 0; u < U; ++u) gw[u] = *reinterpret_cast<const uint4*>(a.gate + zrow + (u * G + lg) * 8);
    }
    float x[U][8];
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unpack8(ow[u], x[u]);
#pragma unroll
        for (int i = 0; i < 8; ++i) s += x[u][i];
    }
    const float mean = group_sum<G>(s) * (1.0f / DV);
    float s2 = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) s2 += (x[u][i] - mean) * (x[u][i] - mean);
    const float rstd = rsqrtf(group_sum<G>(s2) * (1.0f / DV) + a.eps);

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u * G + lg) * 8;  // channel within the head
        float gt[8], wt[8], bs[8];
        if (a.gate) {
            unpack8(gw[u], gt);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) gt[i] = 1.f;
        }
        if (a.gn_weight) {
            const float4* wp = reinterpret_cast<const float4*>(a.gn_weight + h * DV + c);
            const float4 w0 = wp[0], w1 = wp[1];
            wt[0] = w0.x; wt[1] = w0.y; wt[2] = w0.z; wt[3] = w0.w;
            wt[4] = w1.x; wt[5] = w1.y; wt[6] = w1.z; wt[7] = w1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) wt[i] = 1.f;
        }
        if (a.gn_bias) {
            const float4* bp = reinterpret_cast<const float4*>(a.gn_bias + h * DV + c);
            const float4 b0 = bp[0], b1 = bp[1];
            bs[0] = b0.x; bs[1] = b0.y; bs[2] = b0.z; bs[3] = b0.w;
            bs[4] = b1.x; bs[5] = b1.y; bs[6] = b1.z; bs[7] = b1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) bs[i] = 0.f;
        }
        float z[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = ((x[u][i] - mean) * rstd * wt[i] + bs[i]) * gt[i];
        *reinterpret_cast<uint4*>(a.z + zrow + c) = make_uint4(pack2_bf16(z[0], z[1]), pack2_bf16(z[2], z[3]),
                                                              pack2_bf16(z[4], z[5]), pack2_bf16(z[6], z[7]));
    }
}

// ---------------------------------------------------------------- GEMM

// Workgroup tile GM x BN (BN = 256, or 128 when d_out is not a multiple of 256);
// K advances 64 at a time through two LDS stages filled by direct
// global-to-LDS loads (no registers hold the next stage).
//
// LDS layout of a 64-deep panel: rows of 128 bytes, the eight 16-byte chunks
// of row r stored at position chunk ^ (r % 8), so the 16 rows an MFMA operand
// read touches land in different banks. A global-to-LDS load writes 1 KiB per
// wave at consecutive addresses (16 bytes per lane), so lane l of load i fills
// row R = 8 i + l / 8, position l % 8, and fetches the chunk that belongs there.
constexpr int GK = 64;
constexpr int kGroupM = 4;   // row tiles per group of the tile order (4 measured best of 1..32)
// Eight waves in 4 x 2: 64 x 128 output blocks (128 accumulator registers a
// lane, held in ordinary VGPRs), two waves per SIMD (4 x 2 measured 3% faster
// than 2 x 4). Four waves with 128 x 128 blocks would read half the operand
// bytes from LDS but fill the whole accumulator file, and the register
// allocator then shuffles it.
constexpr int kWavesM = 4, kWavesN = 2;

typedef __attribute__((address_space(3))) void* lds_ptr;

// Issue the loads that fill one ROWS x 64 panel: the NW waves share its 1 KiB blocks.
template <int ROWS, int NW>
__device__ __forceinline__ void panel_fill(u16* lds, const u16* base, int row0, int rows_valid, int K, int k0,
                                           int wave, int lane) {
    constexpr int PER_WAVE = ROWS / 8 / NW;  // 1 KiB blocks (8 rows) per wave
    static_assert(PER_WAVE * 8 * NW == ROWS, "panel split");
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int blk = wave * PER_WAVE + i;
        const int R = blk * 8 + (lane >> 3);
        const int chunk = (lane & 7) ^ (R & 7);
        const int r = min(row0 + R, rows_valid - 1);  // rows past the end re-read the last: never stored
        const u16* src = base + static_cast<size_t>(r) * K + k0 + chunk * 8;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr)(lds + blk * 8 * GK), 16, 0, 0);
    }
}

// The 16-byte operand of row r, chunk c (c = 0..7 over the 64-deep panel).
__device__ __forceinline__ uint4 panel_read(const u16* lds, int r, int c) {
    return *reinterpret_cast<const uint4*>(lds + r * GK + ((c ^ (r & 7)) * 8));
}

// Multiply the panels in (as, bs) into the accumulators while the loads of the
// next step fill (an, bn) when `more`; then wait for those loads and
// synchronise. The two stages are distinct LDS objects, so the compiler can
// see that reading one does not wait for the loads into the other.
template <int BM, int BN, int WM, int WN, int NW>
__device__ __forceinline__ void gemm_step(f32x4 (&acc)[WM / 16][WN / 16], const u16* as, const u16* bs, u16* an,
                                          u16* bn, bool more, const GemmArgs& g, int m0, int n0, int knext, int wm,
                                          int wn, int wave, int lane) {
    constexpr int TI = WM / 16, TJ = WN / 16;
    const int l16 = lane & 15, grp = lane >> 4;
    if (more) {
        panel_fill<BM, NW>(an, g.a, m0, g.M, g.K, knext, wave, lane);
        panel_fill<BN, NW>(bn, g.b, n0, g.N, g.K, knext, wave, lane);
    }
#pragma unroll
    for (int ks = 0; ks < GK / 32; ++ks) {
        uint4 bf[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) bf[j] = panel_read(bs, wn * WN + j * 16 + l16, ks * 4 + grp);
        // acc[i][j] = W tile j (rows: output columns) x Z tile i^T (columns: output rows)
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const uint4 af = panel_read(as, wm * WM + i * 16 + l16, ks * 4 + grp);
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16x16x32(bf[j], af, acc[i][j]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads into the other stage have landed
    __syncthreads();
}

// NWM x NWN waves; wave tile (BM / NWM) x (BN / NWN); the whole K range per
// workgroup (few rows take gemm_split_kernel instead).
template <int BM, int BN, int NWM, int NWN>
__global__ __launch_bounds__(NWM * NWN * 64) void gemm_bt_kernel(GemmArgs g) {
    constexpr int GM = BM;
    constexpr int NW = NWM * NWN;
    constexpr int WM = GM / NWM, WN = BN / NWN;  // wave tile
    constexpr int TI = WM / 16, TJ = WN / 16;    // 16 x 16 accumulator tiles per wave
    __shared__ __attribute__((aligned(1024))) u16 a0[GM * GK];
    __shared__ __attribute__((aligned(1024))) u16 a1[GM * GK];
    __shared__ __attribute__((aligned(1024))) u16 b0[BN * GK];
    __shared__ __attribute__((aligned(1024))) u16 b1[BN * GK];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;
    const int l16 = lane & 15, grp = lane >> 4;

    // tile order: consecutive ids on one XCD, grouped by kGroupM row tiles so
    // that the workgroups running together share row and column panels in L2
    const int tiles_m = (g.M + GM - 1) / GM, tiles_n = g.N / BN;
    const int id = xcd_logical_block(blockIdx.x, gridDim.x);
    const int per_group = kGroupM * tiles_n;
    const int first_m = (id / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (id % per_group) % gsize;
    const int tn = (id % per_group) / gsize;
    const int m0 = tm * GM, n0 = tn * BN;

    f32x4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = g.K / GK;  // K steps
    const int kb = 0;         // first K index
    panel_fill<GM, NW>(a0, g.a, m0, g.M, g.K, kb, wave, lane);
    panel_fill<BN, NW>(b0, g.b, n0, g.N, g.K, kb, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; kt += 2) {
        gemm_step<BM, BN, WM, WN, NW>(acc, a0, b0, a1, b1, kt + 1 < KT, g, m0, n0, kb + (kt + 1) * GK, wm, wn, wave,
                                      lane);
        if (kt + 1 < KT)
            gemm_step<BM, BN, WM, WN, NW>(acc, a1, b1, a0, b0, kt + 2 < KT, g, m0, n0, kb + (kt + 2) * GK, wm, wn,
                                          wave, lane);
    }

    // acc[i][j][r]: output row m0 + wm*WM + i*16 + l16, column n0 + wn*WN + j*16 + 4*grp + r:
    // four consecutive columns of one row per lane. Stage SLICE-row slices
    // through LDS and store rows with 16-byte writes.
    constexpr int LDC = BN + 8;
    constexpr int SLICE = GM < 32 ? GM : 32;
    static_assert(SLICE * LDC <= GM * GK, "slice fits one A stage");
    u16* cs = a0;
#pragma unroll
    for (int sl = 0; sl < GM / SLICE; ++sl) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int r = wm * WM + i * 16 + l16;
            if (r / SLICE == sl) {
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const int c = wn * WN + j * 16 + 4 * grp;
                    *reinterpret_cast<uint2*>(&cs[(r - sl * SLICE) * LDC + c]) = make_uint2(
                        pack2_bf16(acc[i][j][0], acc[i][j][1]), pack2_bf16(acc[i][j][2], acc[i][j][3]));
                }
            }
        }
        __syncthreads();
        constexpr int NT = NW * 64;
#pragma unroll
        for (int i = 0; i < (SLICE * BN / 8 + NT - 1) / NT; ++i) {
            const int c = tid + i * NT;
            const int r = c / (BN / 8), col = (c % (BN / 8)) * 8;
            const int row = m0 + sl * SLICE + r;
            if (c < SLICE * BN / 8 && row < g.M)
                *reinterpret_cast<uint4*>(g.c + static_cast<size_t>(row) * g.N + n0 + col) =
                    *reinterpret_cast<const uint4*>(&cs[r * LDC + col]);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- split-K GEMM for few rows
//
// At most 64 rows (a decode step's tokens) the product streams W_O once and is
// bound by how many bytes are in flight, so this kernel keeps three LDS stages:
// step kt multiplies stage kt % 3 while the loads of step kt + 2 fill stage
// (kt + 2) % 3, and waits only for stage kt + 1 before its barrier.

// One step: multiply (as, bs) into the accumulators while (af, bf) fill from K
// index kfill; then wait until the loads issued before this step's (the next
// stage) have landed and synchronise. The stages are restrict arguments: that is
// what lets the compiler tell the direct loads into one stage from the reads of
// another, so it adds no waits of its own.
template <int WM, int WN, int NW>
__device__ __forceinline__ void split_step(f32x4 (&acc)[WM / 16][WN / 16], const u16* __restrict__ as,
                                           const u16* __restrict__ bs, u16* __restrict__ af, u16* __restrict__ bf,
                                           const GemmArgs& g, int m0, int n0, int kfill, int wm, int wn, int wave,
                                           int lane) {
    constexpr int TI = WM / 16, TJ = WN / 16;
    constexpr int kIssued = (64 + 128) / 8 / NW;  // direct loads per thread and step
    const int l16 = lane & 15, grp = lane >> 4;
    panel_fill<64, NW>(af, g.a, m0, g.M, g.K, kfill, wave, lane);
    panel_fill<128, NW>(bf, g.b, n0, g.N, g.K, kfill, wave, lane);
#pragma unroll
    for (int ks = 0; ks < GK / 32; ++ks) {
        uint4 bq[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) bq[j] = panel_read(bs, wn * WN + j * 16 + l16, ks * 4 + grp);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const uint4 aq = panel_read(as, wm * WM + i * 16 + l16, ks * 4 + grp);
#pragma unroll
            for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16x16x32(bq[j], aq, acc[i][j]);
        }
    }
    __builtin_amdgcn_s_waitcnt((kIssued & 15) | ((kIssued >> 4) << 14) | (7 << 4));  // next stage in, LDS done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 64 x 128 output tile, K range (b / tiles) of g.splits equal ranges for tile
// b % tiles, float32 partial sums into g.part (summed by reduce_splits_kernel).
template <int NWM, int NWN>
__global__ __launch_bounds__(NWM * NWN * 64) void gemm_split_kernel(GemmArgs g) {
    constexpr int BM = 64, BN = 128, NW = NWM * NWN;
    constexpr int WM = BM / NWM, WN = BN / NWN;
    constexpr int TI = WM / 16, TJ = WN / 16;
    constexpr int kIssued = (BM + BN) / 8 / NW;
    static_assert(kIssued * 8 * NW == BM + BN, "panel split");
    __shared__ __attribute__((aligned(1024))) u16 a0[BM * GK];
    __shared__ __attribute__((aligned(1024))) u16 a1[BM * GK];
    __shared__ __attribute__((aligned(1024))) u16 a2[BM * GK];
    __shared__ __attribute__((aligned(1024))) u16 b0[BN * GK];
    __shared__ __attribute__((aligned(1024))) u16 b1[BN * GK];
    __shared__ __attribute__((aligned(1024))) u16 b2[BN * GK];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / NWN, wn = wave % NWN;
    const int l16 = lane & 15, grp = lane >> 4;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = g.N / BN;
    const int split = static_cast<int>(blockIdx.x) / (tiles_m * tiles_n);
    const int id = static_cast<int>(blockIdx.x) % (tiles_m * tiles_n);
    const int m0 = (id % tiles_m) * BM, n0 = (id / tiles_m) * BN;

    f32x4 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = g.K / GK / g.splits;  // K steps of this workgroup
    const int kb = split * KT * GK;      // first K index
    auto kof = [&](int kt) { return kb + min(kt, KT - 1) * GK; };  // past the last step: a re-read
    panel_fill<BM, NW>(a0, g.a, m0, g.M, g.K, kof(0), wave, lane);
    panel_fill<BN, NW>(b0, g.b, n0, g.N, g.K, kof(0), wave, lane);
    panel_fill<BM, NW>(a1, g.a, m0, g.M, g.K, kof(1), wave, lane);
    panel_fill<BN, NW>(b1, g.b, n0, g.N, g.K, kof(1), wave, lane);
    __builtin_amdgcn_s_waitcnt((kIssued & 15) | ((kIssued >> 4) << 14) | (7 << 4));  // stage 0 in
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // whole groups of three steps without exits, then the remaining zero to two
    int kt = 0;
    for (; kt + 3 <= KT; kt += 3) {
        split_step<WM, WN, NW>(acc, a0, b0, a2, b2, g, m0, n0, kof(kt + 2), wm, wn, wave, lane);
        split_step<WM, WN, NW>(acc, a1, b1, a0, b0, g, m0, n0, kof(kt + 3), wm, wn, wave, lane);
        split_step<WM, WN, NW>(acc, a2, b2, a1, b1, g, m0, n0, kof(kt + 4), wm, wn, wave, lane);
    }
    if (kt < KT) split_step<WM, WN, NW>(acc, a0, b0, a2, b2, g, m0, n0, kof(kt + 2), wm, wn, wave, lane);
    if (kt + 1 < KT) split_step<WM, WN, NW>(acc, a1, b1, a0, b0, g, m0, n0, kof(kt + 3), wm, wn, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);  // the last fills (re-reads) end before the workgroup's LDS is released

    float* part = g.part + static_cast<size_t>(split) * g.M * g.N;  // four consecutive columns of a row per lane
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int row = m0 + wm * WM + i * 16 + l16;
        if (row < g.M)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                *reinterpret_cast<f32x4*>(part + static_cast<size_t>(row) * g.N + n0 + wn * WN + j * 16 + 4 * grp) =
                    acc[i][j];
    }
}

// c[m][n] = bf16(sum over splits of part[split][m][n]) in split order, 4 outputs
// per thread; the loads of eight splits go out before their sums.
__global__ __launch_bounds__(256) void reduce_splits_kernel(GemmArgs g) {
    const long long e = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) * 4;
    const long long mn = static_cast<long long>(g.M) * g.N;
    if (e >= mn) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < g.splits; s0 += 8) {
        f32x4 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)  // past the last split: a re-read of it, not added
            t[u] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(g.part + static_cast<size_t>(min(s0 + u, g.splits - 1)) * mn + e));
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < g.splits) acc += t[u];
    }
    *reinterpret_cast<uint2*>(g.c + e) = make_uint2(pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]));
}

}  // namespace

hipError_t launch_groupnorm_gate(const EpilogueArgs& a, hipStream_t st) {
    const long long rows = static_cast<long long>(a.B) * a.H * a.N;
    auto grid = [&](int dv) {
        const int u = dv >= 256 ? dv / 128 : 1;
        const int rpb = kNormThreads / (dv / (8 * u));
        return dim3(static_cast<unsigned>((rows + rpb - 1) / rpb));
    };
    switch (a.dv) {
        case 64: hipLaunchKernelGGL(groupnorm_gate_kernel<64>, grid(64), dim3(kNormThreads), 0, st, a); break;
        case 128: hipLaunchKernelGGL(groupnorm_gate_kernel<128>, grid(128), dim3(kNormThreads), 0, st, a); break;
        case 256: hipLaunchKernelGGL(groupnorm_gate_kernel<256>, grid(256), dim3(kNormThreads), 0, st, a); break;
        case 512: hipLaunchKernelGGL(groupnorm_gate_kernel<512>, grid(512), dim3(kNormThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_bt(const GemmArgs& g, hipStream_t st) {
    if (g.M < 1 || g.N % 128 != 0 || g.K % GK != 0 || g.K < GK) return hipErrorInvalidValue;
    const int splits = gemm_splits(g.M, g.N, g.K);
    if (splits > 1) {  // few rows (a decode step's tokens): split K, then sum the partials
        if (!g.part || g.splits != splits) return hipErrorInvalidValue;
        const unsigned tiles = static_cast<unsigned>((g.M + 63) / 64) * (g.N / 128);
        hipLaunchKernelGGL((gemm_split_kernel<kWavesM, kWavesN>), dim3(tiles * splits), dim3(kWavesM * kWavesN * 64),
                           0, st, g);
        const long long n4 = static_cast<long long>(g.M) * g.N / 4;
        hipLaunchKernelGGL(reduce_splits_kernel, dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256), 0, st, g);
        return hipGetLastError();
    }
    const long long tiles_m = (g.M + 255) / 256;
    if (g.N % 256 == 0)
        hipLaunchKernelGGL((gemm_bt_kernel<256, 256, kWavesM, kWavesN>),
                           dim3(static_cast<unsigned>(tiles_m * (g.N / 256))), dim3(kWavesM * kWavesN * 64), 0, st, g);
    else
        hipLaunchKernelGGL((gemm_bt_kernel<256, 128, kWavesM, kWavesN>),
                           dim3(static_cast<unsigned>(tiles_m * (g.N / 128))), dim3(kWavesM * kWavesN * 64), 0, st, g);
    return hipGetLastError();
}

// K splits for c = a b^T: 1 unless there are at most 64 rows, then enough
// splits (a divisor of K/64, at most 16) that the 64 x 128 tiles times the
// splits give about 256 workgroups, one per compute unit.
int gemm_splits(int M, int N, int K) {
    if (M > 64) return 1;
    const int tiles = N / 128, steps = K / GK;
    int s = 1;
    for (int c = 2; c <= 16; ++c)
        if (steps % c == 0 && static_cast<long long>(tiles) * c <= 256) s = c;
    return s;
}

}  // namespace ret
