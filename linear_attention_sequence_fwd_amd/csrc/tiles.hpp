// LDS layouts and HBM->register block loads shared by the bf16 MFMA kernels.
#pragma once

#include "common.hpp"

namespace ret {

// ---------------------------------------------------------------- LDS layouts
//
// Every LDS tile is a row-major [rows][U*8] bf16 array whose 16-byte units
// are XOR-swizzled per row: unit u of row r is stored at u ^ (r mod W),
// W = min(U, 16). Sixteen consecutive rows therefore spread one column of
// units over 16 different bank groups, so MFMA fragment reads (16 rows, one
// unit each) and the transposing block writes are free of bank conflicts.
//
// Because the swizzle depends only on r mod 16, a fragment read at row
// r0 + 16a + l16 and unit 4b + w (a, b unrolled loop indices; l16, w per lane)
// lands at  base[b mod 4] + 16a*U*8 + (b/4)*32*... : four per-lane base
// addresses plus compile-time offsets. Fragment reads then need no address
// arithmetic inside the unrolled loops, which keeps register pressure down.

template <int U>
__device__ __forceinline__ int swz(int row, int unit) {
    constexpr int W = U < 16 ? U : 16;
    return row * (U * 8) + ((unit ^ (row & (W - 1))) << 3);
}

// Per-lane bases for fragment reads of 16-byte unit 4b + w (w in 0..3) at rows
// row_lane + 16a.  at(a, b) returns the element offset for compile-time a, b.
template <int U>
struct FragAddr {
    int base[4];
    __device__ __forceinline__ FragAddr(int row_lane, int w) {
        constexpr int W = U < 16 ? U : 16;
        const int x = row_lane & (W - 1);
        const int y = x >> 2;
        const int z = w ^ (x & 3);
#pragma unroll
        for (int b0 = 0; b0 < 4; ++b0) base[b0] = row_lane * (U * 8) + z * 8 + 32 * (b0 ^ y);
    }
    __device__ __forceinline__ int at(int a, int b) const { return base[b & 3] + a * 16 * (U * 8) + (b >> 2) * 128; }
};

// Element e of bf16 values packed two per dword, as raw 16 bits.
template <int NW32>
__device__ __forceinline__ uint32_t elem16(const uint32_t (&x)[NW32], int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Staging blocks: 8 tokens x BW columns (BW = 8 or 4), each row held as BW/2
// dwords; the 8 tokens of block tb are staged_token(tb, 0..7). Block index ->
// (token block, column block): eight consecutive indices walk down the token
// blocks of one column block, so a wave's 64 lanes read 8 token blocks x 8
// column blocks (each row it touches as BW*2 contiguous bytes per lane), and
// the transposed LDS writes of the 8 lanes that share a column block land in
// different units of the same row.
// TB is the number of token blocks (tokens / 8) of the tile: consecutive
// indices walk min(8, TB) of them (a 32-token chunk has only four).
template <int D, int BW, int TB = 8>
__device__ __forceinline__ void block_coords(int idx, int& tb, int& cb) {
    constexpr int S = TB < 8 ? TB : 8;
    const int rest = idx / S;
    cb = rest % (D / BW);
    tb = (idx % S) + S * (rest / (D / BW));
}

// Token order inside staged 32-token groups. Staging block tb covers tokens
// 32*(tb/4) + 4*(tb%4) + {0,1,2,3, 16,17,18,19}, in that order, so one 16-byte
// unit of a transposed (token-contiguous) LDS row holds exactly the 8 tokens
// that one MFMA lane group contracts over when the other operand is a pair of
// 16x16 accumulator tiles (rows 4g..4g+3 of tile 2t and of tile 2t+1).
__device__ __forceinline__ int staged_token(int tb, int q) {
    return 32 * (tb >> 2) + 4 * (tb & 3) + (q < 4 ? q : 12 + q);
}

template <int BW>
struct BlockRows {
    uint32_t w[8][BW / 2];
};

// Every load is issued unconditionally (rows past `valid` read a clamped,
// in-bounds row and are zeroed by a select): with no branch around a load the
// compiler can count outstanding loads exactly, and a wait for one batch does
// not also wait for a prefetch issued after it. valid == 0 reads row 0.
// Q0..Q1-1: the rows of each block to load (all eight by default), so a caller
// can spread one chunk's loads over several points of its loop.
// With rev, row i of the chunk is memory row (valid - 1 - i) from base (a
// chunk read in reverse token order; base then points at its last token).
template <int D, int BW, int NBLK, int PT, int NTHR, int Q0 = 0, int Q1 = 8>
__device__ __forceinline__ void load_blocks(BlockRows<BW> (&r)[PT], const u16* base, int ld, int valid, int tid,
                                            bool rev = false) {
    // Row pointers are wave-uniform (base + row * ld); the per-lane part is a
    // 32-bit byte offset, so each row load needs one shared offset register
    // and a scalar base instead of its own 64-bit address.
    const int last = valid > 0 ? valid - 1 : 0;
#pragma unroll
    for (int u = 0; u < PT; ++u) {
        const int idx = tid + u * NTHR;
        const bool in_blk = NBLK % NTHR == 0 || idx < NBLK;
        int tb, cb;
        block_coords<D, BW, NBLK / (D / BW)>(in_blk ? idx : 0, tb, cb);
        const int tok0 = staged_token(tb, 0);
#pragma unroll
        for (int q = Q0; q < Q1; ++q) {
            const int dq = staged_token(0, q);  // token offset of row q inside the block
            const bool ok = in_blk && tok0 + dq < valid;
            const int row = rev ? last - min(tok0 + dq, last) : min(tok0 + dq, last);
            const char* rowq = reinterpret_cast<const char*>(base) + static_cast<uint32_t>((row * ld + cb * BW) * 2);
            if constexpr (BW == 8) {
                const uint4 x = *reinterpret_cast<const uint4*>(rowq);
                r[u].w[q][0] = ok ? x.x : 0u;
                r[u].w[q][1] = ok ? x.y : 0u;
                r[u].w[q][2] = ok ? x.z : 0u;
                r[u].w[q][3] = ok ? x.w : 0u;
            } else {
                const uint2 x = *reinterpret_cast<const uint2*>(rowq);
                r[u].w[q][0] = ok ? x.x : 0u;
                r[u].w[q][1] = ok ? x.y : 0u;
            }
        }
    }
}

// Column c of a staged block: 8 consecutive tokens, packed as one uint4.
template <int BW>
__device__ __forceinline__ uint4 block_column(const BlockRows<BW>& b, int c) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) w[p] = elem16(b.w[2 * p], c) | (elem16(b.w[2 * p + 1], c) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Rotate the complex pairs of one staged row in place (BW/2 pairs with
// frequencies th[0..BW/2-1]) at absolute position `position`.
template <int BW>
__device__ __forceinline__ void rotate_row(uint32_t (&w)[BW / 2], const float* th, double position) {
#pragma unroll
    for (int p = 0; p < BW / 2; ++p) {
        float c, s;
        rot_cs_fast(position, th[p], c, s);
        const float re = lo_bf16(w[p]), im = hi_bf16(w[p]);
        w[p] = pack2_bf16(re * c - im * s, re * s + im * c);
    }
}

// The same with the frequencies of pairs j0.. read from the head parameters.
template <int BW>
__device__ __forceinline__ void rotate_row(uint32_t (&w)[BW / 2], const HeadParams& hp, int j0, double position) {
    rotate_row<BW>(w, hp.theta + j0, position);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, lane r supplies the address of 4 consecutive 16-bit elements M[r];
// lane j receives (M[4k + j/4][j%4], k = 0..3). With lane r pointing at row
// t0 + r/4, columns c0 + 4(r%4) .. +3 of a row-major matrix X, lane j gets
// X[t0 + k][c0 + j] for k = 0..3: four consecutive rows of one column, the
// layout of an MFMA operand whose contraction runs down the rows.
__device__ __forceinline__ uint2 lds_read_tr16x4(const u16* p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(p));
    return __builtin_bit_cast(uint2, r);
}

// Staging block width: 8x8 blocks when there are at least as many as
// threads, else 8x4 blocks (half the registers per thread).
constexpr int stage_width(int rows, int cols, int nthr) { return (rows / 8) * (cols / 8) >= nthr ? 8 : 4; }

}  // namespace ret
