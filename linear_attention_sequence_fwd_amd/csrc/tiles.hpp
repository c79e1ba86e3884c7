// LDS layouts and HBM->register block loads shared by the bf16 MFMA kernels.
#pragma once

#include "common.hpp"

namespace ret {

// ---------------------------------------------------------------- LDS index maps

// K row-major [C][DK]: unit (d/8) of row j is XOR-ed with (j + j/8) mod 8, so
// that both the block writes (8 rows of one block column) and the G1 reads
// (16 consecutive rows) spread over banks.
template <int DK>
__device__ __forceinline__ int kidx_rm(int j, int d) {
    return j * DK + ((((d >> 3) ^ ((j + (j >> 3)) & 7))) << 3) + (d & 7);
}
// Transposed [rows][C] (K^T and V^T): unit (token/8) XOR-ed with row mod 8.
template <int C>
__device__ __forceinline__ int tidx(int row, int j) {
    return row * C + ((((j >> 3) ^ (row & 7))) << 3) + (j & 7);
}
// S^T [DVT][DK]: unit (d/8) XOR-ed with column mod 8.
template <int DK>
__device__ __forceinline__ int sidx(int c, int d) {
    return c * DK + ((((d >> 3) ^ (c & 7))) << 3) + (d & 7);
}

// Element e (0..7) of 8 packed bf16, as raw 16 bits.
__device__ __forceinline__ uint32_t elem16(const uint4& x, int e) {
    const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// 8x8 block index -> (token block, column block). Eight consecutive indices
// walk down the token blocks of one column block, so a wave's 64 lanes cover
// 8 token blocks x 8 column blocks: every row it touches is read as 128
// contiguous bytes, and the transposed LDS writes of the 8 lanes that share a
// column block land in different banks.
template <int D>
__device__ __forceinline__ void block_coords(int idx, int& tb, int& cb) {
    const int rest = idx >> 3;
    cb = rest % (D / 8);
    tb = (idx & 7) + 8 * (rest / (D / 8));
}

template <int D, int NBLK, int PT, int NTHR>
__device__ __forceinline__ void load_blocks(uint4 (&r)[PT][8], const u16* base, int ld, int valid,
                                            int tid) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
        const int idx = tid + u * NTHR;
        int tb, cb;
        block_coords<D>(idx < NBLK ? idx : 0, tb, cb);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int row = tb * 8 + q;
            if (idx < NBLK && row < valid)
                r[u][q] = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(row) * ld + cb * 8);
            else
                r[u][q] = make_uint4(0, 0, 0, 0);
        }
    }
}

}  // namespace ret
