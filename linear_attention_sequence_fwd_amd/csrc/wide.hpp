// Device helpers of the single-wave-per-SIMD matrix-core kernels (chunk_wide.hip,
// parallel_wide.hip) on gfx950: buffer resources (loads past a given byte
// count read zero, stores past it are dropped), explicit wait counts, and a
// compile-time software pipeline for LDS fragment reads feeding MFMAs.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace ret {
namespace wide {

constexpr int kBufFlags = 0x00020000;  // buffer resource word 3 for gfx9-family raw buffers

template <int V>
using Ic = std::integral_constant<int, V>;

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufFlags);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ void buf_store8(uint2 v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r,
                                          off, 0, 0);
}

// Eight bf16 (one 16-byte unit) times f, rounded back to bf16.
__device__ __forceinline__ uint4 scale8_bf16(uint4 x, float f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack2_bf16(lo_bf16(w[p]) * f, hi_bf16(w[p]) * f);
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// s_waitcnt with at most VM vector memory operations and no LDS operation
// outstanding (gfx9 fields: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at
// its maximum, lgkmcnt 11:8).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// s_waitcnt lgkmcnt(0), vector memory operations left outstanding.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// 16 bytes through device-coherent buffer accesses (cache policy sc1: past the
// XCD's L2 to the device's point of coherence), for what one workgroup publishes
// for another of the same launch. Whole 16-byte units at consecutive lane
// addresses keep every access a full segment.
constexpr int kCoherent = 16;  // sc1
__device__ __forceinline__ void store_coherent16(const f32x4& v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r,
                                           off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 load_coherent16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(Ic<B>{});
        static_for<B + 1, E>(f);
    }
}

// A software pipeline over NS steps of LDS reads feeding matrix instructions:
// the fragments of step j are read during step j - D, and a scheduling
// barrier closes every step, so each read is issued D steps ahead of its use
// whatever the register pressure (with one wave per SIMD nothing else hides
// the LDS latency). read(Ic<j>) returns step j's fragments, use(Ic<j>, frags)
// issues its matrix instructions, side(Ic<j>) any other work placed in step j
// (global loads and stores spread over the matrix work, so that they never
// queue up behind one another and stall the wave).
template <int NS, int D, typename Read, typename Use, typename Side>
__device__ __forceinline__ void pipelined(Read&& read, Use&& use, Side&& side) {
    using Frag = decltype(read(Ic<0>{}));
    Frag fr[D];
    static_for<0, (D < NS ? D : NS)>([&](auto i) { fr[decltype(i)::value] = read(i); });
    static_for<0, NS>([&](auto i) {
        constexpr int j = decltype(i)::value;
        const Frag cur = fr[j % D];
        if constexpr (j + D < NS) fr[j % D] = read(Ic<j + D>{});
        side(i);
        use(i, cur);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Calls f(Ic<i>) for the items i of M that fall on step J of NS when the M
// items are spread evenly over the steps.
template <int M, int NS, int J, typename F>
__device__ __forceinline__ void spread(F&& f) {
    static_for<0, M>([&](auto i) {
        if constexpr (decltype(i)::value * NS / M == J) f(i);
    });
}


}  // namespace wide
}  // namespace ret
